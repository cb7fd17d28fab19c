/*
 * gdn_oracle.c -- TEST INFRASTRUCTURE ONLY.  The plain, slow, fp64 CPU oracle of the gated
 * delta rule.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * it; the product library never does.  It shares no code, header, table or helper with the
 * HIP path.
 *
 * What it computes, token by token, for each (sequence n, head h) independently:
 *
 *   Gated DeltaNet update (page "Gated DeltaNet与推理脚手架：两个模糊边界的发现", section
 *   发现一, third bullet; page "Gated DeltaNet 架构详解与 Qwen 3.5 的联系", section 6):
 *       S_t = S_{t-1} * alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   alpha_t = exp(g_t)
 *   written out as
 *       S_t = alpha_t S_{t-1} - beta_t alpha_t (S_{t-1} k_t) k_t^T + beta_t v_t k_t^T
 *   and the read-out o_t = scale * S_t q_t.
 *
 *   Optional prologue (page maplevalley.com.cn/news/1910399, section 3.1, 卷积预处理): a
 *   causal depthwise conv1d with 4 taps per channel, followed by SiLU(x) = x / (1 + exp(-x)).
 *   The three raw inputs before a sequence start come from a given conv history (zeros when
 *   none is given), and the conv history after the sequence (its last three raw inputs) can be
 *   returned, so that a sequence can be continued by a later call or by decode steps.
 *   Optional L2 normalisation of q and k over the key dimension, x / sqrt(sum x^2 + 1e-6) (not
 *   on the pages; the eps is this library's reading).
 *
 *   Heads: the model configuration on page "Gated DeltaNet 架构详解与 Qwen 3.5 的联系", section 6,
 *   counts query/key heads and value heads separately.  Value head h uses query/key head
 *   h / (H / Hk): consecutive value heads share one query/key head (this library's reading).
 *
 * Everything is double precision.  Callers pass the exact values the GPU receives, promoted to
 * double.  Parallelism: POSIX threads over independent (n, h) pairs only; the arithmetic of
 * one pair is a single serial loop.
 *
 * Pins (tests/test_oracle_*.py): pure decay for beta = 0, identity for alpha = 1 and beta = 0,
 * exact retrieval S_t k_t = v_t for beta = 1 and unit k, one SGD step on 1/2 ||S k - v||^2,
 * the DeltaNet special case g = 0, a one-hot closed form with dyadic gates, brute-force
 * transition products on tiny inputs, the causal conv against numpy.convolve, varlen packing
 * and split/resume identities.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *s0, *conv_w, *hist;
    double* hist_out;
    const int64_t* cu;
    const unsigned char* mask;
    double *o, *sfin;
    int N, H, Hk, dk, dv, l2norm; /* H value heads, Hk query/key heads (H a multiple of Hk) */
    double scale;
    int next_pair; /* work counter, protected by lock */
    pthread_mutex_t lock;
} job_t;

static double silu(double x) { return x / (1.0 + exp(-x)); }

/* Raw input s of one channel of one sequence, s in [-3, len): tokens of the sequence, or for
 * s < 0 the history value 3 + s (hist holds the three inputs before the sequence start, oldest
 * first, at a stride of hstride doubles; NULL = zeros). */
static double conv_input(const double* x, long stride, const double* hist, long hstride, long s) {
    if (s >= 0) return x[s * stride];
    return hist ? hist[(3 + s) * hstride] : 0.0;
}

/* Causal depthwise conv (4 taps) then SiLU, for one channel of one sequence:
 * x_t' = SiLU(sum_j w[j] * x_{t-3+j}). */
static void conv_silu(const double* x, long stride, const double* hist, long hstride, long len, const double* w,
                      double* out) {
    for (long t = 0; t < len; ++t) {
        double acc = 0.0;
        for (int j = 0; j < 4; ++j) acc += w[j] * conv_input(x, stride, hist, hstride, t - 3 + j);
        out[t] = silu(acc);
    }
}

static void run_pair(job_t* J, int n, int h) {
    const int H = J->H, Hk = J->Hk, dk = J->dk, dv = J->dv;
    const int hk = h / (H / Hk); /* the query/key head shared by this group of value heads */
    const long bos = (long)J->cu[n], len = (long)(J->cu[n + 1] - J->cu[n]);
    double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);
    double* Sk = (double*)malloc(sizeof(double) * dv);
    double* qt = (double*)malloc(sizeof(double) * dk);
    double* kt = (double*)malloc(sizeof(double) * dk);
    double* vt = (double*)malloc(sizeof(double) * dv);
    double *cq = NULL, *ck = NULL, *cv = NULL;

    if (J->s0)
        memcpy(S, J->s0 + ((size_t)n * H + h) * dv * dk, sizeof(double) * (size_t)dv * dk);
    else
        memset(S, 0, sizeof(double) * (size_t)dv * dk);

    if (J->conv_w) {
        /* Channel c of the conv: q channels hk*dk + i, then k (Hk*dk + hk*dk + i), then v
         * (2*Hk*dk + h*dv + i); the history rows of sequence n are [3][C] at n*3*C. */
        const long C = 2L * Hk * dk + (long)H * dv;
        const double* hist = J->hist ? J->hist + (size_t)n * 3 * C : NULL;
        double* hout = J->hist_out ? J->hist_out + (size_t)n * 3 * C : NULL;
        /* Pre-compute the conv+SiLU channels of this (sequence, head), token-major. */
        cq = (double*)malloc(sizeof(double) * (size_t)(len + 1) * dk);
        ck = (double*)malloc(sizeof(double) * (size_t)(len + 1) * dk);
        cv = (double*)malloc(sizeof(double) * (size_t)(len + 1) * dv);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)(len + 1));
        for (int part = 0; part < 3; ++part) {
            const int d = part < 2 ? dk : dv;
            const int heads = part < 2 ? Hk : H, hh = part < 2 ? hk : h;
            const double* x = part == 0 ? J->q : (part == 1 ? J->k : J->v);
            double* dst = part == 0 ? cq : (part == 1 ? ck : cv);
            for (int i = 0; i < d; ++i) {
                const long c = part < 2 ? (long)part * Hk * dk + (long)hk * dk + i : 2L * Hk * dk + (long)h * dv + i;
                const double* xc = x + ((size_t)bos * heads + hh) * d + i;
                const double* hc = hist ? hist + c : NULL;
                conv_silu(xc, (long)heads * d, hc, C, len, J->conv_w + 4 * c, tmp);
                for (long t = 0; t < len; ++t) dst[t * d + i] = tmp[t];
                /* the last three raw inputs, oldest first; a q/k channel shared by several value
                 * heads is written by the first of them */
                if (hout && (part == 2 || h % (H / Hk) == 0))
                    for (int j = 0; j < 3; ++j) hout[j * C + c] = conv_input(xc, (long)heads * d, hc, C, len - 3 + j);
            }
        }
        free(tmp);
    }

    for (long t = 0; t < len; ++t) {
        const long row = (bos + t) * H + h, krow = (bos + t) * Hk + hk;
        for (int i = 0; i < dk; ++i) {
            qt[i] = cq ? cq[t * dk + i] : J->q[krow * dk + i];
            kt[i] = ck ? ck[t * dk + i] : J->k[krow * dk + i];
        }
        for (int i = 0; i < dv; ++i) vt[i] = cv ? cv[t * dv + i] : J->v[row * dv + i];
        if (J->l2norm) {
            double sq = 0.0, sk = 0.0;
            for (int i = 0; i < dk; ++i) {
                sq += qt[i] * qt[i];
                sk += kt[i] * kt[i];
            }
            const double rq = 1.0 / sqrt(sq + 1e-6), rk = 1.0 / sqrt(sk + 1e-6);
            for (int i = 0; i < dk; ++i) {
                qt[i] *= rq;
                kt[i] *= rk;
            }
        }
        const double alpha = exp(J->g[row]);
        const double b = J->beta[row];
        /* Sk = S_{t-1} k_t */
        for (int a = 0; a < dv; ++a) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(size_t)a * dk + i] * kt[i];
            Sk[a] = acc;
        }
        /* S_t = alpha S - beta alpha (S k) k^T + beta v k^T, then o_t = scale S_t q_t */
        for (int a = 0; a < dv; ++a) {
            const double ua = b * (vt[a] - alpha * Sk[a]);
            double* Sa = S + (size_t)a * dk;
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) {
                Sa[i] = alpha * Sa[i] + ua * kt[i];
                acc += Sa[i] * qt[i];
            }
            if (J->o) J->o[row * dv + a] = J->scale * acc;
        }
    }
    if (J->sfin)
        memcpy(J->sfin + ((size_t)n * H + h) * dv * dk, S, sizeof(double) * (size_t)dv * dk);
    free(S);
    free(Sk);
    free(qt);
    free(kt);
    free(vt);
    free(cq);
    free(ck);
    free(cv);
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    const int pairs = J->N * J->H;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int p = J->next_pair++;
        pthread_mutex_unlock(&J->lock);
        if (p >= pairs) break;
        if (J->mask && !J->mask[p]) continue;
        run_pair(J, p / J->H, p % J->H);
    }
    return NULL;
}

/*
 * gdn_oracle_forward -- o and final state of the gated delta rule over packed sequences.
 *  H value heads (state, gates, v, o) and Hk query/key heads, H a multiple of Hk: value head h
 *  reads query/key head h / (H / Hk), so each query/key head serves H / Hk consecutive value
 *  heads (Hk = H: one each).
 *  q, k [T_tot,Hk,dk]; v [T_tot,H,dv]; g, beta [T_tot,H]; s0 [N,H,dv,dk] or NULL (zeros);
 *  cu [N+1] int64 offsets; conv_w [C,4] or NULL with C = 2*Hk*dk + H*dv conv channels (q, k, v);
 *  conv_hist [N,3,C] or NULL (zeros): the raw inputs before each sequence start; conv_hist_out
 *  [N,3,C] or NULL: the last three raw inputs of each sequence (may not alias conv_hist);
 *  o [T_tot,H,dv] or NULL;
 *  sfin [N,H,dv,dk] or NULL; mask [N*H] or NULL: only pairs with mask != 0 are computed (their
 *  o rows, final states and conv history channels are written; others are left untouched).
 *  nthreads <= 0: all cores.  Returns the number of threads used.
 */
int gdn_oracle_forward(const double* q, const double* k, const double* v, const double* g,
                       const double* beta, const double* s0, const int64_t* cu,
                       const double* conv_w, const double* conv_hist, double* conv_hist_out, double* o,
                       double* sfin, const unsigned char* mask, int N, int H, int Hk, int dk, int dv,
                       double scale, int l2norm, int nthreads) {
    job_t J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.s0 = s0; J.conv_w = conv_w;
    J.hist = conv_hist; J.hist_out = conv_hist_out;
    J.cu = cu; J.mask = mask; J.o = o; J.sfin = sfin;
    if (Hk < 1 || H % Hk != 0) return -1;
    J.N = N; J.H = H; J.Hk = Hk; J.dk = dk; J.dv = dv; J.l2norm = l2norm; J.scale = scale;
    J.next_pair = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > N * H) nthreads = N * H > 0 ? N * H : 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
    worker(&J);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return nthreads;
}

/*
 * gdn_oracle_step -- one decode token per sequence (the same update with T = 1), state
 * updated in place.  q, k [N,Hk,dk]; v [N,H,dv]; g, beta [N,H]; state [N,H,dv,dk]; o [N,H,dv];
 * conv_w [C,4] or NULL (C = 2*Hk*dk + H*dv); conv_hist [N,3,C] (with conv_w): the three
 * previous raw inputs, read and replaced by the three latest.  Heads as for gdn_oracle_forward.
 * Page pzsr.cn/news/750, section a、增量更新: decay the whole state first, then erase and write
 * along the current key.
 */
int gdn_oracle_step(const double* q, const double* k, const double* v, const double* g,
                    const double* beta, const double* conv_w, double* conv_hist, double* state, double* o,
                    int N, int H, int Hk, int dk, int dv, double scale, int l2norm, int nthreads) {
    int64_t* cu = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N + 1));
    for (int n = 0; n <= N; ++n) cu[n] = n;
    double* hout = NULL;
    const size_t hn = (size_t)N * 3 * (2 * (size_t)Hk * dk + (size_t)H * dv);
    if (conv_w) hout = (double*)malloc(sizeof(double) * hn);
    int used = gdn_oracle_forward(q, k, v, g, beta, state, cu, conv_w, conv_hist, hout, o, state, NULL, N, H,
                                  Hk, dk, dv, scale, l2norm, nthreads);
    if (conv_w) {
        memcpy(conv_hist, hout, sizeof(double) * hn);
        free(hout);
    }
    free(cu);
    return used;
}

/* gdn_oracle_gates -- the gate parameterisation of page maplevalley.com.cn/news/1910399,
 * section 2.1: g = -exp(A_log[h]) * softplus(a + dt_bias[h]), beta = sigmoid(b), with
 * softplus(x) = log(1 + exp(x)) evaluated as max(x, 0) + log1p(exp(-|x|)).
 * a, b [T,H]; A_log, dt_bias [H]; g, beta [T,H]. */
void gdn_oracle_gates(const double* a, const double* b, const double* A_log,
                      const double* dt_bias, double* g, double* beta, long T, int H) {
    for (long t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            const double x = a[t * H + h] + dt_bias[h];
            const double sp = (x > 0 ? x : 0.0) + log1p(exp(-fabs(x)));
            g[t * H + h] = -exp(A_log[h]) * sp;
            beta[t * H + h] = 1.0 / (1.0 + exp(-b[t * H + h]));
        }
}

/* gdn_oracle_gated_norm -- the output epilogue: a zero-centred RMSNorm of each (token, head) row of
 * o over dv (page maplevalley.com.cn/news/1910399, section 3.2 Zero-Centered RMSNorm: normalise by
 * rsqrt(mean(x^2) + eps), with a learnable scale stored as an offset from 1 and initialised to
 * zero), then a sigmoid output gate (page "GDN融合门控注意力的动态资源分配机制，AI智能体调动实战演练",
 * section 2, the paragraph on the dynamics of Gated DeltaNet: a learned gate, usually a sigmoid,
 * scales the output after the attention computation and before the residual connection):
 *     out[r, i] = o[r, i] / sqrt(mean_i o[r, i]^2 + eps) * (1 + w[i]) * sigmoid(z[r, i]).
 * o, z, out [rows, dv] (out may equal o); w [dv]. */
void gdn_oracle_gated_norm(const double* o, const double* z, const double* w, double* out, long rows, int dv,
                           double eps) {
    for (long r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int i = 0; i < dv; ++i) ss += o[r * dv + i] * o[r * dv + i];
        const double inv = 1.0 / sqrt(ss / dv + eps);
        for (int i = 0; i < dv; ++i)
            out[r * dv + i] = o[r * dv + i] * inv * (1.0 + w[i]) / (1.0 + exp(-z[r * dv + i]));
    }
}
