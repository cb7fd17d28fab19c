// chunk_f32.hip -- chunked prefill of the gated delta rule in exact fp32 arithmetic (VALU).
//
// The sequence is cut into chunks of C = 64 tokens; inside a chunk every product is computed in
// parallel and only the state crosses from chunk to chunk (page pzsr.cn/news/750, section
// 1、为什么要设计为chunk的模式).  The chunk algebra (derived from the per-token rule
// u_t = beta_t (v_t - alpha_t S_{t-1} k_t), S_t = alpha_t S_{t-1} + u_t k_t^T):
//   gamma_i = inclusive prefix sum of g in the chunk, Gamma_i = exp(gamma_i),
//   M_ij = exp(gamma_i - gamma_j) for j <= i (never exp of a positive number),
//   L = strict_lower(diag(beta) (M o K K^T)), T = (I + L)^-1  (forward substitution),
//   X = diag(beta) V - diag(beta Gamma) K S^T,  U = T X      (the stacked u_t),
//   O = diag(Gamma) Q S^T + lower(M o Q K^T) U,
//   S <- Gamma_C S + U^T diag(exp(gamma_C - gamma)) K.
// Rows of S (the value index) are independent, so a workgroup owns one (sequence, head,
// block of BV state rows) and walks the sequence's chunks in order.  Tail chunks are padded
// with zero keys, zero beta and zero g, which contribute nothing.
//
// This is the fp32 dtype path: every product is an fp32 FMA, decay factors use the accurate
// expf.  The bf16 path (chunk_bf16.hip) runs the same algebra on MFMA.
#include "common.hpp"
#include "kernels.hpp"
#include "prologue.hpp"

namespace gdn {

namespace {

constexpr int C = 64;

template <typename T>
struct F32Params {
    const T *q, *k, *v;
    const float *g, *beta, *gate_params, *s0, *conv_w;
    const T* conv_state;  // [N,3,2Hk*dk+H*dv] history before each sequence, or null (zeros)
    const int32_t* cu;
    T* o;
    float* sfin;
    int N, T_tot, H, Hk, dv;  // H value heads, Hk query/key heads
    float scale;
    int l2norm;
};

template <int DK, int BV>
struct F32Smem {
    static constexpr int QS = DK + 1;  // padded row strides
    static constexpr int VS = BV + 1;
    static constexpr int CS = C + 1;
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + C * QS;
    static constexpr int oV = oK + C * QS;
    static constexpr int oS = oV + C * VS;
    static constexpr int oL = oS + BV * QS;
    static constexpr int oT = oL + C * CS;
    static constexpr int oP = oT + C * CS;
    static constexpr int oX = oP + C * CS;
    static constexpr int oU = oX + C * VS;
    static constexpr int oG = oU + C * VS;   // gamma
    static constexpr int oB = oG + C;        // beta
    static constexpr int oD = oB + C;        // exp(gamma_last - gamma_i)
    static constexpr int total = oD + C;
    static constexpr size_t bytes = sizeof(float) * total;
};

template <int DK, int BV, typename T>
__global__ __launch_bounds__(256) void chunk_f32_kernel(F32Params<T> p) {
    using L = F32Smem<DK, BV>;
    extern __shared__ float sm[];
    float* sQ = sm + L::oQ;
    float* sK = sm + L::oK;
    float* sV = sm + L::oV;
    float* sS = sm + L::oS;
    float* sL = sm + L::oL;
    float* sT = sm + L::oT;
    float* sP = sm + L::oP;
    float* sX = sm + L::oX;
    float* sU = sm + L::oU;
    float* sG = sm + L::oG;
    float* sB = sm + L::oB;
    float* sD = sm + L::oD;

    const int tid = threadIdx.x;
    const int nv = p.dv / BV;
    const int vb = blockIdx.x % nv;
    const int h = (blockIdx.x / nv) % p.H;
    const int n = blockIdx.x / (nv * p.H);
    long bos, eos;
    if (p.cu) {
        bos = p.cu[n];
        eos = p.cu[n + 1];
    } else {
        const long len = p.T_tot / p.N;
        bos = (long)n * len;
        eos = bos + len;
    }
    const int H = p.H, Hk = p.Hk, dv = p.dv;
    const int hk = h / (H / Hk);                         // query/key head of this value head
    const size_t hstride = (size_t)2 * Hk * DK + (size_t)H * dv;  // conv channels per token
    const T* hist = p.conv_state ? p.conv_state + (size_t)n * 3 * hstride : nullptr;
    const size_t sbase = ((size_t)n * H + h) * dv * DK + (size_t)vb * BV * DK;

    for (int idx = tid; idx < BV * DK; idx += 256) {
        const int r = idx / DK, c = idx % DK;
        sS[r * L::QS + c] = p.s0 ? p.s0[sbase + (size_t)r * DK + c] : 0.f;
    }

    for (long cs = bos; cs < eos; cs += C) {
        const int len = (int)min((long)C, eos - cs);
        __syncthreads();  // previous chunk finished with every buffer
        // ---- load the chunk (optional conv + SiLU), zero-padded past the tail ----
        for (int idx = tid; idx < C * DK; idx += 256) {
            const int r = idx / DK, c = idx % DK;
            float qv = 0.f, kv = 0.f;
            if (r < len) {
                const long t = cs + r;
                if (p.conv_w) {
                    const size_t cq = (size_t)hk * DK + c, ck = (size_t)Hk * DK + cq;
                    qv = conv_silu_at(p.q, p.conv_w + 4 * cq, t, bos, (size_t)Hk * DK, cq, hist ? hist + cq : nullptr, hstride);
                    kv = conv_silu_at(p.k, p.conv_w + 4 * ck, t, bos, (size_t)Hk * DK, cq, hist ? hist + ck : nullptr, hstride);
                } else {
                    qv = load1(p.q + ((size_t)t * Hk + hk) * DK + c);
                    kv = load1(p.k + ((size_t)t * Hk + hk) * DK + c);
                }
            }
            sQ[r * L::QS + c] = qv;
            sK[r * L::QS + c] = kv;
        }
        for (int idx = tid; idx < C * BV; idx += 256) {
            const int r = idx / BV, c = idx % BV;
            float vv = 0.f;
            if (r < len) {
                const long t = cs + r;
                const int ch = vb * BV + c;
                const size_t cv = (size_t)2 * Hk * DK + (size_t)h * dv + ch;
                vv = p.conv_w ? conv_silu_at(p.v, p.conv_w + 4 * cv, t, bos, (size_t)H * dv, (size_t)h * dv + ch,
                                             hist ? hist + cv : nullptr, hstride)
                              : load1(p.v + ((size_t)t * H + h) * dv + ch);
            }
            sV[r * L::VS + c] = vv;
        }
        if (tid < C) {
            const bool in = tid < len;
            float gv = in ? p.g[(size_t)(cs + tid) * H + h] : 0.f;
            float bv = in ? p.beta[(size_t)(cs + tid) * H + h] : 0.f;
            if (p.gate_params && in) {
                gv = raw_decay(gv, -expf(p.gate_params[h]), p.gate_params[H + h]);
                bv = raw_beta(bv);
            }
            sG[tid] = gv;
            sB[tid] = bv;
        }
        __syncthreads();
        // ---- L2 norm of q and k rows (4 lanes per row) and the gate prefix sum ----
        if (p.l2norm) {
            const int r = tid / 4, part = tid % 4;
            float sq = 0.f, sk = 0.f;
            for (int c = part; c < DK; c += 4) {
                sq += sQ[r * L::QS + c] * sQ[r * L::QS + c];
                sk += sK[r * L::QS + c] * sK[r * L::QS + c];
            }
            sq = group_sum<4>(sq);
            sk = group_sum<4>(sk);
            const float rq = rsqrtf(sq + kL2Eps), rk = rsqrtf(sk + kL2Eps);
            for (int c = part; c < DK; c += 4) {
                sQ[r * L::QS + c] *= rq;
                sK[r * L::QS + c] *= rk;
            }
        }
        if (tid == 0) {
            float acc = 0.f;
            for (int i = 0; i < C; ++i) {
                acc += sG[i];
                sG[i] = acc;
            }
        }
        __syncthreads();
        const float gl = sG[C - 1];
        if (tid < C) sD[tid] = expf(gl - sG[tid]);
        // ---- masked Gram matrices: L (strict lower) and Pm (lower incl. diagonal) ----
        for (int idx = tid; idx < C * C; idx += 256) {
            const int i = idx / C, j = idx % C;
            float kk = 0.f, qk = 0.f;
            if (j <= i) {
#pragma unroll 8
                for (int d = 0; d < DK; ++d) {
                    kk += sK[i * L::QS + d] * sK[j * L::QS + d];
                    qk += sQ[i * L::QS + d] * sK[j * L::QS + d];
                }
                const float m = expf(sG[i] - sG[j]);
                kk *= sB[i] * m;
                qk *= m;
            }
            sL[i * L::CS + j] = j < i ? kk : 0.f;
            sP[i * L::CS + j] = qk;
        }
        __syncthreads();
        // ---- T = (I + L)^-1 by forward substitution, one column per lane ----
        if (tid < C) {
            const int j = tid;
            for (int i = 0; i < C; ++i) {
                float t;
                if (i < j) {
                    t = 0.f;
                } else if (i == j) {
                    t = 1.f;
                } else {
                    float acc = sL[i * L::CS + j];
                    for (int m = j + 1; m < i; ++m) acc += sL[i * L::CS + m] * sT[m * L::CS + j];
                    t = -acc;
                }
                sT[i * L::CS + j] = t;
            }
        }
        // ---- K S^T and Q S^T for this block of state rows; X = beta V - beta Gamma K S^T ----
        constexpr int PER = C * BV / 256;
        float qs[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = tid + 256 * e;
            const int i = idx / BV, c = idx % BV;
            float ks = 0.f, qv = 0.f;
#pragma unroll 8
            for (int d = 0; d < DK; ++d) {
                const float s = sS[c * L::QS + d];
                ks += sK[i * L::QS + d] * s;
                qv += sQ[i * L::QS + d] * s;
            }
            qs[e] = qv;
            sX[i * L::VS + c] = sB[i] * (sV[i * L::VS + c] - expf(sG[i]) * ks);
        }
        __syncthreads();
        // ---- U = T X ----
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = tid + 256 * e;
            const int i = idx / BV, c = idx % BV;
            float acc = 0.f;
            for (int m = 0; m <= i; ++m) acc += sT[i * L::CS + m] * sX[m * L::VS + c];
            sU[i * L::VS + c] = acc;
        }
        __syncthreads();
        // ---- O = Gamma Q S^T + Pm U ----
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = tid + 256 * e;
            const int i = idx / BV, c = idx % BV;
            float acc = expf(sG[i]) * qs[e];
            for (int m = 0; m <= i; ++m) acc += sP[i * L::CS + m] * sU[m * L::VS + c];
            if (i < len) store1(p.o + ((size_t)(cs + i) * H + h) * dv + vb * BV + c, p.scale * acc);
        }
        // ---- S <- Gamma_C S + U^T diag(exp(gamma_C - gamma)) K ----
        const float gC = expf(gl);
        for (int idx = tid; idx < BV * DK; idx += 256) {
            const int c = idx / DK, d = idx % DK;
            float acc = gC * sS[c * L::QS + d];
#pragma unroll 8
            for (int i = 0; i < C; ++i) acc += sU[i * L::VS + c] * sD[i] * sK[i * L::QS + d];
            sS[c * L::QS + d] = acc;
        }
    }
    __syncthreads();
    if (p.sfin) {
        for (int idx = tid; idx < BV * DK; idx += 256) {
            const int r = idx / DK, c = idx % DK;
            p.sfin[sbase + (size_t)r * DK + c] = sS[r * L::QS + c];
        }
    }
}

template <int DK, int BV, typename T>
hipError_t launch_f32_t(const ChunkArgs& a) {
    F32Params<T> p;
    p.q = static_cast<const T*>(a.q);
    p.k = static_cast<const T*>(a.k);
    p.v = static_cast<const T*>(a.v);
    p.g = a.g;
    p.beta = a.beta;
    p.gate_params = a.gate_params;
    p.s0 = a.s0;
    p.conv_w = a.conv_w;
    p.conv_state = static_cast<const T*>(a.conv_state);
    p.cu = a.cu;
    p.o = static_cast<T*>(a.o);
    p.sfin = a.sfin;
    p.N = a.N;
    p.T_tot = a.T_tot;
    p.H = a.H;
    p.Hk = a.Hk;
    p.dv = a.dv;
    p.scale = a.scale;
    p.l2norm = a.l2norm;
    const size_t smem = F32Smem<DK, BV>::bytes;
    hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(&chunk_f32_kernel<DK, BV, T>), (int)smem);
    if (e != hipSuccess) return e;
    const int nv = a.dv / BV;
    hipLaunchKernelGGL((chunk_f32_kernel<DK, BV, T>), dim3(a.N * a.H * nv), dim3(256), smem, a.stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_valu(const ChunkArgs& a) {
    // BV must divide every supported dv (32, 64, 128).
    switch (a.dk) {
        case 32: return launch_f32_t<32, 32, T>(a);
        case 64: return launch_f32_t<64, 32, T>(a);
        case 128: return launch_f32_t<128, 16, T>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_f32(const ChunkArgs& a) { return launch_valu<float>(a); }


}  // namespace gdn
