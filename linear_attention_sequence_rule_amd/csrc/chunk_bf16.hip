// chunk_bf16.hip -- fused chunked prefill of the gated delta rule on gfx950 MFMA (bf16 operands,
// fp32 accumulation, fp32 state held in registers across chunks).
//
// Method: page pzsr.cn/news/750, section 1、为什么要设计为chunk的模式 -- cut the sequence into chunks,
// compute inside a chunk in parallel, carry the state serially between chunks, and block the K/V
// dimensions.  The chunk algebra (derived from u_t = beta_t (v_t - alpha_t S_{t-1} k_t),
// S_t = alpha_t S_{t-1} + u_t k_t^T; no chunk algebra is printed on the pages):
//   gamma = inclusive prefix sum of g in the chunk, M_ij = exp(gamma_i - gamma_j) (j <= i),
//   L = strict_lower(diag(beta) (M o Khat Khat^T)),  T = (I + L)^-1,
//   X = diag(beta) V - diag(beta Gamma) Khat S^T,  U = T X,
//   O = diag(Gamma) Qhat S^T + lower(M o Qhat Khat^T) U,
//   S <- Gamma_C S + U^T diag(exp(gamma_C - gamma)) Khat.
// Khat = diag(rk) K with rk = rsqrt(|k|^2 + eps) (likewise Qhat): the raw bf16 rows are the MFMA
// operands (exact), the norms are folded into the row/column scalings above.
//
// Work decomposition: one workgroup (4 wavefronts) per (sequence n, head h, block of 32 state
// rows).  State rows are independent, so the split over row blocks is exact.
//   * waves 0-1 ("state waves") each own 16 state rows c.  The whole state chain of a chunk
//     (K S^T -> X -> U = T X -> O, S update) stays in registers: every 16x16 MFMA output tile is
//     fed to the next product as an operand without leaving the wave, by reading the LDS operand
//     of that product in the matching k order ("chain order": k = 4g+e and 16+4g+e for lane
//     group g = lane/16).  S lives in fp32 accumulators for the whole sequence.
//   * waves 2-3 ("prep waves") compute the state-independent part: the gate prefix sum and decay
//     factors, the masked Gram matrices L and Pm, and T = (I + L)^-1 (16x16 diagonal blocks by
//     fp32 forward substitution, then two block-merge levels on MFMA with bf16 hi/lo operand
//     splitting, accurate to about 2^-16).
// MFMA: v_mfma_f32_16x16x32_bf16.  A: lane l holds A[l%16][8(l/16)+e]; B: B[8(l/16)+e][l%16];
// D: D[4(l/16)+e][l%16] (e = element index).
#include "common.hpp"
#include "kernels.hpp"
#include "prologue.hpp"

namespace gdn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float fx4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;       // chunk length
constexpr int BV = 32;      // state rows per workgroup
constexpr int TSTR = C + 8; // bf16 row stride of token-contiguous tiles (K^T, V^T, T, Pm)
constexpr int LSTR = C + 4; // fp32 row stride of the solve tiles

__device__ __forceinline__ fx4 mfma(bf16x8 a, bf16x8 b, fx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ fx4 zero4() { return fx4{0.f, 0.f, 0.f, 0.f}; }

// 16-byte natural-order fragment: row[kb + 8g .. +7]
__device__ __forceinline__ bf16x8 frag_nat(const __bf16* row, int kb, int g) {
    return *reinterpret_cast<const bf16x8*>(row + kb + 8 * g);
}
// chain-order fragment: row[kb + 4g .. +3] and row[kb + 16 + 4g .. +3]
__device__ __forceinline__ bf16x8 frag_chain(const __bf16* row, int kb, int g) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(row + kb + 4 * g);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(row + kb + 16 + 4 * g);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Two D fragments (rows 4g+e of consecutive 16-row tiles) as one chain-order operand.
__device__ __forceinline__ bf16x8 pack_chain(fx4 a, fx4 b) {
    bf16x8 r;
    r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
    r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
    return r;
}
// fp32 x -> (hi, lo) bf16 with hi + lo = x to about 2^-16 relative.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = (__bf16)x[e];
        hi[e] = h;
        lo[e] = (__bf16)(x[e] - (float)h);
    }
}
// hi/lo product: A B ~ Ah Bh + Ah Bl + Al Bh
__device__ __forceinline__ fx4 mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, fx4 c) {
    c = mfma(ah, bh, c);
    c = mfma(ah, bl, c);
    return mfma(al, bh, c);
}

template <int DK>
struct Smem {
    static constexpr int KSTR = DK + 8;  // bf16 row stride of token-major K and Q
    static constexpr int oK = 0;                                   // bf16 [C][KSTR]
    static constexpr int oQ = oK + C * KSTR * 2;                   // bf16 [C][KSTR]
    static constexpr int oKt = oQ + C * KSTR * 2;                  // bf16 [DK][TSTR]
    static constexpr int oVt = oKt + DK * TSTR * 2;                // bf16 [BV][TSTR]
    static constexpr int oT = oVt + BV * TSTR * 2;                 // bf16 [C][TSTR]  T, row-major
    static constexpr int oPm = oT + C * TSTR * 2;                  // bf16 [C][TSTR]  Pm, row-major
    static constexpr int oL = oPm + C * TSTR * 2;                  // fp32 [C][LSTR]  L, row-major
    static constexpr int oTf = oL + C * LSTR * 4;                  // fp32 [C][LSTR]  T, row-major
    static constexpr int oTt = oTf + C * LSTR * 4;                 // fp32 [C][LSTR]  T, column-major
    static constexpr int oG = oTt + C * LSTR * 4;                  // fp32 gate arrays [12][C]
    static constexpr int bytes = oG + 12 * C * 4;
};
// gate array slots (fp32 [C] each).  Each state wave w keeps its own decay factors in slots
// G_SKK + 3w (beta Gamma rk), G_SORQ + 3w (Gamma rq) and G_SDRK + 3w (exp(gamma_C - gamma) rk).
enum { G_RAW = 0, G_BETA, G_RK, G_RQ, G_GAM0, G_GAM1, G_SKK, G_SORQ, G_SDRK, G_NSLOT = G_SKK + 6 };
static_assert(G_NSLOT <= 12, "gate slots");

template <int DK>
struct Params {
    const __bf16 *q, *k, *v;
    const float *g, *beta, *s0, *conv_w;
    const int32_t* cu;
    __bf16* o;
    float* sfin;
    int N, T_tot, H, dv, nv;
    float scale;
    int l2norm;
};

// ------------------------------------------------------------------------------------------
// chunk loader: global -> LDS (token-major K/Q, transposed K and V), norms, raw gates.
// 256 lanes; one 16-byte part (8 elements) of a K or Q row per lane per pass.
template <int DK>
struct ChunkRegs {
    static constexpr int PPR = DK / 8;          // 16-byte parts per row
    static constexpr int RPP = 256 / PPR;       // rows per pass
    static constexpr int NP = C / RPP;          // passes
    uint4 kr[NP], qr[NP];
    uint4 vr;
    float gr, br;
};

template <int DK>
__device__ __forceinline__ void fetch_chunk(const Params<DK>& p, ChunkRegs<DK>& R, long t0, int len, int h, int vb,
                                            int tid) {
    // Rows past the tail re-read the last valid row (len >= 1) and are zeroed when stored: the
    // loads stay unconditional, so no wait is forced between them.
    using CR = ChunkRegs<DK>;
    const int part = tid % CR::PPR;
#pragma unroll
    for (int j = 0; j < CR::NP; ++j) {
        const int r = min(tid / CR::PPR + j * CR::RPP, len - 1);
        const size_t off = ((size_t)(t0 + r) * p.H + h) * DK + 8 * part;
        R.kr[j] = *reinterpret_cast<const uint4*>(p.k + off);
        R.qr[j] = *reinterpret_cast<const uint4*>(p.q + off);
    }
    {
        // V: one token per lane (part = wave) so the transposed LDS writes are contiguous
        const int r = min(tid % C, len - 1), pv = tid / C;
        R.vr = *reinterpret_cast<const uint4*>(p.v + ((size_t)(t0 + r) * p.H + h) * p.dv + vb * BV + 8 * pv);
    }
    const int r = min(tid % C, len - 1);
    R.gr = p.g[(size_t)(t0 + r) * p.H + h];
    R.br = p.beta[(size_t)(t0 + r) * p.H + h];
}

__device__ __forceinline__ float sumsq8(uint4 u) {
    float s = 0.f;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = __builtin_bit_cast(float, w[i] << 16), b = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        s += a * a + b * b;
    }
    return s;
}

template <int DK>
__device__ __forceinline__ void store_chunk(const ChunkRegs<DK>& R, unsigned char* sm, int len, int l2norm, int tid) {
    using S = Smem<DK>;
    using CR = ChunkRegs<DK>;
    __bf16* sK = reinterpret_cast<__bf16*>(sm + S::oK);
    __bf16* sQ = reinterpret_cast<__bf16*>(sm + S::oQ);
    __bf16* sVt = reinterpret_cast<__bf16*>(sm + S::oVt);
    float* sG = reinterpret_cast<float*>(sm + S::oG);
    const int part = tid % CR::PPR;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < CR::NP; ++j) {
        const int r = tid / CR::PPR + j * CR::RPP;
        const bool in = r < len;
        const uint4 kv = in ? R.kr[j] : z, qv = in ? R.qr[j] : z;
        *reinterpret_cast<uint4*>(sK + r * S::KSTR + 8 * part) = kv;
        *reinterpret_cast<uint4*>(sQ + r * S::KSTR + 8 * part) = qv;
        float sk = group_sum<CR::PPR>(sumsq8(kv));
        float sq = group_sum<CR::PPR>(sumsq8(qv));
        if (part == 0) {
            sG[G_RK * C + r] = in ? (l2norm ? rsqrtf(sk + kL2Eps) : 1.f) : 0.f;
            sG[G_RQ * C + r] = in ? (l2norm ? rsqrtf(sq + kL2Eps) : 1.f) : 0.f;
        }
    }
    {
        const int r = tid % C, pv = tid / C;
        const uint4 vv = r < len ? R.vr : z;
        const uint16_t* vh = reinterpret_cast<const uint16_t*>(&vv);
        uint16_t* vt = reinterpret_cast<uint16_t*>(sVt);
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[(8 * pv + e) * TSTR + r] = vh[e];
    }
    if (tid < C) {
        const bool in = tid < len;
        sG[G_RAW * C + tid] = in ? R.gr : 0.f;
        sG[G_BETA * C + tid] = in ? R.br : 0.f;
    }
}

// ------------------------------------------------------------------------------------------
// prep waves

// inclusive prefix sum of the raw gate over the 64 lanes of a wave
__device__ __forceinline__ float wave_scan(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Wave p0: the strict-lower masked Gram L = strict_lower(diag(beta) (M o Khat Khat^T)), fp32,
// row-major.  K fragments stay in registers: A and B operands of K K^T are the same data.
template <int DK>
__device__ void prep_gram_L(unsigned char* sm, int lane) {
    using S = Smem<DK>;
    constexpr int KS = DK / 32;
    const __bf16* sK = reinterpret_cast<const __bf16*>(sm + S::oK);
    float* sG = reinterpret_cast<float*>(sm + S::oG);
    float* sL = reinterpret_cast<float*>(sm + S::oL);
    const int g = lane / 16, l16 = lane % 16;

    bf16x8 kf[4][KS];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[rb][ks] = frag_nat(sK + (16 * rb + l16) * S::KSTR, 32 * ks, g);
    sG[G_GAM0 * C + lane] = wave_scan(sG[G_RAW * C + lane], lane);

#pragma unroll
    for (int it = 0; it < 4; ++it) {
        fx4 acc[4];
#pragma unroll
        for (int jt = 0; jt <= it; ++jt) acc[jt] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int jt = 0; jt <= it; ++jt) acc[jt] = mfma(kf[it][ks], kf[jt][ks], acc[jt]);
        const int i0 = 16 * it + 4 * g;
        const fx4 gi = *reinterpret_cast<const fx4*>(sG + G_GAM0 * C + i0);
        const fx4 bi = *reinterpret_cast<const fx4*>(sG + G_BETA * C + i0);
        const fx4 ri = *reinterpret_cast<const fx4*>(sG + G_RK * C + i0);
#pragma unroll
        for (int jt = 0; jt <= it; ++jt) {
            const int j = 16 * jt + l16;
            const float gj = sG[G_GAM0 * C + j], rj = sG[G_RK * C + j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = i0 + e;
                sL[i * LSTR + j] = j < i ? bi[e] * ri[e] * rj * __expf(gi[e] - gj) * acc[jt][e] : 0.f;
            }
        }
    }
}

// Wave p1: Pm = lower(M o Qhat Khat^T) (bf16, row-major [i][m]), computed as D = K Q^T so that
// a lane holds 4 consecutive m of one row i.
template <int DK>
__device__ void prep_gram_P(unsigned char* sm, int lane) {
    using S = Smem<DK>;
    constexpr int KS = DK / 32;
    const __bf16* sK = reinterpret_cast<const __bf16*>(sm + S::oK);
    const __bf16* sQ = reinterpret_cast<const __bf16*>(sm + S::oQ);
    float* sG = reinterpret_cast<float*>(sm + S::oG);
    __bf16* sPm = reinterpret_cast<__bf16*>(sm + S::oPm);
    const int g = lane / 16, l16 = lane % 16;

    bf16x8 kf[4][KS], qf[4][KS];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[rb][ks] = frag_nat(sK + (16 * rb + l16) * S::KSTR, 32 * ks, g);
            qf[rb][ks] = frag_nat(sQ + (16 * rb + l16) * S::KSTR, 32 * ks, g);
        }
    sG[G_GAM1 * C + lane] = wave_scan(sG[G_RAW * C + lane], lane);

#pragma unroll
    for (int it = 0; it < 4; ++it) {
        fx4 acc[4];
#pragma unroll
        for (int mt = 0; mt <= it; ++mt) acc[mt] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int mt = 0; mt <= it; ++mt) acc[mt] = mfma(kf[mt][ks], qf[it][ks], acc[mt]);
        const int i = 16 * it + l16;
        const float gi = sG[G_GAM1 * C + i], rqi = sG[G_RQ * C + i];
#pragma unroll
        for (int mt = 0; mt <= it; ++mt) {
            const int m0 = 16 * mt + 4 * g;
            const fx4 gm = *reinterpret_cast<const fx4*>(sG + G_GAM1 * C + m0);
            const fx4 rkm = *reinterpret_cast<const fx4*>(sG + G_RK * C + m0);
            bf16x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = (__bf16)(m0 + e <= i ? rqi * rkm[e] * __expf(gi - gm[e]) * acc[mt][e] : 0.f);
            *reinterpret_cast<bf16x4*>(sPm + i * TSTR + m0) = out;
        }
    }
}

// Solve level 0: invert the 16x16 unit-lower diagonal blocks b0, b0+1 of (I + L) by forward
// substitution, one column per lane (lanes 0..31).  The block's rows of L are read once with
// 16-byte loads; the right-looking update keeps one FMA on the critical path per step.  Writes
// T (fp32 row- and column-major and bf16 row-major).
__device__ void solve_diag(unsigned char* sm, int b0, int lane, int oL, int oTf, int oTt, int oT) {
    const float* sL = reinterpret_cast<const float*>(sm + oL);
    float* sTf = reinterpret_cast<float*>(sm + oTf);
    float* sTt = reinterpret_cast<float*>(sm + oTt);
    __bf16* sT = reinterpret_cast<__bf16*>(sm + oT);
    const int b = b0 + (lane / 16) % 2, j = lane % 16, base = 16 * b;
    fx4 Lr[16][4];
#pragma unroll
    for (int i = 1; i < 16; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (4 * q < i) Lr[i][q] = *reinterpret_cast<const fx4*>(sL + (base + i) * LSTR + base + 4 * q);
    float acc[16], t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const float tm = m == j ? 1.f : (m > j ? -acc[m] : 0.f);
        t[m] = tm;
#pragma unroll
        for (int i = m + 1; i < 16; ++i) acc[i] += Lr[i][m / 4][m % 4] * tm;
    }
    if (lane >= 32) return;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        sTf[(base + m) * LSTR + base + j] = t[m];
        sT[(base + m) * TSTR + base + j] = (__bf16)t[m];
    }
#pragma unroll
    for (int m = 0; m < 16; m += 4)
        *reinterpret_cast<fx4*>(sTt + (base + j) * LSTR + base + m) = fx4{t[m], t[m + 1], t[m + 2], t[m + 3]};
}

// Solve level 1: T_{b+1,b} = -T_{b+1,b+1} L_{b+1,b} T_{b,b} for the 16x16 block pair (b, b+1).
__device__ void solve_level1(unsigned char* sm, int b, int lane, int oL, int oTf, int oTt, int oT) {
    const float* sL = reinterpret_cast<const float*>(sm + oL);
    float* sTf = reinterpret_cast<float*>(sm + oTf);
    float* sTt = reinterpret_cast<float*>(sm + oTt);
    __bf16* sT = reinterpret_cast<__bf16*>(sm + oT);
    const int g = lane / 16, l16 = lane % 16;
    const int r0 = 16 * (b + 1), c0 = 16 * b;
    // Y = L_{b+1,b} T_bb : A = L rows r0+l16, k = m (natural order, k >= 16 zero)
    float a[8], bb[8];
    {
        const int gg = g & 1;  // lanes with g >= 2 read valid memory and zero it (k >= 16 is padding)
        const fx4 a0 = *reinterpret_cast<const fx4*>(sL + (r0 + l16) * LSTR + c0 + 8 * gg);
        const fx4 a1 = *reinterpret_cast<const fx4*>(sL + (r0 + l16) * LSTR + c0 + 8 * gg + 4);
        const fx4 b0v = *reinterpret_cast<const fx4*>(sTt + (c0 + l16) * LSTR + c0 + 8 * gg);  // T_bb column l16
        const fx4 b1v = *reinterpret_cast<const fx4*>(sTt + (c0 + l16) * LSTR + c0 + 8 * gg + 4);
        const float keep = g < 2 ? 1.f : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = keep * a0[e];
            a[4 + e] = keep * a1[e];
            bb[e] = keep * b0v[e];
            bb[4 + e] = keep * b1v[e];
        }
    }
    bf16x8 ah, al, bh, bl;
    split8(a, ah, al);
    split8(bb, bh, bl);
    fx4 y = mfma3(ah, al, bh, bl, zero4());
    // T_{b+1,b} = -T_{b+1,b+1} Y : B = Y from registers (k = 4g+e), A = T rows in the same order
    float a2[8], y2[8];
    {
        const fx4 tv = *reinterpret_cast<const fx4*>(sTf + (r0 + l16) * LSTR + r0 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a2[e] = tv[e];
            y2[e] = y[e];
            a2[4 + e] = 0.f;
            y2[4 + e] = 0.f;
        }
    }
    split8(a2, ah, al);
    split8(y2, bh, bl);
    fx4 t = mfma3(ah, al, bh, bl, zero4());
    // lane holds T[r0 + 4g + e][c0 + l16] = -t[e]
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float v = -t[e];
        sTf[(r0 + 4 * g + e) * LSTR + c0 + l16] = v;
        sT[(r0 + 4 * g + e) * TSTR + c0 + l16] = (__bf16)v;
    }
    *reinterpret_cast<fx4*>(sTt + (c0 + l16) * LSTR + r0 + 4 * g) = fx4{-t[0], -t[1], -t[2], -t[3]};
}

// Solve level 2: columns [16 half, 16 half + 16) of T_BA = -T_BB L_BA T_AA (32x32 blocks A = rows
// 0..31, B = rows 32..63).  Writes bf16 T only.
__device__ void solve_level2(unsigned char* sm, int half, int lane, int oL, int oTf, int oTt, int oT) {
    const float* sL = reinterpret_cast<const float*>(sm + oL);
    const float* sTf = reinterpret_cast<const float*>(sm + oTf);
    const float* sTt = reinterpret_cast<const float*>(sm + oTt);
    __bf16* sT = reinterpret_cast<__bf16*>(sm + oT);
    const int g = lane / 16, l16 = lane % 16;
    const int jc = 16 * half + l16;  // column of T_AA / T_BA handled by this lane (as N index)
    // B operand: T_AA[m][jc], m = 8g+e (natural order over K = 32), column-major source
    float bb[8];
    {
        const fx4 b0v = *reinterpret_cast<const fx4*>(sTt + jc * LSTR + 8 * g);
        const fx4 b1v = *reinterpret_cast<const fx4*>(sTt + jc * LSTR + 8 * g + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bb[e] = b0v[e];
            bb[4 + e] = b1v[e];
        }
    }
    bf16x8 bh, bl;
    split8(bb, bh, bl);
    fx4 y[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        float a[8];
        const fx4 a0 = *reinterpret_cast<const fx4*>(sL + (32 + 16 * it + l16) * LSTR + 8 * g);
        const fx4 a1 = *reinterpret_cast<const fx4*>(sL + (32 + 16 * it + l16) * LSTR + 8 * g + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = a0[e];
            a[4 + e] = a1[e];
        }
        bf16x8 ah, al;
        split8(a, ah, al);
        y[it] = mfma3(ah, al, bh, bl, zero4());
    }
    // T_BA = -T_BB Y : B = Y (chain order: tiles 0/1 rows 4g+e), A = T_BB rows, chain order
    float yv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        yv[e] = y[0][e];
        yv[4 + e] = y[1][e];
    }
    bf16x8 yh, yl;
    split8(yv, yh, yl);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        float a[8];
        const float* row = sTf + (32 + 16 * it + l16) * LSTR + 32;
        const fx4 a0 = *reinterpret_cast<const fx4*>(row + 4 * g);
        const fx4 a1 = *reinterpret_cast<const fx4*>(row + 16 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = a0[e];
            a[4 + e] = a1[e];
        }
        bf16x8 ah, al;
        split8(a, ah, al);
        const fx4 t = mfma3(ah, al, yh, yl, zero4());
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[(32 + 16 * it + 4 * g + e) * TSTR + jc] = (__bf16)(-t[e]);
    }
}

// ------------------------------------------------------------------------------------------
// state waves: everything of one chunk for 16 state rows, in registers.
template <int DK>
struct StateRegs {
    static constexpr int DT = DK / 16;
    fx4 S[DT];     // S^T tiles: lane (c = l%16, g) holds S[c][16 dt + 4g + e]
    bf16x8 xb[2];  // X (chain order over tokens), carried from phase 1 to phase 4
    fx4 ot[4];     // O^T accumulators (S Q^T part, already scaled by Gamma rq)
    float gc;      // Gamma_C = exp(gamma of the last token)
};

// K^T (token-contiguous copy of K for the state update), written by the two state waves: each
// lane owns one token, so consecutive lanes write consecutive 2-byte slots of a K^T row.
template <int DK>
__device__ void transpose_k(unsigned char* sm, int lane, int sw) {
    using S = Smem<DK>;
    constexpr int PPR = DK / 8;
    const __bf16* sK = reinterpret_cast<const __bf16*>(sm + S::oK);
    uint16_t* kt = reinterpret_cast<uint16_t*>(sm + S::oKt);
#pragma unroll
    for (int q = 0; q < PPR / 2; ++q) {
        const int part = sw * (PPR / 2) + q;
        const uint4 v = *reinterpret_cast<const uint4*>(sK + lane * S::KSTR + 8 * part);
        const uint16_t* vh = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
        for (int e = 0; e < 8; ++e) kt[(8 * part + e) * TSTR + lane] = vh[e];
    }
}

// Phase 1 (needs only the chunk inputs and S): own decay factors, K S^T, S Q^T and X.
template <int DK>
__device__ void state_phase1(StateRegs<DK>& st, unsigned char* sm, int lane, int sw, int cbase) {
    using S = Smem<DK>;
    constexpr int KS = DK / 32;
    const __bf16* sK = reinterpret_cast<const __bf16*>(sm + S::oK);
    const __bf16* sQ = reinterpret_cast<const __bf16*>(sm + S::oQ);
    const __bf16* sVt = reinterpret_cast<const __bf16*>(sm + S::oVt);
    float* sG = reinterpret_cast<float*>(sm + S::oG);
    const int g = lane / 16, l16 = lane % 16;
    const int oKK = (G_SKK + 3 * sw) * C, oORQ = (G_SORQ + 3 * sw) * C, oDRK = (G_SDRK + 3 * sw) * C;

    // operand fragments first (chain order: B/A partner is S from registers)
    bf16x8 kfr[4][KS], qfr[4][KS];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kfr[t][ks] = frag_chain(sK + (16 * t + l16) * S::KSTR, 32 * ks, g);
            qfr[t][ks] = frag_chain(sQ + (16 * t + l16) * S::KSTR, 32 * ks, g);
        }

    // decay factors of this chunk (lane = token)
    {
        const float gam = wave_scan(sG[G_RAW * C + lane], lane);
        const float gl = __shfl(gam, C - 1);
        const float Gi = __expf(gam);
        sG[oKK + lane] = sG[G_BETA * C + lane] * Gi * sG[G_RK * C + lane];
        sG[oORQ + lane] = Gi * sG[G_RQ * C + lane];
        sG[oDRK + lane] = __expf(gl - gam) * sG[G_RK * C + lane];
        st.gc = __expf(gl);
    }

    bf16x8 sb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sb[ks] = pack_chain(st.S[2 * ks], st.S[2 * ks + 1]);

    fx4 ks_acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        ks_acc[t] = zero4();
        st.ot[t] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            ks_acc[t] = mfma(kfr[t][ks], sb[ks], ks_acc[t]);   // K S^T  (M = token, N = c)
            st.ot[t] = mfma(sb[ks], qfr[t][ks], st.ot[t]);     // S Q^T  (M = c, N = token)
        }

    fx4 x[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int m0 = 16 * mt + 4 * g;
        const fx4 bm = *reinterpret_cast<const fx4*>(sG + G_BETA * C + m0);
        const fx4 kk = *reinterpret_cast<const fx4*>(sG + oKK + m0);
        const bf16x4 vv = *reinterpret_cast<const bf16x4*>(sVt + (cbase + l16) * TSTR + m0);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[mt][e] = bm[e] * (float)vv[e] - kk[e] * ks_acc[mt][e];
        const float orq = sG[oORQ + 16 * mt + l16];
#pragma unroll
        for (int e = 0; e < 4; ++e) st.ot[mt][e] *= orq;
    }
    st.xb[0] = pack_chain(x[0], x[1]);
    st.xb[1] = pack_chain(x[2], x[3]);
}

// Phase 4 (after T is ready): U = T X, O += Pm U (stored), S <- Gamma_C S + U^T D K.
template <int DK>
__device__ void state_phase4(const Params<DK>& p, StateRegs<DK>& st, unsigned char* sm, int lane, int sw, int cbase,
                             long t0, int len, int h, int vb) {
    using S = Smem<DK>;
    constexpr int DT = DK / 16;
    const __bf16* sKt = reinterpret_cast<const __bf16*>(sm + S::oKt);
    const __bf16* sT = reinterpret_cast<const __bf16*>(sm + S::oT);
    const __bf16* sPm = reinterpret_cast<const __bf16*>(sm + S::oPm);
    const float* sG = reinterpret_cast<const float*>(sm + S::oG);
    const int g = lane / 16, l16 = lane % 16;
    const int oDRK = (G_SDRK + 3 * sw) * C;

    // T and Pm fragments (k-step 1 only for row tiles 2, 3: both are lower triangular)
    bf16x8 tf[4][2], pf[4][2];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
            if (s2 == 0 || it >= 2) {
                tf[it][s2] = frag_chain(sT + (16 * it + l16) * TSTR, 32 * s2, g);
                pf[it][s2] = frag_chain(sPm + (16 * it + l16) * TSTR, 32 * s2, g);
            }
    bf16x8 kt[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) kt[dt][s2] = frag_chain(sKt + (16 * dt + l16) * TSTR, 32 * s2, g);

    fx4 u[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) u[it] = mfma(tf[it][0], st.xb[0], zero4());
#pragma unroll
    for (int it = 2; it < 4; ++it) u[it] = mfma(tf[it][1], st.xb[1], u[it]);
    bf16x8 ub[2];
    ub[0] = pack_chain(u[0], u[1]);
    ub[1] = pack_chain(u[2], u[3]);

    // U^T scaled by exp(gamma_C - gamma) rk for the state update
    fx4 ut[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const fx4 d = *reinterpret_cast<const fx4*>(sG + oDRK + 16 * it + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) ut[it][e] = u[it][e] * d[e];
    }
    bf16x8 utb[2];
    utb[0] = pack_chain(ut[0], ut[1]);
    utb[1] = pack_chain(ut[2], ut[3]);

#pragma unroll
    for (int it = 0; it < 4; ++it) st.ot[it] = mfma(ub[0], pf[it][0], st.ot[it]);
#pragma unroll
    for (int it = 2; it < 4; ++it) st.ot[it] = mfma(ub[1], pf[it][1], st.ot[it]);

#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) st.S[dt][e] *= st.gc;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) st.S[dt] = mfma(kt[dt][s2], utb[s2], st.S[dt]);

    // store O (lane: token i = 16 it + l16, state rows cbase + 4g .. +3)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int i = 16 * it + l16;
        if (i < len) {
            bf16x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (__bf16)(p.scale * st.ot[it][e]);
            *reinterpret_cast<bf16x4*>(p.o + ((size_t)(t0 + i) * p.H + h) * p.dv + vb * BV + cbase + 4 * g) = out;
        }
    }
}

// ------------------------------------------------------------------------------------------
template <int DK>
__global__ __launch_bounds__(256) void chunk_bf16_kernel(Params<DK> p) {
    using S = Smem<DK>;
    extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
    const int tid = threadIdx.x;
    const int wid = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;

    // XCD-aware order: the nv row-block workgroups of one (n, h) share blockIdx mod 8 (same XCD,
    // same L2) when the pair count allows it.
    const int P = p.N * p.H;
    int pair, vb;
    const int b = blockIdx.x;
    if (P % 8 == 0) {
        vb = (b / 8) % p.nv;
        pair = (b / (8 * p.nv)) * 8 + b % 8;
    } else {
        vb = b % p.nv;
        pair = b / p.nv;
    }
    const int n = pair / p.H, h = pair % p.H;
    long bos, eos;
    if (p.cu) {
        bos = p.cu[n];
        eos = p.cu[n + 1];
    } else {
        const long L = p.T_tot / p.N;
        bos = (long)n * L;
        eos = bos + L;
    }
    const int nchunks = (int)((eos - bos + C - 1) / C);

    // The strict-upper off-diagonal blocks of T (bf16 and both fp32 copies) and the masked-out
    // tiles of Pm are read as zeros but never written: clear them once.
    {
        __bf16* sT = reinterpret_cast<__bf16*>(sm + S::oT);
        __bf16* sPm = reinterpret_cast<__bf16*>(sm + S::oPm);
        float* sTf = reinterpret_cast<float*>(sm + S::oTf);
        float* sTt = reinterpret_cast<float*>(sm + S::oTt);
        for (int i = tid; i < C * TSTR; i += 256) {
            sT[i] = (__bf16)0.f;
            sPm[i] = (__bf16)0.f;
        }
        for (int i = tid; i < C * LSTR; i += 256) {
            sTf[i] = 0.f;
            sTt[i] = 0.f;
        }
    }

    StateRegs<DK> st;
    const bool is_state = wid < 2;
    const int cbase = 16 * wid;
    const int g = lane / 16, l16 = lane % 16;
    const size_t srow0 = ((size_t)pair * p.dv + vb * BV + cbase + l16) * DK;  // state row c of this lane
    if (is_state) {
#pragma unroll
        for (int dt = 0; dt < StateRegs<DK>::DT; ++dt) {
            if (p.s0) {
                const float4 v = *reinterpret_cast<const float4*>(p.s0 + srow0 + 16 * dt + 4 * g);
                st.S[dt] = fx4{v.x, v.y, v.z, v.w};
            } else {
                st.S[dt] = zero4();
            }
        }
    }

    ChunkRegs<DK> R;
    if (nchunks > 0) fetch_chunk<DK>(p, R, bos, (int)min((long)C, eos - bos), h, vb, tid);

    for (int c = 0; c < nchunks; ++c) {
        const long t0 = bos + (long)c * C;
        const int len = (int)min((long)C, eos - t0);
        store_chunk<DK>(R, sm, len, p.l2norm, tid);
        if (c + 1 < nchunks) {
            const long t1 = t0 + C;
            fetch_chunk<DK>(p, R, t1, (int)min((long)C, eos - t1), h, vb, tid);
        }
        __syncthreads();
        if (wid == 2) prep_gram_L<DK>(sm, lane);
        if (wid == 3) prep_gram_P<DK>(sm, lane);
        if (is_state) {
            transpose_k<DK>(sm, lane, wid);
            state_phase1<DK>(st, sm, lane, wid, cbase);
        }
        __syncthreads();
        if (wid == 2) {
            solve_diag(sm, 0, lane, S::oL, S::oTf, S::oTt, S::oT);
            solve_level1(sm, 0, lane, S::oL, S::oTf, S::oTt, S::oT);
        }
        if (wid == 3) {
            solve_diag(sm, 2, lane, S::oL, S::oTf, S::oTt, S::oT);
            solve_level1(sm, 2, lane, S::oL, S::oTf, S::oTt, S::oT);
        }
        __syncthreads();
        if (wid >= 2) solve_level2(sm, wid - 2, lane, S::oL, S::oTf, S::oTt, S::oT);
        __syncthreads();
        if (is_state) state_phase4<DK>(p, st, sm, lane, wid, cbase, t0, len, h, vb);
        __syncthreads();
    }

    if (is_state && p.sfin) {
#pragma unroll
        for (int dt = 0; dt < StateRegs<DK>::DT; ++dt) {
            const fx4 v = st.S[dt];
            *reinterpret_cast<float4*>(p.sfin + srow0 + 16 * dt + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

template <int DK>
hipError_t launch_t(const ChunkArgs& a) {
    Params<DK> p;
    p.q = static_cast<const __bf16*>(a.q);
    p.k = static_cast<const __bf16*>(a.k);
    p.v = static_cast<const __bf16*>(a.v);
    p.g = a.g;
    p.beta = a.beta;
    p.s0 = a.s0;
    p.conv_w = a.conv_w;
    p.cu = a.cu;
    p.o = static_cast<__bf16*>(a.o);
    p.sfin = a.sfin;
    p.N = a.N;
    p.T_tot = a.T_tot;
    p.H = a.H;
    p.dv = a.dv;
    p.nv = a.dv / BV;
    p.scale = a.scale;
    p.l2norm = a.l2norm;
    const int smem = Smem<DK>::bytes;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_bf16_kernel<DK>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    const int grid = a.N * a.H * p.nv;
    hipLaunchKernelGGL((chunk_bf16_kernel<DK>), dim3(grid), dim3(256), smem, a.stream, p);
    return hipGetLastError();
}

}  // namespace

size_t chunk_bf16_workspace(int, int, int, int, int, bool) { return 0; }

hipError_t launch_chunk_bf16(const ChunkArgs& a) {
    if (a.conv_w) return launch_chunk_valu_bf16(a);  // conv prologue: VALU path until the fused loader lands
    switch (a.dk) {
        case 32: return launch_t<32>(a);
        case 64: return launch_t<64>(a);
        case 128: return launch_t<128>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
