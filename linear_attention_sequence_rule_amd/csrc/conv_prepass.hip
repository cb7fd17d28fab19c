// conv_prepass.hip -- the conv prologue of a bf16 prefill as a streaming pass over the raw inputs
// (page maplevalley.com.cn/news/1910399, section 3.1, 卷积预处理): every q, k and v channel of
// every token becomes SiLU(w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t) in bf16, written to the
// workspace in the layout of the input, and the prefill kernel then runs on these rows.
//
// Inside the prefill kernel the same conv is recomputed by every workgroup that reads a head (the
// value rows of a head are split over several workgroups) and costs two transcendentals per element
// on the critical path of a chunk; here each element is computed once, at the cost of writing and
// reading the convolved rows (6 bytes per element more HBM traffic in bf16).
//
// Before a sequence start the taps read the sequence's conv history (conv_state, oldest first) or
// zeros.  One lane owns eight adjacent channels of one tensor (16 bytes) and walks TT consecutive
// tokens of the packed token axis with the last three raw inputs in registers: it issues all of its
// token loads first, and a wavefront's loads and stores are 1 KB contiguous pieces of a token row.
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

namespace {

constexpr int TT = 16;  // tokens per lane
constexpr int CPL = 8;  // channels per lane (16 bytes of bf16)

__device__ __forceinline__ void ld8(const bf16* p, float (&x)[CPL]) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __builtin_bit_cast(float, u[i] << 16);
        x[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xffff0000u);
    }
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// streaming accesses: every raw and convolved element is touched once here
__device__ __forceinline__ uint4 raw8(const bf16* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void out8(bf16* p, uint4 v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void unpack8(uint4 v, float (&x)[CPL]) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __builtin_bit_cast(float, u[i] << 16);
        x[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ float silu_f(float y) { return y / (1.f + __expf(-y)); }

__global__ __launch_bounds__(256) void conv_prepass_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                           const bf16* __restrict__ v, const float* __restrict__ w,
                                                           const bf16* __restrict__ hist, const int32_t* __restrict__ cu,
                                                           bf16* __restrict__ qo, bf16* __restrict__ ko,
                                                           bf16* __restrict__ vo, int N, int T_tot, int H, int Hk,
                                                           int dk, int dv) {
    const long Kc = (long)Hk * dk, Vc = (long)H * dv, CC = 2 * Kc + Vc;
    const long ch = (long)CPL * ((long)blockIdx.y * 256 + threadIdx.x);  // first of the lane's channels
    const long t0 = (long)blockIdx.x * TT, t1 = min((long)T_tot, t0 + TT);
    if (ch >= CC) return;
    const bf16* src;
    bf16* dst;
    long width, col;
    if (ch < Kc) {
        src = q, dst = qo, width = Kc, col = ch;
    } else if (ch < 2 * Kc) {
        src = k, dst = ko, width = Kc, col = ch - Kc;
    } else {
        src = v, dst = vo, width = Vc, col = ch - 2 * Kc;
    }
    src += col;
    dst += col;
    // the lane's token loads first: independent of the sequence bookkeeping below
    uint4 xr[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i)
        if (t0 + i < t1) xr[i] = raw8(src + (t0 + i) * width);

    // the sequence of token t0 (wave-uniform): the last n with start(n) <= t0
    const long L = cu ? 0 : T_tot / N;
    auto start = [&](int n) -> long { return cu ? (long)cu[n] : (long)n * L; };
    int n;
    if (cu) {
        int lo = 0, hi = N;  // start(lo) <= t0 < start(hi) (start(N) = T_tot)
        while (hi - lo > 1) {
            const int mid = (lo + hi) / 2;
            if (cu[mid] <= t0) lo = mid; else hi = mid;
        }
        n = lo;
    } else {
        n = (int)(t0 / L);
    }
    // raw input s of sequence nn (bos <= s) or its history entry (s < bos)
    auto raw = [&](long s, long bos, int nn, float (&x)[CPL]) {
        if (s >= bos) {
            ld8(src + s * width, x);
        } else if (hist) {
            ld8(hist + ((long)nn * 3 + (3 + s - bos)) * CC + ch, x);
        } else {
#pragma unroll
            for (int c = 0; c < CPL; ++c) x[c] = 0.f;
        }
    };
    float wt[CPL][4];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const float4 wv = *reinterpret_cast<const float4*>(w + 4 * (ch + c));
        wt[c][0] = wv.x, wt[c][1] = wv.y, wt[c][2] = wv.z, wt[c][3] = wv.w;
    }
    long bos = start(n);
    float h0[CPL], h1[CPL], h2[CPL];
    raw(t0 - 3, bos, n, h0);
    raw(t0 - 2, bos, n, h1);
    raw(t0 - 1, bos, n, h2);
    long nxt = start(n + 1);  // start(N) = T_tot
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        const long t = t0 + i;
        if (t >= t1) break;
        if (t >= nxt) {  // a new sequence starts at t (after any zero-length ones)
            do {
                ++n;
                bos = nxt;
                nxt = start(n + 1);
            } while (t >= nxt);
            raw(t - 3, bos, n, h0);
            raw(t - 2, bos, n, h1);
            raw(t - 1, bos, n, h2);
        }
        float x[CPL];
        unpack8(xr[i], x);
        uint32_t o[CPL / 2];
#pragma unroll
        for (int c = 0; c < CPL; c += 2) {
            const float ya = wt[c][0] * h0[c] + wt[c][1] * h1[c] + wt[c][2] * h2[c] + wt[c][3] * x[c];
            const float yb = wt[c + 1][0] * h0[c + 1] + wt[c + 1][1] * h1[c + 1] + wt[c + 1][2] * h2[c + 1] +
                             wt[c + 1][3] * x[c + 1];
            o[c / 2] = (uint32_t)f32_to_bf16(silu_f(ya)) | ((uint32_t)f32_to_bf16(silu_f(yb)) << 16);
        }
        out8(dst + t * width, make_uint4(o[0], o[1], o[2], o[3]));
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            h0[c] = h1[c];
            h1[c] = h2[c];
            h2[c] = x[c];
        }
    }
}

}  // namespace

hipError_t launch_conv_prepass(const ChunkArgs& a, void* out, ChunkArgs& conv_args) {
    auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    unsigned char* base = static_cast<unsigned char*>(out);
    bf16* qo = reinterpret_cast<bf16*>(base);
    bf16* ko = reinterpret_cast<bf16*>(base + a256((size_t)a.T_tot * a.Hk * a.dk * 2));
    bf16* vo = reinterpret_cast<bf16*>(base + 2 * a256((size_t)a.T_tot * a.Hk * a.dk * 2));
    conv_args = a;
    conv_args.q = qo;
    conv_args.k = ko;
    conv_args.v = vo;
    conv_args.conv_w = nullptr;
    conv_args.conv_state = nullptr;
    if (a.T_tot == 0) return hipSuccess;
    const long CC = 2L * a.Hk * a.dk + (long)a.H * a.dv;
    const dim3 grid((unsigned)((a.T_tot + TT - 1) / TT), (unsigned)((CC / CPL + 255) / 256));
    hipLaunchKernelGGL(conv_prepass_kernel, grid, dim3(256), 0, a.stream, static_cast<const bf16*>(a.q),
                       static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v), a.conv_w,
                       static_cast<const bf16*>(a.conv_state), a.cu, qo, ko, vo, a.N, a.T_tot, a.H, a.Hk, a.dk, a.dv);
    return hipGetLastError();
}

}  // namespace gdn
