// step.hip -- single-token recurrent decode of the gated delta rule, state updated in place.
//
// Page pzsr.cn/news/750, section a、增量更新: the state has a fixed size (one 128x128 fp32
// matrix per head) and each new token first decays the whole state by alpha, then erases and
// writes along the current key with strength beta.  Per (sequence n, head h) and state row i
// (the value index):
//     r_i = S_i . k,  p_i = S_i . q,  u_i = beta (v_i - alpha r_i),
//     S_i <- alpha S_i + u_i k,        o_i = scale (alpha p_i + u_i (k . q)).
// The second line is o = S_new q expanded, so S is read once and written once.
//
// HBM-bound: 2 * dv * dk * 4 bytes of state traffic per (n, h) against 2 * dv * dk * 3 flops.
// Layout: one workgroup per (n, h), of step_threads lanes (1024 for dk = dv = 128: many waves with
// few loads each keep HBM busier than few waves with many; 173 us against 189 us with 256 lanes
// on the 256 x 32-head decode).  A row of dk fp32 is dk/4 lanes x float4, so each load
// instruction of a wavefront covers whole contiguous rows; all of a lane's row loads are issued
// before the first use.  Row dot
// products reduce over the dk/4 lanes of a row with DPP/swizzle moves.  State loads and
// stores are non-temporal: each state byte is touched once per step.
#include "common.hpp"
#include "kernels.hpp"
#include "prologue.hpp"

namespace gdn {

// lanes per workgroup: up to 1024, and no more than one float4 of the state per lane per pass
template <int DK, int DV>
constexpr int step_threads() {
    return 1024 < DV * (DK / 4) ? 1024 : DV * (DK / 4);
}

// Conv prologue of one decode token (page maplevalley.com.cn/news/1910399, section 3.1, 卷积预处理):
// channel i of the (n, h) pair's 2 DK + DV channels (q and k of its query/key head hk, then v)
// becomes SiLU(w0 h0 + w1 h1 + w2 h2 + w3 x) from the three previous raw inputs h0, h1, h2
// (oldest first) in conv_state [N, 3, 2 Hk DK + H DV] and the raw input x; the result goes to
// xs[i] (LDS).  With shift (each query/key head read by this workgroup only, Hk = H), the
// channel's history is also shifted by one token in place: every history entry is read and
// written by the one lane that owns its channel, so no synchronisation is needed.  When several
// value heads share a query/key head, its history is read by several workgroups and a separate
// launch shifts the whole conv state afterwards.
template <int DK, int DV, typename T>
__device__ __forceinline__ void conv_token(const T* q, const T* k, const T* v, const float* conv_w, T* conv_state,
                                           float* xs, int nh, int H, int Hk, int tid, bool shift) {
    const size_t CC = (size_t)2 * Hk * DK + (size_t)H * DV;  // conv channels per token
    const int n = nh / H, h = nh % H, hk = h / (H / Hk);
    const size_t nk = (size_t)n * Hk + hk;
    T* hs = conv_state + (size_t)n * 3 * CC;
    for (int i = tid; i < 2 * DK + DV; i += step_threads<DK, DV>()) {
        size_t c;
        float x;
        if (i < DK) {
            c = (size_t)hk * DK + i;
            x = load1(q + nk * DK + i);
        } else if (i < 2 * DK) {
            c = (size_t)(Hk + hk) * DK + (i - DK);
            x = load1(k + nk * DK + (i - DK));
        } else {
            c = (size_t)2 * Hk * DK + (size_t)h * DV + (i - 2 * DK);
            x = load1(v + (size_t)nh * DV + (i - 2 * DK));
        }
        const float h0 = load1(hs + c), h1 = load1(hs + CC + c), h2 = load1(hs + 2 * CC + c);
        const float4 w = load4(conv_w + 4 * c);
        const float acc = w.x * h0 + w.y * h1 + w.z * h2 + w.w * x;
        xs[i] = acc / (1.f + expf(-acc));
        if (shift) {
            store1(hs + c, h1);
            store1(hs + CC + c, h2);
            store1(hs + 2 * CC + c, x);
        }
    }
}

// With CONV, q, k and v are the raw inputs of the conv prologue (conv_token above) and conv_state
// carries the history; with gate_params, g and beta are the raw a and b of the gate
// parameterisation (section 2.1 of the same page).  With NORM, the output row goes through the
// epilogue o * rsqrt(mean(o^2) + eps) * (1 + w) * sigmoid(z) before it is stored (zero-centred
// RMSNorm, section 3.2 of the same page; sigmoid output gate, page
// "GDN融合门控注意力的动态资源分配机制，AI智能体调动实战演练", section 2): the workgroup holds the
// whole row, so the epilogue costs no extra pass over o.
// At least 4 waves per SIMD (at most 128 VGPRs): the state streams through at full occupancy.
template <int DK, int DV, typename T, bool CONV, bool NORM>
__global__ __launch_bounds__((step_threads<DK, DV>())) __attribute__((amdgpu_waves_per_eu(4))) void step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const float* __restrict__ g,
                                                   const float* __restrict__ beta, const float* __restrict__ gate_params,
                                                   float* __restrict__ state, const float* __restrict__ conv_w,
                                                   T* __restrict__ conv_state, const T* __restrict__ out_gate,
                                                   const float* __restrict__ norm_weight, T* __restrict__ o, int H,
                                                   int Hk, float scale, float norm_eps, int l2norm) {
    constexpr int LPR = DK / 4;             // lanes per state row
    constexpr int NTH = step_threads<DK, DV>();
    constexpr int RPP = NTH / LPR;          // rows per pass of the workgroup
    constexpr int RPL = DV / RPP > 0 ? DV / RPP : 1;  // rows per lane
    static_assert(DV % RPP == 0 && RPP <= DV, "row tiling: every lane owns rows (no lane leaves early)");
    __shared__ float xs[CONV ? 2 * DK + DV : 1];
    __shared__ float xo[NORM ? DV : 1];     // the output row before the epilogue
    __shared__ float red[NORM ? NTH / 64 : 1];  // per-wave sums of squares
    const int nh = blockIdx.x;
    const int tid = threadIdx.x;
    const int c = tid % LPR;        // float4 column of this lane
    const int r0 = tid / LPR;       // first row of this lane

    // the gates first: their temporaries are dead before the state rows arrive
    float gg = g[nh], b = beta[nh];
    if (gate_params) {
        const int h = nh % H;
        gg = raw_decay(gg, -expf(gate_params[h]), gate_params[H + h]);
        b = raw_beta(b);
    }
    const float alpha = expf(gg);

    float* S = state + (size_t)nh * DV * DK;
    float4 s[RPL];
#pragma unroll
    for (int j = 0; j < RPL; ++j) s[j] = nt_load4(S + (size_t)(r0 + j * RPP) * DK + 4 * c);

    float4 kk, qq;
    float vr[CONV ? 1 : RPL];  // values (with CONV they stay in LDS until used)
    if constexpr (CONV) {
        conv_token<DK, DV, T>(q, k, v, conv_w, conv_state, xs, nh, H, Hk, tid, H == Hk);
        // LDS hand-off only: the barrier need not wait for the state loads in flight
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        qq = *reinterpret_cast<const float4*>(xs + 4 * c);
        kk = *reinterpret_cast<const float4*>(xs + DK + 4 * c);
    } else {
        const size_t nk = (size_t)(nh / H) * Hk + (nh % H) / (H / Hk);  // (sequence, query/key head)
        kk = load4(k + nk * DK + 4 * c);
        qq = load4(q + nk * DK + 4 * c);
#pragma unroll
        for (int j = 0; j < RPL; ++j) vr[j] = load1(v + (size_t)nh * DV + r0 + j * RPP);
    }
    if (l2norm) {
        float sk = group_sum<LPR>(kk.x * kk.x + kk.y * kk.y + kk.z * kk.z + kk.w * kk.w);
        float sq = group_sum<LPR>(qq.x * qq.x + qq.y * qq.y + qq.z * qq.z + qq.w * qq.w);
        const float rk = rsqrtf(sk + kL2Eps), rq = rsqrtf(sq + kL2Eps);
        kk.x *= rk; kk.y *= rk; kk.z *= rk; kk.w *= rk;
        qq.x *= rq; qq.y *= rq; qq.z *= rq; qq.w *= rq;
    }
    const float kq = group_sum<LPR>(kk.x * qq.x + kk.y * qq.y + kk.z * qq.z + kk.w * qq.w);

#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        float r = group_sum<LPR>(s[j].x * kk.x + s[j].y * kk.y + s[j].z * kk.z + s[j].w * kk.w);
        float p = group_sum<LPR>(s[j].x * qq.x + s[j].y * qq.y + s[j].z * qq.z + s[j].w * qq.w);
        const float vj = CONV ? xs[2 * DK + r0 + j * RPP] : vr[CONV ? 0 : j];
        const float u = b * (vj - alpha * r);
        s[j].x = alpha * s[j].x + u * kk.x;
        s[j].y = alpha * s[j].y + u * kk.y;
        s[j].z = alpha * s[j].z + u * kk.z;
        s[j].w = alpha * s[j].w + u * kk.w;
        if (c == 0) {
            const float ov = scale * (alpha * p + u * kq);
            if constexpr (NORM)
                xo[r0 + j * RPP] = ov;
            else
                store1(o + (size_t)nh * DV + r0 + j * RPP, ov);
        }
    }
#pragma unroll
    for (int j = 0; j < RPL; ++j)
        nt_store4(S + (size_t)(r0 + j * RPP) * DK + 4 * c, s[j]);
    if constexpr (NORM) {
        // the epilogue inputs of output element tid, loaded only now so that they hold no registers
        // through the row loop; their latency overlaps the reduction
        float zo = 0.f, wo = 0.f;
        if (tid < DV) {
            zo = load1(out_gate + (size_t)nh * DV + tid);
            wo = norm_weight[tid];
        }
        // LDS hand-offs only: the barriers need not wait for the state stores in flight
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        const float x = tid < DV ? xo[tid] : 0.f;
        const float ss = group_sum<64>(x * x);
        if (tid % 64 == 0) red[tid / 64] = ss;
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        float rs = 0.f;
#pragma unroll
        for (int w = 0; w < NTH / 64; ++w) rs += red[w];
        const float inv = rsqrtf(rs * (1.f / DV) + norm_eps);
        if (tid < DV) store1(o + (size_t)nh * DV + tid, x * inv * (1.f + wo) / (1.f + expf(-zo)));
    }
}

template <int DK, int DV, typename T, bool CONV, bool NORM>
static hipError_t launch_step_v(const StepArgs& a) {
    hipLaunchKernelGGL((step_kernel<DK, DV, T, CONV, NORM>), dim3(a.N * a.H), dim3(step_threads<DK, DV>()), 0, a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.g, a.beta,
                       a.gate_params, a.state, a.conv_w, static_cast<T*>(a.conv_state),
                       static_cast<const T*>(a.out_gate), a.norm_weight, static_cast<T*>(a.o), a.H, a.Hk, a.scale,
                       a.norm_eps, a.l2norm);
    return hipGetLastError();
}

template <int DK, int DV, typename T>
static hipError_t launch_step_t(const StepArgs& a) {
    if (a.conv_w)
        return a.out_gate ? launch_step_v<DK, DV, T, true, true>(a) : launch_step_v<DK, DV, T, true, false>(a);
    return a.out_gate ? launch_step_v<DK, DV, T, false, true>(a) : launch_step_v<DK, DV, T, false, false>(a);
}

template <typename T>
static hipError_t launch_step_dt(const StepArgs& a) {
#define GDN_STEP_CASE(K, V) \
    if (a.dk == K && a.dv == V) return launch_step_t<K, V, T>(a);
    GDN_STEP_CASE(32, 32) GDN_STEP_CASE(32, 64) GDN_STEP_CASE(32, 128)
    GDN_STEP_CASE(64, 32) GDN_STEP_CASE(64, 64) GDN_STEP_CASE(64, 128)
    GDN_STEP_CASE(128, 32) GDN_STEP_CASE(128, 64) GDN_STEP_CASE(128, 128)
#undef GDN_STEP_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_step(const StepArgs& a) {
    return a.bf16 ? launch_step_dt<bf16>(a) : launch_step_dt<float>(a);
}

}  // namespace gdn
