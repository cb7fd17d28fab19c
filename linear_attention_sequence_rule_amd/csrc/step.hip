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
// Layout: one workgroup (256 lanes) per (n, h).  A row of dk fp32 is dk/4 lanes x float4, so
// each load instruction of a wavefront covers whole contiguous rows; all ROWS_PER_LANE row
// loads of a lane are issued before the first use (many KB in flight per CU).  Row dot
// products reduce over the dk/4 lanes of a row with DPP/swizzle moves.  State loads and
// stores are non-temporal: each state byte is touched once per step.
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

template <int DK, int DV, typename T>
__global__ __launch_bounds__(256) void step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const float* __restrict__ g,
                                                   const float* __restrict__ beta, float* __restrict__ state,
                                                   T* __restrict__ o, float scale, int l2norm) {
    constexpr int LPR = DK / 4;             // lanes per state row
    constexpr int RPP = 256 / LPR;          // rows per pass of the workgroup
    constexpr int RPL = DV / RPP > 0 ? DV / RPP : 1;  // rows per lane
    static_assert(DV % RPP == 0 || RPP > DV, "row tiling");
    const int nh = blockIdx.x;
    const int tid = threadIdx.x;
    const int c = tid % LPR;        // float4 column of this lane
    const int r0 = tid / LPR;       // first row of this lane
    const bool active = r0 < DV;    // only when RPP > DV (small heads)

    float* S = state + (size_t)nh * DV * DK;
    float4 s[RPL];
    if (active) {
#pragma unroll
        for (int j = 0; j < RPL; ++j)
            s[j] = nt_load4(S + (size_t)(r0 + j * RPP) * DK + 4 * c);
    }

    float4 kk = load4(k + (size_t)nh * DK + 4 * c);
    float4 qq = load4(q + (size_t)nh * DK + 4 * c);
    const float alpha = expf(g[nh]);
    const float b = beta[nh];
    float vr[RPL];
#pragma unroll
    for (int j = 0; j < RPL; ++j) vr[j] = active ? load1(v + (size_t)nh * DV + r0 + j * RPP) : 0.f;

    if (l2norm) {
        float sk = group_sum<LPR>(kk.x * kk.x + kk.y * kk.y + kk.z * kk.z + kk.w * kk.w);
        float sq = group_sum<LPR>(qq.x * qq.x + qq.y * qq.y + qq.z * qq.z + qq.w * qq.w);
        const float rk = rsqrtf(sk + kL2Eps), rq = rsqrtf(sq + kL2Eps);
        kk.x *= rk; kk.y *= rk; kk.z *= rk; kk.w *= rk;
        qq.x *= rq; qq.y *= rq; qq.z *= rq; qq.w *= rq;
    }
    const float kq = group_sum<LPR>(kk.x * qq.x + kk.y * qq.y + kk.z * qq.z + kk.w * qq.w);

    if (!active) return;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        float r = group_sum<LPR>(s[j].x * kk.x + s[j].y * kk.y + s[j].z * kk.z + s[j].w * kk.w);
        float p = group_sum<LPR>(s[j].x * qq.x + s[j].y * qq.y + s[j].z * qq.z + s[j].w * qq.w);
        const float u = b * (vr[j] - alpha * r);
        s[j].x = alpha * s[j].x + u * kk.x;
        s[j].y = alpha * s[j].y + u * kk.y;
        s[j].z = alpha * s[j].z + u * kk.z;
        s[j].w = alpha * s[j].w + u * kk.w;
        if (c == 0) store1(o + (size_t)nh * DV + r0 + j * RPP, scale * (alpha * p + u * kq));
    }
#pragma unroll
    for (int j = 0; j < RPL; ++j)
        nt_store4(S + (size_t)(r0 + j * RPP) * DK + 4 * c, s[j]);
}

template <int DK, int DV, typename T>
static hipError_t launch_step_t(const StepArgs& a) {
    hipLaunchKernelGGL((step_kernel<DK, DV, T>), dim3(a.N * a.H), dim3(256), 0, a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       a.g, a.beta, a.state, static_cast<T*>(a.o), a.scale, a.l2norm);
    return hipGetLastError();
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
