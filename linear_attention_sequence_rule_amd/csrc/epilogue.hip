// epilogue.hip -- the output epilogue of a prefill call: a zero-centred RMSNorm of each
// (token, head) row of o over dv, then a sigmoid output gate, in place:
//     o[r, i] <- o[r, i] * rsqrt(mean_i o[r, i]^2 + eps) * (1 + w[i]) * sigmoid(z[r, i])
// (page maplevalley.com.cn/news/1910399, section 3.2 Zero-Centered RMSNorm; page
// "GDN融合门控注意力的动态资源分配机制，AI智能体调动实战演练", section 2, on the sigmoid output gate).
//
// The prefill kernel splits a head's dv rows of the state over several workgroups, so no workgroup
// holds a whole output row; this pass runs after it.  (The decode step holds the whole row and
// applies the same epilogue inside its own kernel.)  HBM-bound: o read and written, z read, 6 bytes
// per element in bf16.  Each lane owns 16 contiguous bytes of a row; a row's lanes reduce the sum of
// squares with DPP moves.
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

namespace {

template <int E>
__device__ __forceinline__ void load_vec(const float* p, float (&x)[E]) {
#pragma unroll
    for (int i = 0; i < E; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(p + i);
        x[i] = v.x, x[i + 1] = v.y, x[i + 2] = v.z, x[i + 3] = v.w;
    }
}
template <int E>
__device__ __forceinline__ void load_vec(const bf16* p, float (&x)[E]) {
    static_assert(E == 8, "16 bytes of bf16");
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __builtin_bit_cast(float, u[i] << 16);
        x[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xffff0000u);
    }
}
template <int E>
__device__ __forceinline__ void store_vec(float* p, const float (&x)[E]) {
#pragma unroll
    for (int i = 0; i < E; i += 4) *reinterpret_cast<float4*>(p + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
}
template <int E>
__device__ __forceinline__ void store_vec(bf16* p, const float (&x)[E]) {
    static_assert(E == 8, "16 bytes of bf16");
    uint4 v;
    v.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    v.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
    v.z = (uint32_t)f32_to_bf16(x[4]) | ((uint32_t)f32_to_bf16(x[5]) << 16);
    v.w = (uint32_t)f32_to_bf16(x[6]) | ((uint32_t)f32_to_bf16(x[7]) << 16);
    *reinterpret_cast<uint4*>(p) = v;
}

template <typename T, int DV>
__global__ __launch_bounds__(256) void gated_norm_kernel(T* __restrict__ o, const T* __restrict__ z,
                                                         const float* __restrict__ w, long rows, float eps) {
    constexpr int E = 16 / sizeof(T);   // elements per lane and row
    constexpr int LPR = DV / E;         // lanes per row
    constexpr int RPP = 256 / LPR;      // rows per pass of the workgroup
    constexpr int R = 4;                // passes: every lane has 2 R loads of 16 bytes in flight
    const int tid = threadIdx.x;
    const long row0 = (long)blockIdx.x * (R * RPP) + tid / LPR;
    const int c0 = (tid % LPR) * E;
    float ww[E];
    load_vec<E>(w + c0, ww);
    // a row's lanes are LPR consecutive lanes of one wavefront, aligned: whole rows drop out together
    float x[R][E], zz[R][E];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const long row = row0 + (long)r * RPP;
        if (row < rows) {
            load_vec<E>(o + row * DV + c0, x[r]);
            load_vec<E>(z + row * DV + c0, zz[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const long row = row0 + (long)r * RPP;
        if (row >= rows) break;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) ss += x[r][i] * x[r][i];
        ss = group_sum<LPR>(ss);
        const float inv = rsqrtf(ss * (1.f / DV) + eps);
#pragma unroll
        for (int i = 0; i < E; ++i) x[r][i] = x[r][i] * inv * (1.f + ww[i]) / (1.f + expf(-zz[r][i]));
        store_vec<E>(o + row * DV + c0, x[r]);
    }
}

template <typename T, int DV>
hipError_t launch_t(void* o, const void* z, const float* w, long rows, float eps, hipStream_t stream) {
    constexpr int RPB = 4 * (256 / (DV / (16 / (int)sizeof(T))));  // rows per workgroup
    if (rows <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((rows + RPB - 1) / RPB);
    hipLaunchKernelGGL((gated_norm_kernel<T, DV>), dim3(grid), dim3(256), 0, stream, static_cast<T*>(o),
                       static_cast<const T*>(z), w, rows, eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_norm(void* o, const void* z, const float* w, long rows, int dv, float eps, bool is_bf16,
                             hipStream_t stream) {
    switch (dv) {
        case 32: return is_bf16 ? launch_t<bf16, 32>(o, z, w, rows, eps, stream) : launch_t<float, 32>(o, z, w, rows, eps, stream);
        case 64: return is_bf16 ? launch_t<bf16, 64>(o, z, w, rows, eps, stream) : launch_t<float, 64>(o, z, w, rows, eps, stream);
        case 128: return is_bf16 ? launch_t<bf16, 128>(o, z, w, rows, eps, stream) : launch_t<float, 128>(o, z, w, rows, eps, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
