// common.hpp -- device helpers shared by the gfx950 kernels of libgdn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr float kL2Eps = 1e-6f;  // eps of the q/k L2 normalisation, x * rsqrt(sum x^2 + eps)

// ---- element types ------------------------------------------------------------------------
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// float -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return uint16_t((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte accesses: data touched once per call.
__device__ __forceinline__ float4 nt_load4(const float* p) {
    f32x4 r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(r.x, r.y, r.z, r.w);
}
__device__ __forceinline__ void nt_store4(float* p, float4 v) {
    f32x4 r = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(p));
}

// Load 4 consecutive elements as float.
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const bf16* p) {
    uint2 r = *reinterpret_cast<const uint2*>(p);
    return make_float4(__builtin_bit_cast(float, r.x << 16), __builtin_bit_cast(float, r.x & 0xffff0000u),
                       __builtin_bit_cast(float, r.y << 16), __builtin_bit_cast(float, r.y & 0xffff0000u));
}
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const bf16* p) { return bf16_to_f32(p->bits); }
__device__ __forceinline__ void store1(float* p, float x) { *p = x; }
__device__ __forceinline__ void store1(bf16* p, float x) { p->bits = f32_to_bf16(x); }
// Store 4 consecutive elements (16-byte aligned for float, 8-byte for bf16).
__device__ __forceinline__ void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, float4 v) {
    const uint2 r = {(uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16),
                     (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16)};
    *reinterpret_cast<uint2*>(p) = r;
}

// ---- cross-lane sums over aligned lane groups (DPP / swizzle, no LDS traffic) ---------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// DPP controls: quad_perm xor1 = 0xB1, quad_perm xor2 = 0x4E, row_half_mirror = 0x141 (lane
// l <-> 7-l within 8), row_mirror = 0x140 (l <-> 15-l within 16).  After the quad sums every
// lane of a quad holds the same value, so a mirror adds exactly the neighbouring group.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(LANES == 4 || LANES == 8 || LANES == 16 || LANES == 32 || LANES == 64, "group");
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    if constexpr (LANES >= 8) x += dpp<0x141>(x);
    if constexpr (LANES >= 16) x += dpp<0x140>(x);
    if constexpr (LANES >= 32) {
        // ds_swizzle bit mode: and_mask 0x1f, or_mask 0, xor_mask 0x10 -> lane ^ 16 within 32
        x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
    }
    if constexpr (LANES >= 64) x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

}  // namespace gdn
