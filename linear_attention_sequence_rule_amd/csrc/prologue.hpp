// prologue.hpp -- per-token input transforms applied before the rule.
#pragma once

#include "common.hpp"

namespace gdn {

// Raw gates (page maplevalley.com.cn/news/1910399, section 2.1, 门控机制的精准控制): the decay
// g = -exp(A_log) * softplus(a + dt_bias) and the write strength beta = sigmoid(b).  softplus is
// evaluated without overflow as max(x, 0) + log1p(exp(-|x|)), with no threshold cut-off.
// neg_decay_rate = -exp(A_log) of the head; fp32 throughout.
__device__ __forceinline__ float raw_decay(float a, float neg_decay_rate, float dt_bias) {
    const float x = a + dt_bias;
    return neg_decay_rate * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))));
}
__device__ __forceinline__ float raw_beta(float b) { return 1.f / (1.f + expf(-b)); }

// Causal depthwise conv1d with 4 taps, then SiLU, for one channel at token t of a sequence
// starting at token bos (page maplevalley.com.cn/news/1910399, section 3.1, 卷积预处理; SiLU
// and the history before each sequence start are this library's reading):
//     x'_t = SiLU(sum_{j=0..3} w[j] x_{t-3+j}),
// with x_s for s < bos taken from hist (the three raw inputs before the sequence, oldest first,
// hstride elements apart, already offset to the channel) or zero when hist is null.
// x points at the packed tensor, `stride` elements between tokens, `off` the channel offset.
template <typename T>
__device__ __forceinline__ float conv_silu_at(const T* x, const float* w, long t, long bos, size_t stride,
                                              size_t off, const T* hist, size_t hstride) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const long s = t - 3 + j;
        if (s >= bos)
            acc += w[j] * load1(x + (size_t)s * stride + off);
        else if (hist)
            acc += w[j] * load1(hist + (size_t)(3 + s - bos) * hstride);
    }
    return acc / (1.f + expf(-acc));
}

}  // namespace gdn
