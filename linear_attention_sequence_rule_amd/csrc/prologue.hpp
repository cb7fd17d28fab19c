// prologue.hpp -- per-token input transforms applied before the rule.
#pragma once

#include "common.hpp"

namespace gdn {

// Causal depthwise conv1d with 4 taps, then SiLU, for one channel at token t of a sequence
// starting at token bos (page maplevalley.com.cn/news/1910399, section 3.1, 卷积预处理; SiLU
// and the zero history before each sequence start are this library's reading):
//     x'_t = SiLU(sum_{j=0..3} w[j] x_{t-3+j}),  x_s = 0 for s < bos.
// x points at the packed tensor, `stride` elements between tokens, `off` the channel offset.
template <typename T>
__device__ __forceinline__ float conv_silu_at(const T* x, const float* w, long t, long bos, size_t stride,
                                              size_t off) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const long s = t - 3 + j;
        if (s >= bos) acc += w[j] * load1(x + (size_t)s * stride + off);
    }
    return acc / (1.f + expf(-acc));
}

}  // namespace gdn
