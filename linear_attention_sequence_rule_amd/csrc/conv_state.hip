// conv_state.hip -- the conv history left by a prefill call, for the call or decode step that
// continues the sequence (page maplevalley.com.cn/news/1910399, section 3.1, 卷积预处理: the causal
// conv over 4 tokens needs the three raw inputs before the token it starts at).
//
// After the chunk kernels have read conv_state as the history before each sequence start, this
// kernel replaces it, per sequence n and conv channel c, by the three raw inputs before the token
// after the sequence, oldest first:
//     new[j] = x[eos - 3 + j][c]     if eos - 3 + j >= bos,
//              old[j + len][c]       otherwise (len = eos - bos < 3: the history moves down).
// j runs upwards and j + len >= j, so old[j + len] has not been overwritten when it is read: the
// update is in place.  One lane per (sequence, channel); a copy of a few KB per sequence.
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void conv_state_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                         const T* __restrict__ v, const int32_t* __restrict__ cu,
                                                         T* __restrict__ hist, int N, int T_tot, int H, int dk,
                                                         int dv) {
    const long CC = (long)H * (2 * dk + dv);
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)N * CC) return;
    const int n = (int)(i / CC);
    const long c = i % CC;
    long bos, eos;
    if (cu) {
        bos = cu[n];
        eos = cu[n + 1];
    } else {
        bos = (long)n * (T_tot / N);
        eos = bos + T_tot / N;
    }
    // channel c of token t: q channels, then k, then v ([T, H, d] rows are H d consecutive channels)
    const T* src;
    long width, col;
    if (c < (long)H * dk) {
        src = q, width = (long)H * dk, col = c;
    } else if (c < 2L * H * dk) {
        src = k, width = (long)H * dk, col = c - (long)H * dk;
    } else {
        src = v, width = (long)H * dv, col = c - 2L * H * dk;
    }
    T* hn = hist + (size_t)n * 3 * CC + c;
    const long len = eos - bos;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const long t = eos - 3 + j;
        hn[j * CC] = t >= bos ? src[t * width + col] : hn[(j + len) * CC];
    }
}

template <typename T>
hipError_t launch_t(const ChunkArgs& a) {
    const long total = (long)a.N * a.H * (2 * a.dk + a.dv);
    const unsigned grid = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(conv_state_kernel<T>, dim3(grid), dim3(256), 0, a.stream, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.cu, static_cast<T*>(a.conv_state),
                       a.N, a.T_tot, a.H, a.dk, a.dv);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_state_update(const ChunkArgs& a) {
    return a.bf16 ? launch_t<bf16>(a) : launch_t<float>(a);
}

}  // namespace gdn
