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
                                                         T* __restrict__ hist, int N, int T_tot, int H, int Hk,
                                                         int dk, int dv) {
    const long CC = 2L * Hk * dk + (long)H * dv;  // q, k channels of the Hk query/key heads, v of the H value heads
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
    // channel c of token t: q channels, then k, then v ([T, heads, d] rows are heads * d consecutive
    // channels); one load per source tensor
    const long Kc = (long)Hk * dk;
    T* hn = hist + (size_t)n * 3 * CC + c;
    const long len = eos - bos;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const long t = eos - 3 + j;
        T x;
        if (t < bos)
            x = hn[(j + len) * CC];
        else if (c < Kc)
            x = q[t * Kc + c];
        else if (c < 2 * Kc)
            x = k[t * Kc + c - Kc];
        else
            x = v[t * (long)H * dv + c - 2 * Kc];
        hn[j * CC] = x;
    }
}

template <typename T>
hipError_t launch_t(const ChunkArgs& a) {
    const long total = (long)a.N * (2L * a.Hk * a.dk + (long)a.H * a.dv);
    const unsigned grid = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(conv_state_kernel<T>, dim3(grid), dim3(256), 0, a.stream, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.cu, static_cast<T*>(a.conv_state),
                       a.N, a.T_tot, a.H, a.Hk, a.dk, a.dv);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_state_update(const ChunkArgs& a) {
    return a.bf16 ? launch_t<bf16>(a) : launch_t<float>(a);
}

}  // namespace gdn
