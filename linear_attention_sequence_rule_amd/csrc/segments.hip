// segments.hip -- planning, workspace layout and the combine step of the segmented long-sequence
// path.
//
// The chunked schedule carries the state serially from chunk to chunk (page pzsr.cn/news/750,
// section 1、为什么要设计为chunk的模式), so one long sequence is one serial chain per (head, block of
// state rows): too few workgroups to fill 256 compute units.  The state map of a stretch of tokens
// is affine in the state that enters it (the rule is linear in S): S_out = S_in A + B, with
// A = the product of the per-token transitions alpha_t (I - beta_t k_t k_t^T) and B = the end state
// from a zero start.  Cutting the sequence into P segments, every segment runs in parallel from a
// zero start (B_p) and as a transition (A_p); the serial part shrinks to the P-step combine below.
#include "kernels.hpp"

namespace gdn {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// E_0 = B_0, E_p = E_{p-1} A_p + B_p for p = 1 .. P-1, in place over the B slots (slot p ends as
// E_p, the state entering segment p + 1); final_state = E_{P-1}.  A transition marked negligible
// (its norm bound is below 2^-40) is skipped: E_p = B_p.  One workgroup per (sequence, head,
// block of 32 state rows); thread (column c, row group) keeps its rows of E in registers, and E_{p-1}
// is staged in LDS for the product.  fp32 throughout.
template <int DK>
__global__ __launch_bounds__(256) void seg_combine_kernel(float* E, const float* A, const int* negl, float* sfin,
                                                          int P, int H, int dv) {
    constexpr int RB = 32;           // state rows per workgroup
    constexpr int G = 256 / DK;      // row groups
    constexpr int RPG = RB / G;      // rows per thread
    __shared__ float prev[RB][DK];
    const int nv = dv / RB;
    const int rb = blockIdx.x % nv, nh = blockIdx.x / nv;
    const int n = nh / H, h = nh % H;
    const int tid = threadIdx.x, c = tid % DK, r0 = (tid / DK) * RPG;
    auto rows = [&](int p) { return E + (((size_t)(n * P + p) * H + h) * dv + rb * RB) * DK; };

    float cur[RPG];
    {
        const float* B0 = rows(0);
#pragma unroll
        for (int r = 0; r < RPG; ++r) cur[r] = B0[(r0 + r) * DK + c];
    }
    for (int p = 1; p < P; ++p) {
        float* Bp = rows(p);
        const size_t slot = (size_t)(n * P + p) * H + h;
        if (negl[slot]) {
#pragma unroll
            for (int r = 0; r < RPG; ++r) cur[r] = Bp[(r0 + r) * DK + c];
            continue;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < RPG; ++r) prev[r0 + r][c] = cur[r];
        __syncthreads();
        const float* Ap = A + slot * DK * DK;
        float acc[RPG];
#pragma unroll
        for (int r = 0; r < RPG; ++r) acc[r] = Bp[(r0 + r) * DK + c];
        for (int j = 0; j < DK; ++j) {
            const float a = Ap[(size_t)j * DK + c];
#pragma unroll
            for (int r = 0; r < RPG; ++r) acc[r] = fmaf(prev[r0 + r][j], a, acc[r]);
        }
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            cur[r] = acc[r];
            Bp[(r0 + r) * DK + c] = acc[r];
        }
    }
    if (sfin) {
        float* dst = sfin + (((size_t)n * H + h) * dv + rb * RB) * DK;
#pragma unroll
        for (int r = 0; r < RPG; ++r) dst[(r0 + r) * DK + c] = cur[r];
    }
}

}  // namespace

SegLayout seg_layout(int N, int H, int dk, int dv, int P) {
    SegLayout L;
    const size_t units = (size_t)N * P * H;
    L.off_E = 0;
    L.off_A = align256(units * dv * dk * 4);
    L.off_negl = L.off_A + align256(units * dk * dk * 4);
    L.bytes = L.off_negl + align256(units * 4);
    return L;
}

int plan_segments(int N, int T_tot, int H, int dk, int dv, int requested) {
    if (requested > 0) return requested;
    int cus = 256;  // MI355X; the current device's count when it can be read
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
        cus = v;
    const int rows = chunk_rows_per_workgroup(dk, dv);
    const long units = (long)N * H * (dv >= rows ? dv / rows : 1);  // workgroups of one pass
    if (units >= cus) return 1;
    const long chunks = ((long)T_tot / N + 63) / 64;
    long P = cus / units;
    if (P > chunks / 16) P = chunks / 16;
    if (P > 255) P = 255;
    return P < 1 ? 1 : (int)P;
}

hipError_t launch_seg_combine(float* E, const float* A, const int* negl, float* sfin, int N, int P, int H, int dk,
                              int dv, hipStream_t stream) {
    const int grid = N * H * (dv / 32);
    switch (dk) {
        case 32: hipLaunchKernelGGL(seg_combine_kernel<32>, dim3(grid), dim3(256), 0, stream, E, A, negl, sfin, P, H, dv); break;
        case 64: hipLaunchKernelGGL(seg_combine_kernel<64>, dim3(grid), dim3(256), 0, stream, E, A, negl, sfin, P, H, dv); break;
        case 128: hipLaunchKernelGGL(seg_combine_kernel<128>, dim3(grid), dim3(256), 0, stream, E, A, negl, sfin, P, H, dv); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gdn
