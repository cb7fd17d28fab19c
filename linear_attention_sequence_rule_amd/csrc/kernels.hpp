// kernels.hpp -- internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct StepArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    float* state;
    void* o;
    int N, H, dk, dv;
    bool bf16;
    float scale;
    int l2norm;
    hipStream_t stream;
};

struct ChunkArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const float* s0;          // [N,H,dv,dk] or null
    const int32_t* cu;        // [N+1] or null (equal lengths T_tot / N)
    const float* conv_w;      // [H*(2dk+dv),4] or null
    void* o;
    float* sfin;              // [N,H,dv,dk] or null
    void* workspace;
    size_t workspace_bytes;
    int N, T_tot, H, dk, dv;
    bool bf16;
    float scale;
    int l2norm;
    hipStream_t stream;
};

hipError_t launch_step(const StepArgs& a);
hipError_t launch_chunk_f32(const ChunkArgs& a);
hipError_t launch_chunk_bf16(const ChunkArgs& a);
hipError_t launch_chunk_valu_bf16(const ChunkArgs& a);
size_t chunk_bf16_workspace(int N, int T_tot, int H, int dk, int dv, bool has_cu);

}  // namespace gdn
