// kernels.hpp -- internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct StepArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const float* gate_params; // [2,H] (A_log, dt_bias): g, beta hold the raw a, b; or null
    float* state;
    const float* conv_w;      // [2Hk*dk+H*dv,4] or null
    void* conv_state;         // [N,3,2Hk*dk+H*dv] dtype, with conv_w
    const void* out_gate;     // [N,H,dv] dtype: output gate z of the epilogue, or null
    const float* norm_weight; // [dv]: zero-centred RMSNorm scale offset (with out_gate)
    float norm_eps;
    void* o;
    int N, H, Hk, dk, dv;     // H value heads, Hk query/key heads (H a multiple of Hk)
    bool bf16;
    float scale;
    int l2norm;
    hipStream_t stream;
};

struct ChunkArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const float* gate_params; // [2,H] (A_log, dt_bias): g, beta hold the raw a, b; or null
    const float* s0;          // [N,H,dv,dk] or null
    const int32_t* cu;        // [N+1] or null (equal lengths T_tot / N)
    const float* conv_w;      // [2Hk*dk+H*dv,4] or null
    void* conv_state;         // [N,3,2Hk*dk+H*dv] dtype: history before each sequence, or null
    const void* out_gate;     // [T_tot,H,dv] dtype: output gate z of the epilogue, or null
    const float* norm_weight; // [dv]: zero-centred RMSNorm scale offset (with out_gate)
    float norm_eps;
    void* o;
    float* sfin;              // [N,H,dv,dk] or null
    void* workspace;
    size_t workspace_bytes;
    int N, T_tot, H, Hk, dk, dv;  // H value heads, Hk query/key heads (H a multiple of Hk)
    bool bf16;
    float scale;
    int l2norm;
    int segments;             // segments per sequence (1 = single pass), from plan_segments
    hipStream_t stream;
};

// Workspace of the segmented long-sequence path (P segments per sequence), byte offsets.
struct SegLayout {
    size_t off_E;     // fp32 [N*P, H, dv, dk]: B_p, the end states from a zero start
    size_t off_A;     // fp32 [N*P, H, dk, dk]: segment transitions A_p
    size_t off_negl;  // int32 [N*P, H]: 1 where A_p is below the decay bound
    size_t off_pre;   // [N*P, H] x kSegPrepBytes: prepared operands of each segment's first chunk
    size_t off_ein;   // fp32 [N*P, H, dv, dk]: entering states E_{p-1} that had to be chained
    size_t bytes;
};
// Bytes per (segment, head) of the first chunk's prepared operands that the first pass keeps for
// the rerun (two 64 x 72 bf16 tiles, 64 fp32, and the chunk's 1088 bytes of gates).
constexpr size_t kSegPrepBytes = 2 * 64 * 72 * 2 + 64 * 4 + 1088;
SegLayout seg_layout(int N, int H, int dk, int dv, int P);
// State rows per workgroup of the bf16 chunk kernel for a pass with `rows` state rows:
// 128 (wide workgroups) for d_k = 128 and rows a multiple of 128; else 64, or 32 for a 32-row
// state.
int chunk_rows_per_workgroup(int dk, int rows);
// Whether the chunk kernels apply the output epilogue themselves (bf16 with 128-row workgroups,
// which hold a head's whole output row); otherwise it runs as a separate pass over o.
bool chunk_fuses_epilogue(int dk, int dv, bool bf16);
// Segments per sequence for a bf16 call: `requested` if > 0, else enough to give every compute
// unit of the current device a workgroup when (sequence, head, row block) units alone do not
// (row blocks of chunk_rows_per_workgroup rows), and only for sequences of at least 16 chunks per
// segment.
int plan_segments(int N, int T_tot, int H, int dk, int dv, int requested);
// Facts of the current device, read from the runtime on its first use and kept (a call to
// hipDeviceGetAttribute per launch would cost host time on every prefill).
struct DeviceInfo {
    int cus = 0;      // compute units
    int lds_max = 0;  // bytes of LDS one workgroup may use
};
hipError_t current_device_info(DeviceInfo* out);
// hipFuncSetAttribute(fn, MaxDynamicSharedMemorySize, bytes) on the current device, once per
// (kernel, device, size): later calls return at once.
hipError_t set_dynamic_lds(const void* fn, int bytes);

hipError_t launch_step(const StepArgs& a);
hipError_t launch_chunk_f32(const ChunkArgs& a);
hipError_t launch_chunk_bf16(const ChunkArgs& a);
// Conv prologue of a bf16 prefill as a separate pass: q, k, v convolved (+ SiLU) into `out`
// (conv_prepass_bytes of workspace); conv_args = a with q, k, v pointing there and no conv.
size_t conv_prepass_bytes(int T_tot, int H, int Hk, int dk, int dv);
hipError_t launch_conv_prepass(const ChunkArgs& a, void* out, ChunkArgs& conv_args);
// conv_state <- the three raw inputs before the token after each sequence (in place, after the
// chunk kernels have read it as history).
hipError_t launch_conv_state_update(const ChunkArgs& a);
// o <- o * rsqrt(mean over dv of o^2 + eps) * (1 + w) * sigmoid(z), in place, rows of dv elements.
hipError_t launch_gated_norm(void* o, const void* z, const float* w, long rows, int dv, float eps, bool is_bf16,
                             hipStream_t stream);

}  // namespace gdn
