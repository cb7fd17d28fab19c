/*
 * gdn.h -- C ABI of libgdn.so: the Gated DeltaNet gated delta rule on AMD Instinct MI355X
 * (gfx950), chunked prefill and single-token recurrent decode.
 *
 * The operation (page "Gated DeltaNet 架构详解与 Qwen 3.5 的联系", section 6; page
 * "Gated DeltaNet与推理脚手架：两个模糊边界的发现", section 发现一, the Gated DeltaNet update
 * rule): for every sequence n and head h independently, with a state S in R^{dv x dk},
 *
 *     S_t = S_{t-1} * alpha_t * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,    o_t = scale * S_t q_t
 *
 * with alpha_t = exp(g_t).  The equivalent form every kernel evaluates is
 *     u_t = beta_t (v_t - alpha_t S_{t-1} k_t),   S_t = alpha_t S_{t-1} + u_t k_t^T.
 * The page maplevalley.com.cn/news/1910399, section 2.1 (门控机制的精准控制), gives the gate
 * parameterisation g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b).  The caller passes
 * either g and beta, or (with gate_params) the raw a and b, which the kernels turn into g and beta
 * as they load them ("Raw gates" below).  With GDN_QK_L2NORM, q and k are replaced by
 * x * rsqrt(sum(x^2) + 1e-6) over the key dimension, per (token, head), inside the kernels.
 *
 * Raw gates (both entry points).  gate_params = NULL: g and beta are the log decay and the write
 * strength.  gate_params = [2, H] fp32, row 0 = A_log, row 1 = dt_bias: g holds the raw a and beta
 * the raw b (same shapes, fp32), and every use computes
 *     g = -exp(A_log[h]) * softplus(a + dt_bias[h]),   beta = 1 / (1 + exp(-b))
 * in fp32, softplus(x) = max(x, 0) + log1p(exp(-|x|)) (no threshold).  The inputs are not modified.
 *
 * Heads (both entry points).  H value heads carry the states, gates, values and outputs; Hk query/key
 * heads carry q and k, with H a multiple of Hk: value head h reads query/key head h / (H / Hk), so
 * each query/key head serves H / Hk consecutive value heads (Hk = H: one query/key head per value
 * head).  The model configuration on page "Gated DeltaNet 架构详解与 Qwen 3.5 的联系", section 6,
 * counts the two separately; the grouping order is this library's reading.
 *
 * Conv state (both entry points).  conv_state [N, 3, C] dtype, C = 2*Hk*dk + H*dv, holds, per sequence, the
 * three raw inputs (before conv) that precede its next token, oldest first, in the channel order of
 * conv_w.  It makes the conv prologue continue across calls: a prefill reads it as the history
 * before each sequence start instead of zeros, and both entry points overwrite it in place with the
 * three raw inputs before the token that would come next (for a sequence shorter than three tokens
 * the newest entries of the old state move down; a zero-length sequence keeps it).  The values are
 * stored in the input dtype exactly, so a prefill split at any point and resumed, or followed by
 * decode steps, sees the same conv inputs as one call over the whole sequence.
 *
 * Output epilogue (both entry points).  out_gate z [rows of o, dv] dtype and norm_weight w [dv]
 * fp32, both NULL or both given: then every (token, head) row of o leaves as
 *     o * rsqrt(mean over dv of o^2 + norm_eps) * (1 + w) * sigmoid(z)
 * -- a zero-centred RMSNorm (page maplevalley.com.cn/news/1910399, section 3.2: the learnable scale
 * is stored as an offset from 1, initialised to zero; section 4.2 suggests an eps of 1e-3 in bf16)
 * followed by a sigmoid output gate (page "GDN融合门控注意力的动态资源分配机制，AI智能体调动实战演练",
 * section 2).  The decode step applies it inside its kernel, and so does the bf16 prefill for
 * dk = 128 with dv a multiple of 128 (one workgroup holds a head's whole output row); other
 * prefill shapes run it as one more pass over o after the rule.
 *
 * Conventions shared by every entry point
 *  - All pointers are DEVICE pointers to contiguous, row-major memory, 16-byte aligned, except
 *    where stated.  Nothing is copied to or from the host.
 *  - Ownership: the caller allocates and frees every buffer.  The library allocates nothing,
 *    frees nothing, launches only on `hip_stream` (a hipStream_t; NULL = the null stream) and
 *    never synchronises.  Its only mutable state is the static scratch of gdn_chunk_fwd_noalloc
 *    (and the device addresses of it).  Buffers must stay alive until the stream's work has
 *    completed.  Calls are asynchronous: a returned GDN_OK means the
 *    arguments were valid and the launches were enqueued without a launch error.
 *  - Errors: every argument check runs on the host before any HIP call; on an invalid argument
 *    nothing is launched and nothing is written.  No C++ exception crosses this ABI.  Device-side
 *    contents (cu_seqlens values, NaN/Inf in data) are not checked: inconsistent cu_seqlens is
 *    undefined behaviour; a NaN in one (sequence, head) never reaches another.
 *  - Determinism: no atomics; results are bitwise reproducible run to run on the same device.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define GDN_OK 0
#define GDN_ERR_INVALID_ARG 1  /* null pointer where one is required, negative size, bad alignment */
#define GDN_ERR_UNSUPPORTED 2  /* shape/dtype/chunk this build does not implement                  */
#define GDN_ERR_WORKSPACE 3    /* workspace missing or smaller than *workspace_bytes               */
#define GDN_ERR_HIP 4          /* a HIP launch reported an error (hipGetLastError after launch)    */
#define GDN_ERR_SCRATCH 5      /* gdn_chunk_fwd_noalloc: the call needs more scratch than the
                                  library's static buffer holds (GDN_NOALLOC_SCRATCH_BYTES)         */

/* Element types of q, k, v and o.  g, beta and every state are always fp32. */
#define GDN_F32 0
#define GDN_BF16 1

/* flags */
#define GDN_QK_L2NORM 1u       /* L2-normalise q and k per (token, head) over dk, eps = 1e-6 */
/* Segments per sequence for gdn_chunk_fwd (bits 8..15; 0 = chosen automatically).  See
 * "Long sequences" under gdn_chunk_fwd.  Not accepted by gdn_recurrent_step. */
#define GDN_SEGMENTS(n) ((((unsigned)(n)) & 0xFFu) << 8)
/* bf16 prefill with conv_w: run the conv prologue inside the chunk kernel instead of as a separate
 * pass into the workspace (see "Workspace" under gdn_chunk_fwd).  For dk = 128 with dv a multiple
 * of 128 the conv always runs inside the chunk kernel.  No effect otherwise. */
#define GDN_CONV_FUSED (1u << 16)

/*
 * gdn_chunk_fwd -- chunked prefill over packed variable-length sequences.
 *
 * Defines: the call chunk_gated_delta_rule(query, key, value, g, beta, initial_state) ->
 * (core_attn_out, last_state) on page maplevalley.com.cn/news/1910399, section 3.1
 * (记忆系统的工程优化), computed by chunks: tokens inside a chunk in parallel, the state carried
 * serially from chunk to chunk (page pzsr.cn/news/750, section 1、为什么要设计为chunk的模式).
 * The chunk size changes only the rounding, never the result in exact arithmetic.
 *
 * Arguments (T_tot = total tokens of all sequences, packed back to back):
 *  q, k        [T_tot, Hk, dk] dtype   raw queries / keys (before conv, before L2 norm)
 *  v           [T_tot, H, dv]  dtype   raw values
 *  g           [T_tot, H]      fp32    log decay, alpha = exp(g); g <= 0 expected (any finite g
 *                                      works); with gate_params: the raw a
 *  beta        [T_tot, H]      fp32    write strength; with gate_params: the raw b
 *  gate_params [2, H]          fp32    NULL, or A_log and dt_bias ("Raw gates" above)
 *  initial_state [N, H, dv, dk] fp32   S_0 per (sequence, head), S as in o = S q; NULL = zeros
 *  cu_seqlens  [N + 1]         int32   sequence offsets into the packed token axis, non-decreasing,
 *                                      cu_seqlens[0] = 0, cu_seqlens[N] = T_tot; NULL = N equal
 *                                      sequences of T_tot / N tokens (then N must divide T_tot).
 *                                      Zero-length sequences are allowed: final = initial, no o.
 *  conv_w      [C, 4] fp32             NULL, or the depthwise causal conv1d (4 taps) applied per
 *                                      channel to q, k and v before SiLU and the L2 norm (page
 *                                      maplevalley.com.cn/news/1910399, section 3.1, 卷积预处理).
 *                                      C = 2*Hk*dk + H*dv: channel c < Hk*dk is q channel
 *                                      (hk*dk + i), the next Hk*dk are k channels, the last H*dv
 *                                      are v channels (h*dv + i).  Tap j multiplies
 *                                      token t-3+j (tap 3 = current token); history before a
 *                                      sequence start is conv_state, else zero; no bias.
 *  conv_state  [N, 3, C] dtype         NULL, or the conv history, read and overwritten in
 *                                      place ("Conv state" above); requires conv_w.  Must not
 *                                      overlap any other buffer.
 *  out_gate    [T_tot, H, dv]  dtype   NULL, or z of the output epilogue (above); with norm_weight
 *  norm_weight [dv]            fp32    NULL, or w of the output epilogue; with out_gate.  When
 *                                      T_tot = 0 either may be NULL alone (nothing to gate) and
 *                                      neither is read.
 *  o           [T_tot, H, dv]  dtype   output; must not alias any input
 *  final_state [N, H, dv, dk] fp32     last state per (sequence, head), or NULL = not written.
 *                                      May alias initial_state exactly (same pointer).
 *  workspace, workspace_bytes          device scratch: the long-sequence path (below) and, for a
 *                                      bf16 call with conv_w (unless GDN_CONV_FUSED, or dk = 128
 *                                      with dv a multiple of 128), the convolved q, k, v
 *                                      (T_tot * (2*Hk*dk + H*dv) bf16): the conv prologue then
 *                                      runs as one streaming pass before the chunk kernel.  If
 *                                      *workspace_bytes is smaller than the size this call needs,
 *                                      the call sets *workspace_bytes to that size and returns
 *                                      GDN_ERR_WORKSPACE without launching (a NULL workspace with
 *                                      *workspace_bytes = 0 is the size query).  workspace_bytes
 *                                      may be NULL only when the call needs no workspace.  The
 *                                      workspace must not overlap any other buffer; its contents
 *                                      on entry are ignored and on return are unspecified.
 *  N, T_tot, H, Hk, dk, dv             sizes; dk, dv in {32, 64, 128}; N >= 1, T_tot >= 0, H >= 1,
 *                                      1 <= Hk, H a multiple of Hk ("Heads" above)
 *  dtype       GDN_F32 or GDN_BF16     (fp32 path: exact fp32 arithmetic throughout; bf16 path:
 *                                      bf16 MFMA operands, fp32 accumulation, fp32 state)
 *  chunk       64                      chunk length; other values -> GDN_ERR_UNSUPPORTED
 *  scale       output scale (1.0 = o_t = S_t q_t), applied before the epilogue
 *  norm_eps    eps of the epilogue's RMSNorm (finite, >= 0; ignored without out_gate)
 *  flags       GDN_QK_L2NORM, optionally | GDN_SEGMENTS(n) | GDN_CONV_FUSED
 *  hip_stream  hipStream_t to launch on
 *
 * Long sequences (bf16 path).  Each sequence is cut into P segments of whole chunks
 * that run in parallel; the exact affine map of a segment, S_out = S_in A_p + B_p, joins them:
 * the segments run from a zero state (B_p and o), then as transitions (A_p: identity in, zero
 * values), and a last pass reruns each segment from its true entering state E_{p-1}
 * (E_0 = B_0, E_p = E_{p-1} A_p + B_p, formed by that pass itself), overwriting o.  A transition
 * and a rerun stop once the bound exp(sum of g since the segment start) on the segment's
 * transition is <= 2^-40: past that point the state entering the segment has no effect above that
 * factor (the bound holds with GDN_QK_L2NORM and 0 <= beta <= 2; otherwise nothing stops early
 * and every pass runs the whole segment).  A transition whose bound over the whole segment is
 * already below 2^-40 is not formed (E_p = B_p), and a rerun whose first chunk reaches the bound
 * reuses that chunk's prepared operands from the first pass.  P = 1 is the plain single pass.
 * With GDN_SEGMENTS(0), P is chosen so that (N * P * H * dv / R) workgroups cover the current
 * device's compute units (R = 128 state rows per workgroup for dk = 128 and dv a multiple of 128,
 * else 64, or 32 for dv = 32), with at least 16 chunks per segment.
 */
int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  const float* gate_params, const float* initial_state, const int32_t* cu_seqlens,
                  const float* conv_w, void* conv_state, const void* out_gate,
                  const float* norm_weight, void* o, float* final_state, void* workspace,
                  size_t* workspace_bytes, int N, int T_tot, int H, int Hk, int dk, int dv,
                  int dtype, int chunk, float scale, float norm_eps, unsigned flags,
                  void* hip_stream);

/*
 * gdn_chunk_fwd_noalloc -- gdn_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It calls no allocating routine: where gdn_chunk_fwd needs a workspace
 * (gdn_chunk_workspace_size > 0), this entry point uses a static device buffer of the library,
 * GDN_NOALLOC_SCRATCH_BYTES on every device it runs on, held until the process ends.
 *
 *  Arguments, results and errors: as gdn_chunk_fwd, without workspace and workspace_bytes; a call
 *  whose workspace would exceed GDN_NOALLOC_SCRATCH_BYTES returns GDN_ERR_SCRATCH and launches
 *  nothing (the automatic segment plans of the long-sequence path stay below it on a 256-CU
 *  device; the separate conv pass of shapes other than dk = 128 with dv a multiple of 128 needs
 *  T_tot * (2*Hk*dk + H*dv) * 2 bytes, so long inputs there need GDN_CONV_FUSED or gdn_chunk_fwd).
 *  The buffer's contents never need clearing (each call writes every part it reads).
 *  Concurrency: all calls on one device share its buffer; calls that overlap in time on one device
 *  (two streams, or two host threads) race on it and give undefined results.  Calls on different
 *  devices do not interact.
 *  The first call on a device resolves the buffer's device address (a host-side runtime query, no
 *  allocation); a failure there returns GDN_ERR_HIP.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const float* gate_params, const float* initial_state, const int32_t* cu_seqlens,
                          const float* conv_w, void* conv_state, const void* out_gate,
                          const float* norm_weight, void* o, float* final_state, int N, int T_tot, int H,
                          int Hk, int dk, int dv, int dtype, int chunk, float scale, float norm_eps,
                          unsigned flags, void* hip_stream);

/*
 * gdn_chunk_workspace_size -- the workspace gdn_chunk_fwd needs for these sizes, flags and
 * (nonzero = present) cu_seqlens / conv_w (0 bytes when the call runs as a single pass).  Host
 * function; with automatic segments it reads the compute-unit count of the current device (256
 * when no device can be queried), exactly as gdn_chunk_fwd does.  Returns GDN_OK and sets *bytes,
 * or the error code gdn_chunk_fwd would return for these arguments.
 */
int gdn_chunk_workspace_size(int N, int T_tot, int H, int Hk, int dk, int dv, int dtype, int chunk,
                             int has_cu_seqlens, int has_conv, unsigned flags, size_t* bytes);

/*
 * gdn_recurrent_step -- one decode token per sequence, state updated in place.
 *
 * Defines: the incremental (recurrent) update with a fixed-size state (page pzsr.cn/news/750,
 * section a、增量更新: decay the whole state by alpha first, then erase and write along the
 * current key with strength beta), which is the rule above with T = 1:
 *     u = beta (v - alpha S k),  S <- alpha S + u k^T,  o = scale * S q.
 *
 *  q, k   [N, Hk, dk] dtype;  v [N, H, dv] dtype;  g, beta [N, H] fp32 (raw a, b with
 *         gate_params)
 *  gate_params [2, H] fp32 or NULL, as for gdn_chunk_fwd
 *  state  [N, H, dv, dk] fp32, read and overwritten in place
 *  conv_w [C, 4] fp32 and conv_state [N, 3, C] dtype (C = 2*Hk*dk + H*dv): both NULL, or both
 *         given: then q, k and v are the raw inputs of the conv prologue, conv + SiLU (and the L2
 *         norm) run on them with the three previous raw inputs from conv_state, and conv_state is
 *         shifted in place by one token (the oldest dropped, this token's raw inputs appended)
 *  out_gate [N, H, dv] dtype and norm_weight [dv] fp32: both NULL, or the output epilogue (above),
 *         applied inside the step kernel
 *  o      [N, H, dv] dtype, must not alias any input
 *  N, H, Hk >= 1 (N = 0 is a no-op returning GDN_OK), H a multiple of Hk; dk, dv in {32, 64, 128}
 *  dtype, scale, norm_eps, flags, hip_stream as for gdn_chunk_fwd
 */
int gdn_recurrent_step(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* gate_params, float* state,
                       const float* conv_w, void* conv_state, const void* out_gate,
                       const float* norm_weight, void* o, int N, int H, int Hk, int dk, int dv,
                       int dtype, float scale, float norm_eps, unsigned flags, void* hip_stream);

/* gdn_status_string -- static, human-readable name of a status code (never NULL). */
const char* gdn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
