// api.hip -- the C ABI of libgdn.so (declared in include/gdn.h): host-side argument checks, then
// dispatch to the gfx950 kernels on the caller's stream.  No allocation and no synchronisation;
// every check runs before the first HIP call.  The only state the library keeps is the static
// scratch of gdn_chunk_fwd_noalloc and the per-device addresses of it.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/gdn.h"
#include "kernels.hpp"

// Scratch of gdn_chunk_fwd_noalloc: device memory the library holds itself, for callers that
// cannot allocate.  Every device the library runs on keeps one copy until the process ends.  In
// host code the name stands for a host-side shadow, not the device address: the address comes
// from hipGetSymbolAddress, once per device (scratch_for_current_device).
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

bool dim_ok(int d) { return d == 32 || d == 64 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + na) and [b, b + nb) overlap (byte ranges); null or empty never overlaps.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

constexpr unsigned kSegMask = 0xFFu << 8;
constexpr unsigned kConvFused = 1u << 16;  // GDN_CONV_FUSED

int check_common(int H, int dk, int dv, int dtype, float scale, unsigned flags) {
    if (H < 1) return GDN_ERR_INVALID_ARG;
    if (flags & ~(GDN_QK_L2NORM | kSegMask | kConvFused)) return GDN_ERR_INVALID_ARG;
    if (!isfinite(scale)) return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

// Segments per sequence for this call (1 = single pass).  A request for more than one segment is
// honoured on the bf16 path only.
int segments_for(int N, int T_tot, int H, int dk, int dv, int dtype, unsigned flags, int* P) {
    const int req = (int)((flags & kSegMask) >> 8);
    if (dtype != GDN_BF16) {
        if (req > 1) return GDN_ERR_UNSUPPORTED;
        *P = 1;
        return GDN_OK;
    }
    *P = gdn::plan_segments(N, T_tot, H, dk, dv, req);
    return GDN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Segment buffers first (the long-sequence path), then the convolved q, k, v of the conv pass.
// The bf16 path convolves inside the chunk kernel where its 128-row workgroups run (d_k = 128, d_v
// a multiple of 128) or when GDN_CONV_FUSED asks for it; otherwise a separate streaming pass writes
// the convolved inputs to the workspace first.
bool conv_pass(bool has_conv, int dtype, unsigned flags, int dk, int dv) {
    return has_conv && dtype == GDN_BF16 && !(flags & kConvFused) && gdn::chunk_rows_per_workgroup(dk, dv) != 128;
}
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch array, resolved with that device current
// the first time a call runs on it.
int scratch_for_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GDN_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GDN_OK;
}

size_t seg_bytes(int N, int H, int dk, int dv, int P) { return P > 1 ? align256(gdn::seg_layout(N, H, dk, dv, P).bytes) : 0; }
size_t workspace_for(int N, int T_tot, int H, int Hk, int dk, int dv, int P, bool conv) {
    return seg_bytes(N, H, dk, dv, P) + (conv ? gdn::conv_prepass_bytes(T_tot, H, Hk, dk, dv) : 0);
}

}  // namespace

extern "C" {

const char* gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
        case GDN_ERR_HIP: return "GDN_ERR_HIP";
        case GDN_ERR_SCRATCH: return "GDN_ERR_SCRATCH";
    }
    return "GDN_ERR_UNKNOWN";
}

int gdn_chunk_workspace_size(int N, int T_tot, int H, int Hk, int dk, int dv, int dtype, int chunk,
                             int has_cu_seqlens, int has_conv, unsigned flags, size_t* bytes) {
    if (!bytes) return GDN_ERR_INVALID_ARG;
    if (N < 1 || T_tot < 0) return GDN_ERR_INVALID_ARG;
    if (Hk < 1 || H < 1 || H % Hk != 0) return GDN_ERR_INVALID_ARG;
    int st = check_common(H, dk, dv, dtype, 1.0f, flags);
    if (st != GDN_OK) return st;
    if (chunk != 64) return GDN_ERR_UNSUPPORTED;
    if (!has_cu_seqlens && T_tot % N != 0) return GDN_ERR_INVALID_ARG;
    int P = 1;
    st = segments_for(N, T_tot, H, dk, dv, dtype, flags, &P);
    if (st != GDN_OK) return st;
    *bytes = workspace_for(N, T_tot, H, Hk, dk, dv, P, conv_pass(has_conv != 0, dtype, flags, dk, dv));
    return GDN_OK;
}

}  // extern "C"

namespace {

// gdn_chunk_fwd with the caller's workspace, or (own_scratch) with the library's static scratch.
int chunk_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
              const float* gate_params, const float* initial_state, const int32_t* cu_seqlens, const float* conv_w,
              void* conv_state, const void* out_gate, const float* norm_weight, void* o, float* final_state,
              void* workspace, size_t* workspace_bytes, bool own_scratch, int N, int T_tot, int H, int Hk, int dk,
              int dv, int dtype, int chunk, float scale, float norm_eps, unsigned flags, void* hip_stream) {
    if (N < 1 || T_tot < 0) return GDN_ERR_INVALID_ARG;
    if (Hk < 1 || H < 1 || H % Hk != 0) return GDN_ERR_INVALID_ARG;
    int st = check_common(H, dk, dv, dtype, scale, flags);
    if (st != GDN_OK) return st;
    if (chunk != 64) return GDN_ERR_UNSUPPORTED;
    if (!cu_seqlens && T_tot % N != 0) return GDN_ERR_INVALID_ARG;
    if (T_tot > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_INVALID_ARG;
    if (conv_state && !conv_w) return GDN_ERR_INVALID_ARG;
    // with no token there is no output to gate: out_gate (an empty tensor) may then be NULL alone
    if (T_tot > 0 && (out_gate == nullptr) != (norm_weight == nullptr)) return GDN_ERR_INVALID_ARG;
    if (out_gate && !(isfinite(norm_eps) && norm_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
    if (T_tot == 0) out_gate = norm_weight = nullptr;
    const void* ptrs[] = {q, k, v, g, beta, gate_params, initial_state, cu_seqlens, conv_w, conv_state, out_gate,
                          norm_weight, o, final_state};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;

    const size_t es = dtype == GDN_BF16 ? 2 : 4;
    const size_t cc = (size_t)2 * Hk * dk + (size_t)H * dv;  // conv channels per token
    const size_t tq = (size_t)T_tot * Hk * dk * es, tv = (size_t)T_tot * H * dv * es;
    const size_t tg = (size_t)T_tot * H * 4, ts = (size_t)N * H * dv * dk * 4;
    const size_t tcu = cu_seqlens ? (size_t)(N + 1) * 4 : 0, tcw = conv_w ? cc * 16 : 0;
    const size_t tgp = gate_params ? (size_t)H * 8 : 0;
    const size_t tcs = conv_state ? (size_t)N * 3 * cc * es : 0;
    const size_t tz = out_gate ? tv : 0, tw = norm_weight ? (size_t)dv * 4 : 0;
    // o must not overlap any input; final_state may equal initial_state exactly but not overlap otherwise.
    if (overlaps(o, tv, out_gate, tz) || overlaps(o, tv, norm_weight, tw) ||
        overlaps(final_state, ts, out_gate, tz) || overlaps(final_state, ts, norm_weight, tw) ||
        overlaps(conv_state, tcs, out_gate, tz) || overlaps(conv_state, tcs, norm_weight, tw))
        return GDN_ERR_INVALID_ARG;
    if (overlaps(o, tv, q, tq) || overlaps(o, tv, k, tq) || overlaps(o, tv, v, tv) || overlaps(o, tv, g, tg) ||
        overlaps(o, tv, beta, tg) || overlaps(o, tv, initial_state, ts) || overlaps(o, tv, final_state, ts) ||
        overlaps(o, tv, cu_seqlens, tcu) || overlaps(o, tv, conv_w, tcw) || overlaps(o, tv, gate_params, tgp) ||
        overlaps(o, tv, conv_state, tcs))
        return GDN_ERR_INVALID_ARG;
    if (final_state && final_state != initial_state &&
        (overlaps(final_state, ts, initial_state, ts) || overlaps(final_state, ts, q, tq) ||
         overlaps(final_state, ts, k, tq) || overlaps(final_state, ts, v, tv) || overlaps(final_state, ts, g, tg) ||
         overlaps(final_state, ts, beta, tg) || overlaps(final_state, ts, cu_seqlens, tcu) ||
         overlaps(final_state, ts, conv_w, tcw) || overlaps(final_state, ts, gate_params, tgp)))
        return GDN_ERR_INVALID_ARG;
    // conv_state is written in place: it may share memory with nothing else.
    if (overlaps(conv_state, tcs, q, tq) || overlaps(conv_state, tcs, k, tq) || overlaps(conv_state, tcs, v, tv) ||
        overlaps(conv_state, tcs, g, tg) || overlaps(conv_state, tcs, beta, tg) ||
        overlaps(conv_state, tcs, gate_params, tgp) || overlaps(conv_state, tcs, initial_state, ts) ||
        overlaps(conv_state, tcs, final_state, ts) || overlaps(conv_state, tcs, cu_seqlens, tcu) ||
        overlaps(conv_state, tcs, conv_w, tcw))
        return GDN_ERR_INVALID_ARG;

    int P = 1;
    st = segments_for(N, T_tot, H, dk, dv, dtype, flags, &P);
    if (st != GDN_OK) return st;
    const bool cpass = conv_pass(conv_w != nullptr, dtype, flags, dk, dv);
    const size_t need = workspace_for(N, T_tot, H, Hk, dk, dv, P, cpass);
    size_t have = workspace_bytes ? *workspace_bytes : 0;
    if (own_scratch) {
        // every part of the workspace is written before it is read: nothing to clear
        if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH;
        workspace = nullptr;
        have = 0;
        if (need > 0) {
            st = scratch_for_current_device(&workspace);
            if (st != GDN_OK) return st;
            have = (size_t)GDN_NOALLOC_SCRATCH_BYTES;
        }
    } else if (need > 0) {
        if (!workspace_bytes) return GDN_ERR_INVALID_ARG;
        if (!workspace || *workspace_bytes < need) {
            *workspace_bytes = need;
            return GDN_ERR_WORKSPACE;
        }
        if (!aligned16(workspace)) return GDN_ERR_INVALID_ARG;
        const size_t twk = *workspace_bytes;
        if (overlaps(workspace, twk, q, tq) || overlaps(workspace, twk, k, tq) || overlaps(workspace, twk, v, tv) ||
            overlaps(workspace, twk, g, tg) || overlaps(workspace, twk, beta, tg) ||
            overlaps(workspace, twk, initial_state, ts) || overlaps(workspace, twk, final_state, ts) ||
            overlaps(workspace, twk, o, tv) || overlaps(workspace, twk, cu_seqlens, tcu) ||
            overlaps(workspace, twk, conv_w, tcw) || overlaps(workspace, twk, gate_params, tgp) ||
            overlaps(workspace, twk, conv_state, tcs) || overlaps(workspace, twk, out_gate, tz) ||
            overlaps(workspace, twk, norm_weight, tw))
            return GDN_ERR_INVALID_ARG;
    }

    gdn::ChunkArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.gate_params = gate_params;
    a.s0 = initial_state;
    a.cu = cu_seqlens;
    a.conv_w = conv_w;
    a.conv_state = conv_state;
    a.out_gate = out_gate;
    a.norm_weight = norm_weight;
    a.norm_eps = norm_eps;
    a.o = o;
    a.sfin = final_state;
    a.workspace = workspace;
    a.workspace_bytes = have;
    a.N = N;
    a.T_tot = T_tot;
    a.H = H;
    a.Hk = Hk;
    a.dk = dk;
    a.dv = dv;
    a.bf16 = dtype == GDN_BF16;
    a.scale = scale;
    a.l2norm = (flags & GDN_QK_L2NORM) ? 1 : 0;
    a.segments = P;
    a.stream = static_cast<hipStream_t>(hip_stream);
    hipError_t e;
    if (cpass) {
        gdn::ChunkArgs c;
        e = gdn::launch_conv_prepass(a, static_cast<unsigned char*>(workspace) + seg_bytes(N, H, dk, dv, P), c);
        if (e == hipSuccess) e = gdn::launch_chunk_bf16(c);
    } else {
        e = a.bf16 ? gdn::launch_chunk_bf16(a) : gdn::launch_chunk_f32(a);
    }
    if (e == hipSuccess && conv_state) e = gdn::launch_conv_state_update(a);
    if (e == hipSuccess && out_gate && !gdn::chunk_fuses_epilogue(dk, dv, a.bf16))
        e = gdn::launch_gated_norm(o, a.out_gate, a.norm_weight, (long)T_tot * H, dv, a.norm_eps, a.bf16, a.stream);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace

extern "C" {

int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  const float* gate_params, const float* initial_state, const int32_t* cu_seqlens,
                  const float* conv_w, void* conv_state, const void* out_gate, const float* norm_weight, void* o,
                  float* final_state, void* workspace, size_t* workspace_bytes, int N, int T_tot, int H, int Hk,
                  int dk, int dv, int dtype, int chunk, float scale, float norm_eps, unsigned flags,
                  void* hip_stream) {
    return chunk_fwd(q, k, v, g, beta, gate_params, initial_state, cu_seqlens, conv_w, conv_state, out_gate,
                     norm_weight, o, final_state, workspace, workspace_bytes, false, N, T_tot, H, Hk, dk, dv, dtype,
                     chunk, scale, norm_eps, flags, hip_stream);
}

int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const float* gate_params, const float* initial_state, const int32_t* cu_seqlens,
                          const float* conv_w, void* conv_state, const void* out_gate, const float* norm_weight,
                          void* o, float* final_state, int N, int T_tot, int H, int Hk, int dk, int dv, int dtype,
                          int chunk, float scale, float norm_eps, unsigned flags, void* hip_stream) {
    return chunk_fwd(q, k, v, g, beta, gate_params, initial_state, cu_seqlens, conv_w, conv_state, out_gate,
                     norm_weight, o, final_state, nullptr, nullptr, true, N, T_tot, H, Hk, dk, dv, dtype, chunk, scale,
                     norm_eps, flags, hip_stream);
}

int gdn_recurrent_step(const void* q, const void* k, const void* v, const float* g, const float* beta,
                       const float* gate_params, float* state, const float* conv_w, void* conv_state,
                       const void* out_gate, const float* norm_weight, void* o, int N, int H, int Hk, int dk, int dv,
                       int dtype, float scale, float norm_eps, unsigned flags, void* hip_stream) {
    if (N < 0 || (flags & kSegMask)) return GDN_ERR_INVALID_ARG;
    if (Hk < 1 || H < 1 || H % Hk != 0) return GDN_ERR_INVALID_ARG;
    int st = check_common(H, dk, dv, dtype, scale, flags);
    if (st != GDN_OK) return st;
    if (N == 0) return GDN_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return GDN_ERR_INVALID_ARG;
    if ((conv_w == nullptr) != (conv_state == nullptr)) return GDN_ERR_INVALID_ARG;
    if ((out_gate == nullptr) != (norm_weight == nullptr)) return GDN_ERR_INVALID_ARG;
    if (out_gate && !(isfinite(norm_eps) && norm_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, g, beta, gate_params, state, conv_w, conv_state, out_gate, norm_weight, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;
    const size_t es = dtype == GDN_BF16 ? 2 : 4;
    const size_t cc = (size_t)2 * Hk * dk + (size_t)H * dv;  // conv channels per token
    const size_t tq = (size_t)N * Hk * dk * es, tv = (size_t)N * H * dv * es, tg = (size_t)N * H * 4;
    const size_t ts = (size_t)N * H * dv * dk * 4, tgp = gate_params ? (size_t)H * 8 : 0;
    const size_t tcw = conv_w ? cc * 16 : 0;
    const size_t tcs = conv_state ? (size_t)N * 3 * cc * es : 0;
    const size_t tz = out_gate ? tv : 0, tnw = norm_weight ? (size_t)dv * 4 : 0;
    // o, state and conv_state are written: none of them may share memory with another buffer.
    const void* bufs[] = {q, k, v, g, beta, gate_params, conv_w, out_gate, norm_weight, state, conv_state, o};
    const size_t lens[] = {tq, tq, tv, tg, tg, tgp, tcw, tz, tnw, ts, tcs, tv};
    constexpr int nb = 12, first_written = 9;
    for (int w = first_written; w < nb; ++w)
        for (int i = 0; i < nb; ++i)
            if (i != w && overlaps(bufs[w], lens[w], bufs[i], lens[i])) return GDN_ERR_INVALID_ARG;
    gdn::StepArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.gate_params = gate_params;
    a.state = state;
    a.conv_w = conv_w;
    a.conv_state = conv_state;
    a.out_gate = out_gate;
    a.norm_weight = norm_weight;
    a.norm_eps = norm_eps;
    a.o = o;
    a.N = N;
    a.H = H;
    a.Hk = Hk;
    a.dk = dk;
    a.dv = dv;
    a.bf16 = dtype == GDN_BF16;
    a.scale = scale;
    a.l2norm = (flags & GDN_QK_L2NORM) ? 1 : 0;
    a.stream = static_cast<hipStream_t>(hip_stream);
    hipError_t e = gdn::launch_step(a);
    if (e == hipSuccess && conv_w && Hk != H) {
        // a query/key head's history is read by all its value heads' workgroups: shift the conv
        // state afterwards, as the update after N sequences of one token each
        gdn::ChunkArgs c{};
        c.q = q;
        c.k = k;
        c.v = v;
        c.cu = nullptr;
        c.conv_state = conv_state;
        c.N = N;
        c.T_tot = N;
        c.H = H;
        c.Hk = Hk;
        c.dk = dk;
        c.dv = dv;
        c.bf16 = a.bf16;
        c.stream = a.stream;
        e = gdn::launch_conv_state_update(c);
    }
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
