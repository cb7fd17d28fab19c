// segments.hip -- host-side planning of the prefill: rows per workgroup, segments of the
// long-sequence path, the workspace layout, and the per-device facts the launches need (read once
// per device, not once per call).
//
// The chunked schedule carries the state serially from chunk to chunk (page pzsr.cn/news/750,
// section 1、为什么要设计为chunk的模式), so one long sequence is one serial chain per (head, block of
// state rows): too few workgroups to fill 256 compute units.  The state map of a stretch of tokens
// is affine in the state that enters it (the rule is linear in S): S_out = S_in A + B, with
// A = the product of the per-token transitions alpha_t (I - beta_t k_t k_t^T) and B = the end state
// from a zero start.  Cutting the sequence into P segments, every segment runs in parallel from a
// zero start (B_p) and as a transition (A_p); the serial part shrinks to the P-step chain
// E_p = E_{p-1} A_p + B_p, which the rerun of each segment forms for itself (chunk_bf16.hip).
#include "kernels.hpp"

#include <mutex>
#include <vector>

namespace gdn {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

SegLayout seg_layout(int N, int H, int dk, int dv, int P) {
    SegLayout L;
    const size_t units = (size_t)N * P * H;
    L.off_E = 0;
    L.off_A = align256(units * dv * dk * 4);
    L.off_negl = L.off_A + align256(units * dk * dk * 4);
    L.off_pre = L.off_negl + align256(units * 4);
    L.off_ein = L.off_pre + align256(units * kSegPrepBytes);
    L.bytes = L.off_ein + align256(units * dv * dk * 4);
    return L;
}

int chunk_rows_per_workgroup(int dk, int rows) {
    if (dk == 128 && rows % 128 == 0) return 128;
    return rows >= 64 ? 64 : 32;
}

bool chunk_fuses_epilogue(int dk, int dv, bool bf16) { return bf16 && chunk_rows_per_workgroup(dk, dv) == 128; }

// The convolved q, k, v of the separate conv pass, each tensor 256-byte aligned.
size_t conv_prepass_bytes(int T_tot, int H, int Hk, int dk, int dv) {
    return 2 * align256((size_t)T_tot * Hk * dk * 2) + align256((size_t)T_tot * H * dv * 2);
}

hipError_t current_device_info(DeviceInfo* out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static DeviceInfo table[kMaxDevices];
    static bool known[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!known[dev]) {
        DeviceInfo d;
        e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&d.lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess) return e;
        table[dev] = d;
        known[dev] = true;
    }
    *out = table[dev];
    return hipSuccess;
}

hipError_t set_dynamic_lds(const void* fn, int bytes) {
    struct Done {
        const void* fn;
        int dev, bytes;
    };
    static std::mutex mu;
    static std::vector<Done> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    for (const Done& d : done)
        if (d.fn == fn && d.dev == dev && d.bytes >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.push_back(Done{fn, dev, bytes});
    return e;
}

int plan_segments(int N, int T_tot, int H, int dk, int dv, int requested) {
    if (requested > 0) return requested;
    int cus = 256;  // MI355X; the current device's count when it can be read
    DeviceInfo d;
    if (current_device_info(&d) == hipSuccess && d.cus > 0) cus = d.cus;
    const int rows = chunk_rows_per_workgroup(dk, dv);
    const long units = (long)N * H * (dv >= rows ? dv / rows : 1);  // workgroups of one pass
    if (units >= cus) return 1;
    const long chunks = ((long)T_tot / N + 63) / 64;
    long P = cus / units;
    if (P > chunks / 16) P = chunks / 16;
    if (P > 255) P = 255;
    return P < 1 ? 1 : (int)P;
}

}  // namespace gdn
