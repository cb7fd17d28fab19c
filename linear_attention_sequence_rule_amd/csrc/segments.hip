// segments.hip -- planning and workspace layout of the segmented long-sequence path.
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

}  // namespace gdn
