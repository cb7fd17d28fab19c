// chunk_bf16.hip -- fused chunked prefill of the gated delta rule on gfx950 MFMA (bf16 operands,
// fp32 accumulation, fp32 state held in registers across chunks).
//
// Method: page pzsr.cn/news/750, section 1、为什么要设计为chunk的模式 -- cut the sequence into chunks,
// compute inside a chunk in parallel, carry the state serially between chunks, and block the K/V
// dimensions.  The chunk algebra (derived from u_t = beta_t (v_t - alpha_t S_{t-1} k_t),
// S_t = alpha_t S_{t-1} + u_t k_t^T; the pages print no chunk algebra):
//   gamma = inclusive prefix sum of g in the chunk, M_ij = exp(gamma_i - gamma_j) (j <= i),
//   L = strict_lower(diag(beta) (M o Khat Khat^T)),  T = (I + L)^-1,
//   X = diag(beta) V - diag(beta Gamma) Khat S^T,  U = T X,
//   O = diag(Gamma) Qhat S^T + lower(M o Qhat Khat^T) U,
//   S <- Gamma_C S + U^T diag(exp(gamma_C - gamma)) Khat.
// Khat = diag(rk) K with rk = rsqrt(|k|^2 + eps) (likewise Qhat): the raw bf16 rows are the MFMA
// operands (exact); the norms come from the diagonals of K K^T and Q Q^T and are folded into the
// row and column scalings above.  Every decay factor is exp of a non-positive number.
//
// Work decomposition: one workgroup per (segment of a sequence, head h, block of state rows); state
// rows are independent, so the split is exact, and the per-chunk preparation (Grams, masks, solve,
// gates) is shared by the rows of the block.  Wide workgroups (dk = 128, 128 rows = the whole head)
// have 12 wavefronts, narrow ones (64 or 32 rows) 8.  Roles:
//   row waves (0..7 wide, 0..3 narrow; 16 state rows each): S, the output accumulators and U in
//     registers across the chunks.  Sub-stage A: K S^T and S Q^T, X, U = T X blockwise; sub-stage
//     B: the S update and O.  Wide: every row wave also loads an eighth of the next chunks;
//     narrow: waves 2 and 3 load them.
//   prep waves (8..11 wide, 4..7 narrow; prep index pw = 0..3): sub-stage A: pw 0, 3 K K^T and the
//     masked L of chunk k+1 (two row-tile halves, pw 0 also the norms); pw 1, 2 the masked Pm of
//     chunk k (likewise).  Sub-stage B: pw 0, 1 invert the two 32x32 diagonal blocks of I + L,
//     pw 2 copies the off-diagonal block L_BA next to them and pw 3 writes the gates of chunk k+1.
// U = T X is applied blockwise, so T's off-diagonal 32x32 block is never formed:
//   U_A = T_AA X_A,  U_B = T_BB (X_B - L_BA U_A).
// Two barriers per chunk; with the conv prologue a third sub-stage runs it on the chunks whose
// loads have landed.  Narrow workgroups keep each chunk's K, Q, V, g, beta in one of three
// buffers (loaded two chunks ahead); wide ones keep K, g, beta likewise but Q and V in two buffers
// loaded one chunk ahead (read only in sub-stage A).  The gates are double buffered; T, Pm and L
// single buffered (each is rewritten only after the barrier that ends its readers' sub-stage).
// K, Q and V rows are stored unpadded with their 16-byte slots XOR-swizzled by the row index
// (slot = part ^ (row mod parts-per-row)), which keeps every fragment read conflict-free and
// lets a 1 KB load instruction fill whole rows.  Each 16x16 MFMA output tile is fed to the next
// product as an operand ("chain order": lane group g = lane/16 holds k = 4g+e and 16+4g+e).
// Operands stored in the other orientation (T, V, K for the state update) are read with the
// gfx950 transposing LDS read ds_read_b64_tr_b16 (within each 16-lane group, output lane i
// element e is element i%4 of the 8 bytes addressed by lane 4e + i/4).
// MFMA v_mfma_f32_16x16x32_bf16: A lane l holds A[l%16][8(l/16)+e]; B: B[8(l/16)+e][l%16];
// D: D[4(l/16)+e][l%16].
#include <utility>

#include "common.hpp"
#include "kernels.hpp"
#include "prologue.hpp"

namespace gdn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float fx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int C = 64;        // chunk length
constexpr int BVMAX = 64;    // state rows of a narrow workgroup: 64, or 32 when the state has 32 rows
constexpr int BVW = 128;     // state rows of a wide workgroup (d_k = 128; chunk_rows_per_workgroup)
// Threads of a workgroup: 8 waves (narrow), 12 (wide).
template <int BV>
constexpr int kernel_threads() { return BV > BVMAX ? 768 : 512; }
constexpr int TSTR = C + 8;  // bf16 row stride of T^T, Pm and L^T

__device__ __forceinline__ fx4 mfma(bf16x8 a, bf16x8 b, fx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ fx4 zero4() { return fx4{0.f, 0.f, 0.f, 0.f}; }
// A copy of x that the compiler cannot see through: lane-dependent address arithmetic derived
// from it is recomputed where it is used instead of being hoisted out of the chunk loop, where
// it would stay live in registers across every role's code.  x is a lane or thread index: the
// range is restated after the asm, so that x / 16, x % 4 and the like stay single shifts and
// masks (for an int the compiler cannot prove non-negative they are signed divisions, five
// instructions each).
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    __builtin_assume(x >= 0 && x < 1024);
    return x;
}
// Keep every instruction before this point (typically a batch of LDS operand reads) ahead of
// everything after it: with one wavefront per SIMD the reads must be in flight early.
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }
// Make this wave's LDS writes visible to its other lanes.  The hardware runs a wave's LDS
// accesses in order, but the compiler models every lane as a thread of its own: without a
// synchronising operation it may treat a lane's read of another lane's write as a race and, for
// instance, forward the lane's own stored value instead of reading LDS.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Swizzled row-major tile of R rows x W bf16 (W/8 16-byte slots per row): element (r, c) lives at
// r*W + 8*((c/8) ^ (r % (W/8))) + c%8.
template <int W>
__device__ __forceinline__ int swz(int r, int c) {  // r, c >= 0: unsigned arithmetic, masks and shifts
    const unsigned ur = (unsigned)r, uc = (unsigned)c;
    return (int)(ur * W + 8u * ((uc / 8u) ^ (ur % (W / 8))) + (uc % 8u));
}
// 16-byte natural-order fragment of a swizzled tile: row r, columns kb + 8g .. +7
template <int W>
__device__ __forceinline__ bf16x8 sfrag_nat(const __bf16* M, int r, int kb, int g) {
    return *reinterpret_cast<const bf16x8*>(M + swz<W>(r, kb + 8 * g));
}
// chain-order fragment of a swizzled tile: row r, columns kb + 4g .. +3 and kb + 16 + 4g .. +3
template <int W>
__device__ __forceinline__ bf16x8 sfrag_chain(const __bf16* M, int r, int kb, int g) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(M + swz<W>(r, kb + 4 * g));
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(M + swz<W>(r, kb + 16 + 4 * g));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// chain-order fragment of a padded row-major tile: row[kb + 4g .. +3] and row[kb + 16 + 4g .. +3]
__device__ __forceinline__ bf16x8 frag_chain(const __bf16* row, int kb, int g) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(row + kb + 4 * g);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(row + kb + 16 + 4 * g);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Transposing reads (ds_read_b64_tr_b16): the calling lane, lane i of its 16-lane group, receives
// M[r0 .. r0+3][c0 + i].  r0, c0 are group-uniform.  Source lane s of the group addresses
// M[r0 + s/4][c0 + 4(s%4) .. +3].
__device__ __forceinline__ bf16x4 tr_read(const __bf16* src) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(const void*)src);
}
template <int W>
__device__ __forceinline__ bf16x4 str4(const __bf16* M, int r0, int c0, int l16) {  // swizzled tile
    return tr_read(M + swz<W>(r0 + l16 / 4, c0 + 4 * (l16 % 4)));
}
__device__ __forceinline__ bf16x4 tr4(const __bf16* M, int stride, int r0, int c0, int l16) {  // padded tile
    return tr_read(M + (r0 + l16 / 4) * stride + c0 + 4 * (l16 % 4));
}
// chain-order fragments of the transpose: lane (i, g) gets M[kb + 4g .. +3][c0 + i] and
// M[kb + 16 + 4g .. +3][c0 + i]
template <int W>
__device__ __forceinline__ bf16x8 sfrag_tr_chain(const __bf16* M, int kb, int c0, int g, int l16) {
    const bf16x4 a = str4<W>(M, kb + 4 * g, c0, l16);
    const bf16x4 b = str4<W>(M, kb + 16 + 4 * g, c0, l16);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 frag_tr_chain(const __bf16* M, int stride, int kb, int c0, int g, int l16) {
    const bf16x4 a = tr4(M, stride, kb + 4 * g, c0, l16);
    const bf16x4 b = tr4(M, stride, kb + 16 + 4 * g, c0, l16);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// natural-order fragment of the transpose: lane (i, g) gets M[kb + 8g .. +7][c0 + i]
__device__ __forceinline__ bf16x8 frag_tr_nat(const __bf16* M, int stride, int kb, int c0, int g, int l16) {
    const bf16x4 a = tr4(M, stride, kb + 8 * g, c0, l16);
    const bf16x4 b = tr4(M, stride, kb + 8 * g + 4, c0, l16);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Lane-constant element offsets into a swizzled DK-wide tile (PPR = DK/8 slots per row), so that
// fragment reads become base + constant + immediate.  For rows 16t + l16 the XOR key is l16 % PPR.
//   chain(ks, h): row l16, columns 32ks + 16h + 4g .. +3   (add 16t*DK for row tile t)
//   nat(ks):      row l16, columns 32ks + 8g .. +7         (add 16t*DK)
//   trk(dt):      row 4g + l16/4, columns 16dt + 4(l16%4)  (transposing source; add row offset kb*DK)
template <int DK>
__device__ __forceinline__ int off_chain(int ks, int h, int g, int l16) {
    constexpr int PPR = DK / 8;
    const int key = l16 % PPR;
    return l16 * DK + 8 * ((4 * ks + 2 * h + g / 2) ^ key) + 4 * (g % 2);
}
template <int DK>
__device__ __forceinline__ int off_nat(int ks, int g, int l16) {
    constexpr int PPR = DK / 8;
    const int key = l16 % PPR;
    return l16 * DK + 8 * ((4 * ks + g) ^ key);
}
template <int DK>
__device__ __forceinline__ int off_trk(int dt, int g, int l16) {
    // source lane 4e + q of the group addresses row 4g + e, columns kcol(dt, 4q) .. +3, so that
    // output lane i receives column kcol(dt, i) (the state tile's key order, see kcol)
    constexpr int PPR = DK / 8;
    const int row = 4 * g + l16 / 4;
    const int key = row % PPR;
    return row * DK + 8 * ((4 * (dt / 2) + (l16 % 4)) ^ key) + 4 * (dt % 2);
}
// Key column held by row r (0..15) of state tile dt: the tiles are ordered so that the pair
// (2ks, 2ks+1) gives lane group g the eight consecutive columns 32ks + 8g .. +7 (the natural
// operand order of a 16x16x32 MFMA), i.e. tile 2ks holds 32ks + 8(r/4) + r%4 and tile 2ks+1 the
// same plus 4.
__device__ __forceinline__ int kcol(int dt, int r) { return 32 * (dt / 2) + 8 * (r / 4) + 4 * (dt % 2) + r % 4; }
template <typename T>
__device__ __forceinline__ T lds_at(const __bf16* base, int off) {
    return *reinterpret_cast<const T*>(base + off);
}

// Two D fragments (rows 4g+e of consecutive 16-row tiles) as one chain-order operand.
__device__ __forceinline__ bf16x8 pack_chain(fx4 a, fx4 b) {
    bf16x8 r;
    r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
    r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
    return r;
}
// The bf16 rounding residuals of pack_chain(a, b) = hi: a + b - hi in bf16, so that hi + lo carries
// the fp32 values to about 16 significant bits.
__device__ __forceinline__ bf16x8 pack_chain_lo(fx4 a, fx4 b, bf16x8 hi) {
    fx4 ra, rb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        ra[e] = a[e] - (float)hi[e];
        rb[e] = b[e] - (float)hi[4 + e];
    }
    return pack_chain(ra, rb);
}
__device__ __forceinline__ float sel4(fx4 v, int e) {
    return e == 0 ? v[0] : (e == 1 ? v[1] : (e == 2 ? v[2] : v[3]));
}

// ------------------------------------------------------------------------------------------
// LDS layout (bytes).  A chunk's K, g and beta sit in one of three buffers that rotate by chunk
// index mod 3.  Narrow workgroups (up to 64 state rows) keep its Q and V in the same buffer; wide
// ones (128 rows) keep them in one of two buffers of their own that rotate by chunk parity: Q and V
// are read only in the first sub-stage of the chunk's iteration, so they are loaded one chunk
// ahead instead of two.  Gate buffers rotate by chunk parity.
template <int DK, int BV>
struct Smem {
    static constexpr bool WIDE = BV > BVMAX;
    // K buffer (narrow: the whole raw chunk buffer); K, Q, V swizzled, unpadded
    static constexpr int rK = 0;                                  // bf16 [C][DK]
    static constexpr int rQ = WIDE ? 0 : rK + C * DK * 2;         // bf16 [C][DK] (wide: in the Q/V buffer)
    static constexpr int rV = rQ + C * DK * 2;                    // bf16 [C][BV] (narrow: room for BVMAX)
    static constexpr int rG = WIDE ? C * DK * 2 : rV + C * BVMAX * 2;  // raw g [C]
    static constexpr int rB = rG + C * 4;                         // beta [C]
    static constexpr int rBytes = rB + C * 4;
    static constexpr int qvBytes = WIDE ? rV + C * BV * 2 : 0;    // wide: Q/V buffer
    static constexpr int NQV = WIDE ? 2 : 0;
    // gates of a chunk
    static constexpr int gKK = 0;                    // beta Gamma rk^2 [C]
    static constexpr int gVB = gKK + C * 4;          // beta rk [C]
    static constexpr int gDR = gVB + C * 4;          // exp(gamma_C - gamma) [C]
    static constexpr int gGAM = gDR + C * 4;         // Gamma [C]
    static constexpr int gGC = gGAM + C * 4;         // Gamma_C, log bound of the chunk's transition (2 of 16 floats)
    static constexpr int gBytes = gGC + 64;
    // layout
    static constexpr int R0 = 0;
    static constexpr int Q0 = R0 + 3 * rBytes;
    static constexpr int G0 = Q0 + NQV * qvBytes;
    static constexpr int T = G0 + 2 * gBytes;        // T^T bf16 [C][TSTR] (T^T[m][i] = T_im); L_BA in the T_BA block
    static constexpr int PM = T + C * TSTR * 2;      // Pm bf16 [C][TSTR], row-major [i][m]
    static constexpr int L = PM + C * TSTR * 2;      // L^T bf16 [C][TSTR]: L^T[j][i] = L_ij
    static constexpr int ORQ = L + C * TSTR * 2;     // rq [C]
    static constexpr int WL = ORQ + C * 4;           // L-prep scratch [4][C]: rk, gamma log2e (part 0), f, gamma log2e (part 1)
    static constexpr int WP = WL + 4 * C * 4;        // P-prep scratch, per wave: rq, gamma log2e [2][2][C]
    static constexpr int HB = WP + 4 * C * 4;        // conv halo: 3 raw rows [3][DK + BV/2] channel pairs
    static constexpr int CW = HB + 3 * (DK + (WIDE ? BV : BVMAX) / 2) * 4;  // wide: conv weights [8][48][4] fp32 (x -log2 e)
    static constexpr int EP = CW + (WIDE ? 48 * 8 * 16 : 0);  // wide epilogue: row sums of o^2 [C][8 row waves]
    static constexpr int NW = EP + (WIDE ? C * 8 * 4 : 0);    // wide epilogue: w of the block's rows [BV]
    static constexpr int bytes = NW + (WIDE ? BV * 4 : 0);
    static_assert(rBytes % 16 == 0 && gBytes % 16 == 0 && qvBytes % 16 == 0, "alignment");
    static_assert(bytes <= 160 * 1024, "LDS of one gfx950 compute unit");
    static __device__ __forceinline__ int raw(int c) { return R0 + (c % 3) * rBytes; }  // K, g, beta (narrow: all)
    static __device__ __forceinline__ int qv(int c) { return WIDE ? Q0 + (c & 1) * qvBytes : raw(c); }  // Q, V
    static __device__ __forceinline__ int gates(int c) { return G0 + (c & 1) * gBytes; }
};

// The prepared operands of a segment's first chunk as kept in the workspace, per (segment, head):
// the T region (T'^T with L'_BA in its BA block), Pm, rq and the chunk's gates, each as laid out
// in LDS.  The same for every DK and row block.
constexpr int PRE_T = 0;                       // bf16 [C][TSTR]
constexpr int PRE_PM = PRE_T + C * TSTR * 2;   // bf16 [C][TSTR]
constexpr int PRE_RQ = PRE_PM + C * TSTR * 2;  // fp32 [C]
constexpr int PRE_G = PRE_RQ + C * 4;          // gates [gBytes]
constexpr int PRE_BYTES = PRE_G + Smem<32, 32>::gBytes;
static_assert(PRE_BYTES == (int)kSegPrepBytes, "workspace layout of the kept operands");
static_assert(Smem<128, 128>::PM == Smem<128, 128>::T + C * TSTR * 2 && PRE_BYTES % 16 == 0, "layout");

// How a workgroup starts its state, and what it does with o (one launch runs one of the passes of
// the segmented long-sequence path, or the plain single pass).
enum InitMode { INIT_S0 = 0, INIT_IDENTITY = 1, INIT_PREV = 2 };
enum NeglMode { NEGL_NONE = 0, NEGL_MARK = 1, NEGL_SKIP = 2 };
enum OutMode { OUT_NONE = 0, OUT_STORE = 1 };
// The prepared operands of a segment's first chunk: kept by the first pass of the segmented path,
// used by the rerun when that chunk alone brings the transition bound below 2^-40.
enum PreMode { PRE_NONE = 0, PRE_KEEP = 1, PRE_USE = 2 };

template <int DK>
struct Params {
    const __bf16 *q, *k, *v;
    const float *g, *beta, *s0, *conv_w;
    const float* gate_params;  // [2, H]: g and beta hold the raw a and b; or null
    const __bf16* conv_state;  // [N, 3, 2 Hk DK + H dv]: conv history before each sequence; or null
    const int32_t* cu;
    __bf16* o;
    const __bf16* out_gate;     // wide workgroups: z of the output epilogue [T_tot, H, dv], or null
    const float* norm_weight;   // w of the output epilogue [dv] (with out_gate)
    float norm_eps;
    float* sfin;   // end state per (segment, head): [N*P, H, dv, dk]
    int* negl;     // per (segment, head): nonzero if the segment's transition is negligible (or null)
    int N, T_tot, H, dv, nv;
    int Hk, grp;   // query/key heads; value heads per query/key head (H = Hk grp)
    int P;         // segments per sequence (1 = the sequence in one piece)
    int init;      // InitMode: S0 = s0[n] for segment 0 and zero for the others; IDENTITY = I
                   // (dv = dk rows); PREV = the state entering segment p: s0[(n P + p - 1) H + h]
                   // (B_{p-1}) where A_{p-1} is negligible, else the chain formed in place (ein)
    int out;       // OutMode: o stored, or not written
    int v_zero;    // values taken as zero (v is not read)
    int early_exit;  // stop once the product of the decays since the start is <= 2^-40
    int skip_first;  // segment 0 does nothing
    int negl_mode;   // NEGL_MARK: record whether the whole segment's transition bound is <= 2^-40;
                     // NEGL_SKIP: skip segments so marked, record a stop at the bound
    unsigned char* pre;  // per (segment, head): the first chunk's prepared operands [PRE_BYTES]
    int pre_mode;        // PreMode
    // rerun of the segmented path: the state entering segment p is formed here from the end
    // states B_j (s0), the transitions A_j and their marks (nonzero = negligible)
    const int* marks;     // [N*P, H], or null (no chaining)
    const float* trans;   // A_j [N*P, H, DK, DK]
    float* ein;           // per (segment, head): the entering state where it had to be chained
    float* fin;           // the final state [N, H, dv, DK], or null: the first pass stores B_{P-1} there
                          // (not in its slot of s0), which is E_{P-1} where A_{P-1} is negligible; the
                          // rerun of the last segment chains E_{P-1} over it otherwise
    int fin_in_slot;      // the final state is the initial state's buffer (read by the first pass's
                          // segment 0 while the last segment would write it): the first pass then
                          // keeps B_{P-1} in its slot of s0 and the rerun of the last segment always
                          // writes the final state (a copy of B_{P-1} where A_{P-1} is negligible)
    // transition and rerun in one launch (chunk_bf16_tail_kernel): a workgroup that forms its
    // pair's transition adds its completion to the pair's mark, and a rerun waits for the marks it
    // reads (wait_transitions)
    int tr_signal;  // transition: add 4 (+ stopped, first row block) to negl[pair] at the end
    int tr_wait;    // rerun: the mark of a pair whose transition has finished is >= this (0: no wait)
    float scale;
    int l2norm;
};

// A pair's mark: 1 = negligible from the first pass's gate bound; otherwise 0 until its transition
// workgroups finish (in a launch of their own: 0 or 1 = whether they stopped at the bound; with
// the reruns in the same launch: 4 per workgroup plus that bit).  Bit 0 says negligible.
__device__ __forceinline__ bool mark_negligible(int m) { return (m & 1) != 0; }

// ------------------------------------------------------------------------------------------
// chunk loads: direct global -> LDS (global_load_lds_dwordx4 / _dword).  One instruction moves
// 1 KB (64 lanes x 16 B) into a contiguous LDS range; lane l fills 16-byte slot l of that range,
// so each lane fetches the global part that the swizzle places in its slot.  A wave loads a block
// of rows of K, Q and V (and g or beta); rows past the tail re-read the last valid row and are
// cleared once the loads have landed.
// One global_load_lds instruction (scalar-base form): lane l copies 16 (or 4) bytes from
// base + voff(l) to LDS byte address lds + 16 l (4 l).  base and lds are wave-uniform; voff is a
// per-lane byte offset below 4 GiB (the base already points at the chunk's first token).  Issued
// through asm so that the compiler does not make every later LDS read of this wave wait for it:
// the issuing wave waits explicitly (wait_loads) before the data is published.
__device__ __forceinline__ void dma16(const void* base, unsigned voff, unsigned lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, unsigned voff, unsigned lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}
// LDS byte addresses are formed as integers from the address of the shared array itself (a
// constant), never by converting a computed flat pointer into LDS: that conversion made the
// backend materialise the shared aperture base under register pressure, illegally.
typedef __attribute__((address_space(3))) unsigned char lds_u8;
__device__ __forceinline__ unsigned lds_base(unsigned char* sm) {
    return static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_u8*)(void*)sm));
}
__device__ __forceinline__ unsigned lds_addr(unsigned a) { return __builtin_amdgcn_readfirstlane(a); }
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
    const uintptr_t u = reinterpret_cast<uintptr_t>(p);
    const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(u));
    const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(u >> 32));
    return reinterpret_cast<const T*>((static_cast<uintptr_t>(hi) << 32) | lo);
}

// Rows [r0, r0 + NR) of a swizzled W-wide bf16 tile (W/8 16-byte slots per row, swz<W>) from global
// rows rowb bytes apart starting at base (wave-uniform: the chunk's first token); tile = LDS byte
// address of the tile.  Rows past the tail re-read the last valid row.
template <int W, int NR>
__device__ __forceinline__ void dma_tile(const __bf16* base, unsigned rowb, unsigned tile, int len, unsigned r0,
                                         unsigned ul) {
    constexpr unsigned PPR = W / 8;    // 16-byte slots per row
    constexpr unsigned RPI = 64 / PPR;  // rows per 1 KB instruction
    static_assert(NR % RPI == 0, "whole instructions per part");
    const unsigned lrow = ul / PPR, slot = ul % PPR;
#pragma unroll
    for (unsigned j = 0; j < NR / RPI; ++j) {
        const unsigned row0 = r0 + RPI * j;
        const unsigned part = slot ^ ((row0 + lrow) % PPR);  // the swizzle key of the lane's row
        const unsigned voff = len == C ? (lrow + row0) * rowb + 16u * part
                                       : (unsigned)min((int)(row0 + lrow), len - 1) * rowb + 16u * part;
        dma16(base, voff, lds_addr(tile + row0 * W * 2));
    }
}
// g (which = 0) or beta (1) of the chunk's tokens into [C] floats at LDS byte address dst
template <int DK>
__device__ __forceinline__ void dma_gates_in(const Params<DK>& p, unsigned dst, long t0, int len, int h, int which,
                                             int lane) {
    const float* gbase = uniform_ptr((which == 0 ? p.g : p.beta) + (size_t)t0 * p.H + h);
    const unsigned voff = (unsigned)min(lane, len - 1) * (unsigned)p.H * 4u;
    dma4(gbase, voff, lds_addr(dst));
}
template <int DK, int NR>
__device__ __forceinline__ void dma_k(const Params<DK>& p, unsigned tile, long t0, int len, int hk, int r0, int lane) {
    const size_t tokk = (size_t)t0 * p.Hk + hk;
    dma_tile<DK, NR>(uniform_ptr(p.k + tokk * DK), (unsigned)(p.Hk * DK) * 2u, tile, len, r0, (unsigned)opaque(lane));
}
template <int DK, int NR>
__device__ __forceinline__ void dma_q(const Params<DK>& p, unsigned tile, long t0, int len, int hk, int r0, int lane) {
    const size_t tokk = (size_t)t0 * p.Hk + hk;
    dma_tile<DK, NR>(uniform_ptr(p.q + tokk * DK), (unsigned)(p.Hk * DK) * 2u, tile, len, r0, (unsigned)opaque(lane));
}
template <int DK, int BV, int NR>
__device__ __forceinline__ void dma_v(const Params<DK>& p, unsigned tile, long t0, int len, int h, int vb, int r0,
                                      int lane) {
    const size_t tok0 = (size_t)t0 * p.H + h;
    dma_tile<BV, NR>(uniform_ptr(p.v + tok0 * p.dv + vb * BV), (unsigned)(p.H * p.dv) * 2u, tile, len, r0,
                     (unsigned)opaque(lane));
}

template <int DK, int BV, int NR>
__device__ __forceinline__ void dma_z(const Params<DK>& p, unsigned tile, long t0, int len, int h, int vb, int r0,
                                      int lane) {
    const size_t tok0 = (size_t)t0 * p.H + h;
    dma_tile<BV, NR>(uniform_ptr(p.out_gate + tok0 * p.dv + vb * BV), (unsigned)(p.H * p.dv) * 2u, tile, len, r0,
                     (unsigned)opaque(lane));
}

// Narrow workgroups: part w (0..3) of a chunk is rows [16w, 16w + 16) of K, Q and V, and g (part 0)
// or beta (part 1).
template <int DK, int BV>
__device__ __forceinline__ void dma_chunk(const Params<DK>& p, unsigned smb, int rawoff, long t0, int len, int h,
                                          int hk, int vb, int wid, int lane) {
    using S = Smem<DK, BV>;
    dma_k<DK, 16>(p, smb + rawoff + S::rK, t0, len, hk, 16 * wid, lane);
    dma_q<DK, 16>(p, smb + rawoff + S::rQ, t0, len, hk, 16 * wid, lane);
    if (!p.v_zero) dma_v<DK, BV, 16>(p, smb + rawoff + S::rV, t0, len, h, vb, 16 * wid, lane);
    if (wid < 2) dma_gates_in<DK>(p, smb + rawoff + (wid == 0 ? S::rG : S::rB), t0, len, h, wid, lane);
}

// Rows >= len of rows [r0, r0 + NR) of a W-wide tile set to zero (whole rows, so the swizzle does
// not matter).
template <int W, int NR>
__device__ __forceinline__ void zero_rows(__bf16* M, int len, int r0, int lane) {
    const __bf16 z = (__bf16)0.f;
    for (int i = lane; i < NR * W; i += 64) {
        const int row = r0 + i / W;
        if (row >= len) M[row * W + i % W] = z;
    }
}

// After this wave's loads landed: clear its rows past the tail (last chunk of a sequence only).
template <int DK, int BV>
__device__ __forceinline__ void zero_tail(unsigned char* raw, int len, int wid, int lane) {
    lane = opaque(lane);
    using S = Smem<DK, BV>;
    if (len >= C) return;
    zero_rows<DK, 16>(reinterpret_cast<__bf16*>(raw + S::rK), len, 16 * wid, lane);
    zero_rows<DK, 16>(reinterpret_cast<__bf16*>(raw + S::rQ), len, 16 * wid, lane);
    zero_rows<BV, 16>(reinterpret_cast<__bf16*>(raw + S::rV), len, 16 * wid, lane);
    if (wid < 2 && lane >= len) reinterpret_cast<float*>(raw + (wid == 0 ? S::rG : S::rB))[lane] = 0.f;
}

// After this wave's loads landed: with raw gates, turn the raw a (part 0) and b (part 1) of the
// chunk's valid rows into g and beta in place, before anything reads them.  The same formulas as
// raw_decay / raw_beta, on the hardware exp2 / log2 / reciprocal: log1p(y) for y = exp(-|x|) in
// (0, 1] is taken as log(1 + y), whose absolute error (below 2^-23) is far under the bf16 path's
// rounding, and this runs once per token on the wave that loaded the chunk.
template <int DK, int BV>
__device__ __forceinline__ void raw_gates(const Params<DK>& p, unsigned char* raw, int len, int part, int lane, int h) {
    using S = Smem<DK, BV>;
    if (part >= 2) return;
    float* x = reinterpret_cast<float*>(raw + (part == 0 ? S::rG : S::rB));
    if (lane < len) {
        const float a = x[lane];
        float r;
        if (part == 0) {
            const float z = a + p.gate_params[p.H + h];
            const float sp = fmaxf(z, 0.f) + __logf(1.f + __expf(-fabsf(z)));
            r = -__expf(p.gate_params[h]) * sp;
        } else {
            r = __builtin_amdgcn_rcpf(1.f + __expf(-a));
        }
        x[lane] = r;
    }
}

__device__ __forceinline__ void wait_loads() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's global->LDS loads have landed
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS accesses (lgkmcnt(0)) but,
// unlike __syncthreads(), not for its global loads and stores, so the chunk prefetch and the
// output stores stay in flight across it.  The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------------------------------
// Conv prologue (page maplevalley.com.cn/news/1910399, section 3.1, 卷积预处理): a depthwise causal
// conv over 4 tokens (tap 3 = current token; before the sequence start the given conv history, else
// zeros) and SiLU on every q, k and v channel, in place in the chunk's LDS tiles once all of its
// loads have landed.
// Work item = (channel pair, block of 8 rows), taken in turn by all lanes.  An item first
// reads its 8 raw rows and the 3 raw rows before them (from the tile, or for the first block from
// the halo buffer that keeps the previous chunk's last 3 raw rows); after a barrier -- no raw row
// is overwritten before every item has read it -- it writes its results, and the items of the last
// block store their raw rows in the halo buffer for the next chunk.  fp32 arithmetic, bf16 result.
typedef __attribute__((address_space(3))) uint32_t lds_u32;
__device__ __forceinline__ uint32_t ld32(unsigned a) { return *reinterpret_cast<lds_u32*>(static_cast<uintptr_t>(a)); }
__device__ __forceinline__ void st32(unsigned a, uint32_t v) { *reinterpret_cast<lds_u32*>(static_cast<uintptr_t>(a)) = v; }

__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
}
typedef float fx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {  // one v_cvt_pk_bf16_f32
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(fx2{a, b}, bf16x2));
}

template <int DK, int BV>
struct ConvPlan {
    static constexpr int NP = DK + BV / 2;              // channel pairs: K (DK/2), Q (DK/2), V (BV/2)
    static constexpr int ITEMS = NP * (C / 8);
    static constexpr int NT = kernel_threads<BV>();
    static constexpr int PER = (ITEMS + NT - 1) / NT;   // items per lane, at most
};

// Where channel pair pc lives in a raw buffer: tile offset, row width W (bf16), its 16-byte slot
// and offset in the slot; then row r is at tile + 2 (r W + 8 (slot ^ (r mod W/8)) + off)
// (the swizzle of swz<W>), computed without branches.
struct PairLoc {
    unsigned tile, w, mask, slot, off;
};
template <int DK, int BV>
__device__ __forceinline__ PairLoc pair_loc(int pc) {
    using S = Smem<DK, BV>;
    const bool isv = pc >= DK, isq = !isv && pc >= DK / 2;
    const int c = 2 * (isv ? pc - DK : (isq ? pc - DK / 2 : pc));
    PairLoc l;
    l.tile = isv ? S::rV : (isq ? S::rQ : S::rK);
    l.w = isv ? BV : DK;
    l.mask = l.w / 8 - 1;
    l.slot = c / 8;
    l.off = c % 8;
    return l;
}
__device__ __forceinline__ unsigned pair_addr(unsigned raw, const PairLoc& l, int r) {
    return raw + l.tile + 2u * (r * l.w + 8u * (l.slot ^ (r & l.mask)) + l.off);
}
// conv_w row of the first channel of pair pc (q channels of the Hk query/key heads, then k, then
// v of the H value heads)
template <int DK, int BV>
__device__ __forceinline__ int pair_wrow(const Params<DK>& p, int pc, int h, int hk, int vb) {
    if (pc < DK / 2) return (p.Hk + hk) * DK + 2 * pc;
    if (pc < DK) return hk * DK + 2 * (pc - DK / 2);
    return 2 * p.Hk * DK + h * p.dv + vb * BV + 2 * (pc - DK);
}

// Halo before the first chunk, by `from`: HALO_ZERO; HALO_TOKENS, the three raw tokens before bos
// (a segment that starts inside a sequence); HALO_STATE, the conv history of sequence n (a sequence
// start with conv_state).  Layout [3 rows][NP pairs] of 4-byte words, oldest row first.
enum HaloFrom { HALO_ZERO = 0, HALO_TOKENS = 1, HALO_STATE = 2 };
template <int DK, int BV>
__device__ void conv_halo_init(const Params<DK>& p, unsigned halo, int tid, int n, int h, int hk, int vb, long bos,
                               int from) {
    constexpr int NP = ConvPlan<DK, BV>::NP;
    const size_t CC = (size_t)2 * p.Hk * DK + (size_t)p.H * p.dv;  // conv channels per token
    for (int i = tid; i < 3 * NP; i += ConvPlan<DK, BV>::NT) {
        const int j = i / NP, pc = i % NP;
        uint32_t v = 0;
        const bool isv = pc >= DK, isq = !isv && pc >= DK / 2;
        if (from != HALO_ZERO && !(isv && p.v_zero)) {
            // one load per source tensor (no selected pointer, which the compiler would keep in memory)
            const int c2 = 2 * (isv ? pc - DK : (isq ? pc - DK / 2 : pc));  // channel within the head's block
            if (from == HALO_STATE) {
                const size_t hc = isv ? (size_t)2 * p.Hk * DK + h * p.dv + vb * BV + c2
                                      : (isq ? (size_t)hk * DK + c2 : (size_t)(p.Hk + hk) * DK + c2);
                v = *reinterpret_cast<const uint32_t*>(p.conv_state + ((size_t)n * 3 + j) * CC + hc);
            } else {
                const size_t t = (size_t)(bos - 3 + j);
                if (isv)
                    v = *reinterpret_cast<const uint32_t*>(p.v + (t * p.H + h) * p.dv + vb * BV + c2);
                else if (isq)
                    v = *reinterpret_cast<const uint32_t*>(p.q + (t * p.Hk + hk) * DK + c2);
                else
                    v = *reinterpret_cast<const uint32_t*>(p.k + (t * p.Hk + hk) * DK + c2);
            }
        }
        st32(halo + 4u * (j * NP + pc), v);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing of this stays pending into the chunk loop
}

// The weights of a lane's items: the same items every chunk, so they are loaded once.
template <int DK, int BV>
struct ConvW {
    float w[ConvPlan<DK, BV>::PER][8];  // taps 0..3 of the pair's first channel, then of the second
};
template <int DK, int BV>
__device__ void conv_weights(ConvW<DK, BV>& cw, const Params<DK>& p, int tid, int h, int hk, int vb) {
    using CP = ConvPlan<DK, BV>;
#pragma unroll
    for (int q = 0; q < CP::PER; ++q) {
        const int it = tid + CP::NT * q, pc = it % CP::NP;
        const bool on = it < CP::ITEMS && !(pc >= DK && p.v_zero);
        const float* w = p.conv_w + (size_t)(on ? pair_wrow<DK, BV>(p, pc, h, hk, vb) : 0) * 4;
#pragma unroll
        for (int e = 0; e < 8; ++e) cw.w[q][e] = on ? w[e] : 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing of this stays pending into the chunk loop
}

// The conv + SiLU of one chunk's tiles; called by every lane.  rawK / rawQV: LDS byte addresses of
// the buffers holding the K tile and the Q, V tiles (the same buffer for narrow workgroups; wide
// ones convolve K of one chunk and Q, V of the previous one in the same call), lenK / lenQV the
// valid rows of each; parts: bit 0 the K channels, bit 1 the Q and V channels.  The halo keeps the
// last three raw rows of each channel pair, so each part must be convolved in chunk order.
template <int DK, int BV>
__device__ void conv_chunk(const Params<DK>& p, const ConvW<DK, BV>& cw, unsigned rawK, int lenK, unsigned rawQV,
                           int lenQV, unsigned halo, int parts, int tid) {
    tid = opaque(tid);
    using CP = ConvPlan<DK, BV>;
    constexpr int NP = CP::NP, PER = CP::PER;
    uint32_t xr[PER][11];
    bool act[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int it = tid + CP::NT * q, pc = it % NP, rb = it / NP;
        const bool isk = pc < DK / 2;
        act[q] = it < CP::ITEMS && !(pc >= DK && p.v_zero) && (parts & (isk ? 1 : 2));
        if (!act[q]) continue;
        const PairLoc l = pair_loc<DK, BV>(pc);
        const unsigned raw = isk ? rawK : rawQV;
#pragma unroll
        for (int j = 0; j < 3; ++j)
            xr[q][j] = ld32(rb == 0 ? halo + 4u * (j * NP + pc) : pair_addr(raw, l, 8 * rb - 3 + j));
#pragma unroll
        for (int j = 0; j < 8; ++j) xr[q][3 + j] = ld32(pair_addr(raw, l, 8 * rb + j));
    }
    lds_barrier();  // every raw row has been read
    tid = opaque(tid);                   // recompute the store addresses rather than keep them live
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (!act[q]) continue;
        const int it = tid + CP::NT * q, pc = it % NP, rb = it / NP;
        const bool isk = pc < DK / 2;
        const PairLoc l = pair_loc<DK, BV>(pc);
        const unsigned raw = isk ? rawK : rawQV;
        const int len = isk ? lenK : lenQV;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 8 * rb + j;
            float lo[4], hi[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                lo[d] = __uint_as_float(xr[q][j + d] << 16);
                hi[d] = __uint_as_float(xr[q][j + d] & 0xFFFF0000u);
            }
            const float* a = cw.w[q];
            const float y0 = a[0] * lo[0] + a[1] * lo[1] + a[2] * lo[2] + a[3] * lo[3];
            const float y1 = a[4] * hi[0] + a[5] * hi[1] + a[6] * hi[2] + a[7] * hi[3];
            if (r < len)  // rows past the tail stay zero
                st32(pair_addr(raw, l, r), pack_bf16(silu(y0), silu(y1)));
        }
        if (rb == C / 8 - 1)
#pragma unroll
            for (int j = 0; j < 3; ++j) st32(halo + 4u * (j * NP + pc), xr[q][8 + j]);
    }
    lds_barrier();
}

// ------------------------------------------------------------------------------------------
// prep waves

// inclusive prefix sum over the 64 lanes of a wave
// (DPP row shifts inside each 16-lane row, then the three row totals added through readlane).
template <int N>
__device__ __forceinline__ float dpp_shr(float x) {  // lane l - N of the row, 0 for the first N lanes
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ float wave_scan(float x, int lane) {
    x += dpp_shr<1>(x);
    x += dpp_shr<2>(x);
    x += dpp_shr<4>(x);
    x += dpp_shr<8>(x);
    const float s0 = lane_value(x, 15), s1 = lane_value(x, 31), s2 = lane_value(x, 47);
    const int r = lane >> 4;
    return x + (r == 0 ? 0.f : (r == 1 ? s0 : (r == 2 ? s0 + s1 : (s0 + s1) + s2)));
}

// Norm of row 16 t + l16 from a diagonal Gram tile held in D layout: lane (l16, g = l16/4) holds
// the diagonal at element l16 % 4.  Writes rsqrt(x + eps) (0 past the tail, 1 without L2 norm).
__device__ __forceinline__ void write_norm(float* dst, fx4 diag, int t, int lane, int len, int l2norm) {
    const int g = lane / 16, l16 = lane % 16;
    if (g == l16 / 4) {
        const int i = 16 * t + l16;
        const float x = sel4(diag, l16 % 4);
        dst[i] = i < len ? (l2norm ? rsqrtf(x + kL2Eps) : 1.f) : 0.f;
    }
}

// write_norm for the K rows of L', which also leaves the row factor f_i = beta_i rk_i^2 of L'.
__device__ __forceinline__ void write_norm_f(float* rk, float* f, const float* beta, fx4 diag, int t, int lane, int len,
                                             int l2norm) {
    const int g = lane / 16, l16 = lane % 16;
    if (g == l16 / 4) {
        const int i = 16 * t + l16;
        const float x = sel4(diag, l16 % 4);
        const float r = i < len ? (l2norm ? rsqrtf(x + kL2Eps) : 1.f) : 0.f;
        rk[i] = r;
        f[i] = beta[i] * r * r;
    }
}

constexpr float kLog2e = 1.4426950408889634f;


// The norms are kept out of the masks by a diagonal similarity.  With D = diag(rk) (rk = 1 on
// padded rows, whose K, V and beta are zero), G = K K^T of the raw rows and
// G_m = strict_lower(M o G):  I + L = D^-1 (I + L') D  with  L' = diag(f) G_m,  f = beta rk^2,
// so T = D^-1 T' D with T' = (I + L')^-1, and with U' = D U:
//   U' = T' Y,   Y = diag(beta rk) V - diag(beta Gamma rk^2) K S^T,
//   O  = diag(rq) [ diag(Gamma) Q S^T + lower(M o Q K^T) U' ],
//   S <- Gamma_C S + U'^T diag(exp(gamma_C - gamma)) K.
// The masks need only the gates; f enters the solve as a row factor.

// Prep waves 0 and 3 on chunk k+1: K K^T row tiles {0, 3} (part 0) or {1, 2} (part 1) masked with
// M (those rows of L^T: bf16, L^T[j][i] = M_ij G_ij for j < i); each part also leaves the norms rk
// of its rows (from its two diagonal tiles) and gamma log2e for the next sub-stage.
// exp(gamma_i - gamma_j) = exp2 of a non-positive number.
template <int DK, int BV, int part>
__device__ __forceinline__ void prep_L(const unsigned char* raw, unsigned char* sm, int lane, int len, int l2norm) {
    lane = opaque(lane);
    using S = Smem<DK, BV>;
    constexpr int KS = DK / 32;
    constexpr int t0 = part ? 1 : 0, t1 = part ? 2 : 3;  // my row tiles
    const __bf16* K = reinterpret_cast<const __bf16*>(raw + S::rK);
    const float* gr = reinterpret_cast<const float*>(raw + S::rG);
    __bf16* sLt = reinterpret_cast<__bf16*>(sm + S::L);
    float* own = reinterpret_cast<float*>(sm + S::WL) + part * 2 * C;  // rk [C], gamma log2e [C]
    const int g = lane / 16, l16 = lane % 16;

    const float gam = wave_scan(gr[lane], lane);
    own[C + lane] = gam * kLog2e;
    wave_sync();  // the masks read other lanes' prefix sums

    // k-step outer: only one k-step of fragments is live at a time
    fx4 acc[2][4];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) acc[s2][jt] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int o = off_nat<DK>(ks, g, l16);
        bf16x8 kf[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) kf[rb] = lds_at<bf16x8>(K, o + 16 * rb * DK);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int it = s2 ? t1 : t0;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                if (jt <= it) acc[s2][jt] = mfma(kf[it], kf[jt], acc[s2][jt]);
        }
    }
    const float* g2 = own + C;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        const int it = s2 ? t1 : t0;
        const int i0 = 16 * it + 4 * g;
        const fx4 ai = *reinterpret_cast<const fx4*>(g2 + i0);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            if (jt > it) continue;
            const int j = 16 * jt + l16;
            const float bj = g2[j];
            bf16x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float val = __builtin_amdgcn_exp2f(ai[e] - bj) * acc[s2][jt][e];
                out[e] = (__bf16)((jt < it || j < i0 + e) ? val : 0.f);
            }
            *reinterpret_cast<bf16x4*>(sLt + j * TSTR + i0) = out;
        }
    }
    // rk of this part's rows (from the diagonal tiles of its own Gram tiles) for the gates of the
    // next sub-stage, and the row factors f = beta rk^2 of L' for the solve: both parts write
    // part 0's rk array and the f array
    float* rk = reinterpret_cast<float*>(sm + S::WL);
    const float* beta = reinterpret_cast<const float*>(raw + S::rB);
    write_norm_f(rk, rk + 2 * C, beta, acc[0][t0], t0, lane, len, l2norm);
    write_norm_f(rk, rk + 2 * C, beta, acc[1][t1], t1, lane, len, l2norm);
}

// Prep wave 3, sub-stage B, on chunk k+1: the gates, from rk and gamma log2e left by part 0 of prep_L.
template <int DK, int BV>
__device__ __forceinline__ void make_gates(const unsigned char* raw, unsigned char* gb, const unsigned char* sm,
                                           int lane, int l2norm) {
    lane = opaque(lane);
    using S = Smem<DK, BV>;
    const float* own = reinterpret_cast<const float*>(sm + S::WL);  // part 0: rk [C], gamma log2e [C]
    const float b = reinterpret_cast<const float*>(raw + S::rB)[lane];
    const float rk = own[lane];
    const float gam = own[C + lane] * (1.f / kLog2e);
    const float gl = lane_value(gam, C - 1);
    const float G = __expf(gam);
    reinterpret_cast<float*>(gb + S::gKK)[lane] = b * G * rk * rk;
    reinterpret_cast<float*>(gb + S::gVB)[lane] = b * rk;
    reinterpret_cast<float*>(gb + S::gDR)[lane] = __expf(gl - gam);
    reinterpret_cast<float*>(gb + S::gGAM)[lane] = G;
    // log of the bound on the norm of this chunk's state transition: every token multiplies the
    // state by alpha (I - beta khat khat^T), whose norm is <= alpha when 0 <= beta <= 2 and
    // |khat| <= 1 (L2 norm on); no bound otherwise.
    const bool in_range = b >= 0.f && b <= 2.f && l2norm;
    const bool all_in = __ballot(!in_range) == 0;
    if (lane == 0) {
        float* gGC = reinterpret_cast<float*>(gb + S::gGC);
        gGC[0] = __expf(gl);
        gGC[1] = all_in ? gl : 1e30f;
    }
}

// Row factors f_i = beta_i rk_i^2 of L' for rows i0 .. i0 + 4n - 1 (left by prep_L).
template <int N>
__device__ __forceinline__ void row_factors(float (&f)[4 * N], const float* fr, int i0) {
#pragma unroll
    for (int q = 0; q < N; ++q) {
        const fx4 r = *reinterpret_cast<const fx4*>(fr + i0 + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[4 * q + e] = r[e];
    }
}

// Prep waves 1, 2 on chunk k: row tiles {0, 3} (half 0) or {1, 2} (half 1) of
// Pm' = diag(rq) lower(M o Q K^T) of the raw rows, computed as D = K Q^T so that a lane holds 4
// consecutive m of row i (bf16, row-major; rq_i enters as log2 rq_i in the exponent of the mask),
// and Gamma rq of those rows (rq from the diagonal of Q Q^T): the factor of the state part of O.
template <int DK, int BV, int half>
__device__ __forceinline__ void prep_P(const unsigned char* raw, const unsigned char* qv, unsigned char* sm, int lane,
                                       int len, int l2norm) {
    lane = opaque(lane);
    using S = Smem<DK, BV>;
    constexpr int KS = DK / 32;
    const __bf16* K = reinterpret_cast<const __bf16*>(raw + S::rK);
    const __bf16* Q = reinterpret_cast<const __bf16*>(qv + S::rQ);
    const float* gr = reinterpret_cast<const float*>(raw + S::rG);
    float* own = reinterpret_cast<float*>(sm + S::WP) + half * 2 * C;  // rq [C], gamma log2e [C]
    __bf16* Pm = reinterpret_cast<__bf16*>(sm + S::PM);
    float* orq = reinterpret_cast<float*>(sm + S::ORQ);
    const int g = lane / 16, l16 = lane % 16;
    constexpr int t0 = half ? 1 : 0, t1 = half ? 2 : 3;  // my row tiles

    own[C + lane] = wave_scan(gr[lane], lane) * kLog2e;
    wave_sync();  // the masks read other lanes' prefix sums

    fx4 acc[2][4], dq[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        dq[s] = zero4();
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[s][mt] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int o = off_nat<DK>(ks, g, l16);
        bf16x8 kf[4], qf[2];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            if (rb <= t1) kf[rb] = lds_at<bf16x8>(K, o + 16 * rb * DK);
        qf[0] = lds_at<bf16x8>(Q, o + 16 * t0 * DK);
        qf[1] = lds_at<bf16x8>(Q, o + 16 * t1 * DK);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int it = s ? t1 : t0;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                if (mt <= it) acc[s][mt] = mfma(kf[mt], qf[s], acc[s][mt]);
            dq[s] = mfma(qf[s], qf[s], dq[s]);
        }
    }
    write_norm(own, dq[0], t0, lane, len, l2norm);
    write_norm(own, dq[1], t1, lane, len, l2norm);
    wave_sync();  // each row's norm was written by the lane holding its diagonal element
    const float* g2 = own + C;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int it = s ? t1 : t0;
        const int i = 16 * it + l16;
        // rq_i = 0 past the tail: log2 gives -inf and the row is zero
        const float ai = g2[i] + __builtin_amdgcn_logf(own[i]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (mt > it) continue;
            const int m0 = 16 * mt + 4 * g;
            const fx4 bm = *reinterpret_cast<const fx4*>(g2 + m0);
            bf16x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float val = __builtin_amdgcn_exp2f(ai - bm[e]) * acc[s][mt][e];
                out[e] = (__bf16)((mt < it || m0 + e <= i) ? val : 0.f);
            }
            *reinterpret_cast<bf16x4*>(Pm + i * TSTR + m0) = out;
        }
    }
    if (lane / 16 == t0 || lane / 16 == t1) orq[lane] = own[lane] * __builtin_amdgcn_exp2f(g2[lane]);
}

// Solve level 0: invert the 16x16 unit-lower diagonal blocks b0, b0+1 of (I + L) by forward
// substitution, one column per lane (lanes 0..15 block b0, 16..31 block b0+1; lanes 32..63 compute
// a duplicate and discard it).  With L = diag(f) G (G strictly lower), lane j solves for
// z = T e_j - e_j, i.e. (I + L) z = -L e_j: z_m = -f_m (G_mj + sum_{i<m} G_mi z_i), which is zero
// for m <= j, so every lane runs the same steps with no select; the unit diagonal is written
// afterwards.  Each lane reads its own column of G once (row j of G^T, two 16-byte loads), which
// is also the start of its accumulators; at step m the column of lane m is broadcast within the
// 16-lane row with the DPP row broadcast (as a DPP operand of the FMA), so the substitution reads
// nothing else from LDS.  The right-looking update keeps one FMA on the critical path per step.
// Writes the blocks of T^T (bf16; column j of T = row j of T^T).
// step M: z_M is final; acc[i] += G[i][M] z_M for i > M, G[i][M] taken from lane M of the row by
// the FMA's DPP row-broadcast operand
template <int M>
__device__ __forceinline__ void fmac_bcast(float& acc, float l, float t) {  // acc += (lane M's l) * t
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(acc) : "v"(l), "v"(t), "i"(M));
}
template <int M>
__device__ __forceinline__ void solve_step(const float (&col)[16], const float (&f)[16], float (&acc)[16],
                                           float (&t)[16]) {
    const float tm = __builtin_fmaf(-f[M], acc[M], 0.f);  // + 0: a zero z_M is +0
    t[M] = tm;
#pragma unroll
    for (int i = M + 1; i < 16; ++i) fmac_bcast<M>(acc[i], col[i], tm);
}
template <int... Ms>
__device__ __forceinline__ void solve_steps(const float (&col)[16], const float (&f)[16], float (&acc)[16],
                                            float (&t)[16], std::integer_sequence<int, Ms...>) {
    (solve_step<Ms>(col, f, acc, t), ...);
}
__device__ __forceinline__ void solve_diag(const __bf16* sLt, __bf16* Tt, const float* fr, int b0, int lane) {
    lane = opaque(lane);
    const int b = b0 + (lane / 16) % 2, j = lane % 16, base = 16 * b;
    float f[16];  // row factors of the block
    row_factors<4>(f, fr, base);
    const bf16x8 c0 = *reinterpret_cast<const bf16x8*>(sLt + (base + j) * TSTR + base);
    const bf16x8 c1 = *reinterpret_cast<const bf16x8*>(sLt + (base + j) * TSTR + base + 8);
    float col[16], acc[16], t[16];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        col[e] = (float)c0[e];
        col[8 + e] = (float)c1[e];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = col[i];
    // two wait states between the VALU writes of col and its first DPP read; the operands pin the
    // writes before this point
    asm volatile("s_nop 1"
                 : "+v"(col[0]), "+v"(col[1]), "+v"(col[2]), "+v"(col[3]), "+v"(col[4]), "+v"(col[5]),
                   "+v"(col[6]), "+v"(col[7]), "+v"(col[8]), "+v"(col[9]), "+v"(col[10]), "+v"(col[11]),
                   "+v"(col[12]), "+v"(col[13]), "+v"(col[14]), "+v"(col[15]));
    solve_steps(col, f, acc, t, std::make_integer_sequence<int, 16>{});
    if (lane < 32) {
        bf16x8 lo, hi;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo[e] = (__bf16)t[e];
            hi[e] = (__bf16)t[8 + e];
        }
        __bf16* row = Tt + (base + j) * TSTR + base;
        *reinterpret_cast<bf16x8*>(row) = lo;
        *reinterpret_cast<bf16x8*>(row + 8) = hi;
        row[j] = (__bf16)1.f;  // T = I + (z columns): after the row's store, in the wave's order
    }
}

// Solve level 1: T_{b+1,b} = -T_{b+1,b+1} (L_{b+1,b} T_{b,b}) for the 16x16 block pair (b, b+1)
// (L' = diag(f) G_m: the row factor is applied to the first product).  bf16 operands (K = 16 real,
// padded to 32 with zeros).
__device__ __forceinline__ void solve_level1(const __bf16* sLt, __bf16* Tt, const float* fr, int b, int lane) {
    lane = opaque(lane);
    const int g = lane / 16, l16 = lane % 16;
    const int r0 = 16 * (b + 1), c0 = 16 * b;
    const int gg = g & 1;
    // Y = L_{b+1,b} T_bb: A = L[r0 + l16][c0 + 8gg ..] (= L^T columns, transposing read),
    // B = T_bb[c0 + 8gg ..][c0 + l16] (= T^T row c0 + l16)
    bf16x8 a = frag_tr_nat(sLt, TSTR, c0, r0, gg, l16);
    bf16x8 bt = *reinterpret_cast<const bf16x8*>(Tt + (c0 + l16) * TSTR + c0 + 8 * gg);
    if (g >= 2) {
        const bf16x8 zb = {};
        a = zb;
        bt = zb;
    }
    float f[4];
    row_factors<1>(f, fr, r0 + 4 * g);
    const fx4 y = mfma(a, bt, zero4()) * fx4{f[0], f[1], f[2], f[3]};  // rows r0 + 4g + e
    // T_{b+1,b} = -T_{b+1,b+1} Y: A = rows of T_{b+1,b+1} (chain order, k = 4g+e real), B = Y
    const bf16x4 tr = tr4(Tt, TSTR, r0 + 4 * g, r0, l16);  // T[r0 + l16][r0 + 4g .. +3]
    const bf16x4 z4 = {};
    const bf16x8 at = __builtin_shufflevector(tr, z4, 0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x8 by = pack_chain(y, zero4());
    const fx4 t = mfma(at, by, zero4());
    // lane holds T[r0 + 4g + e][c0 + l16] = -t[e] -> T^T row c0 + l16
    bf16x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (__bf16)(-t[e]);
    *reinterpret_cast<bf16x4*>(Tt + (c0 + l16) * TSTR + r0 + 4 * g) = out;
}

// Prep wave 2: L'_BA = diag(f) G_m (rows 32..63, columns 0..31) into the T_BA block of T^T, which the
// state waves read in its place (U'_B = T'_BB (Y_B - L'_BA U'_A)).  Both are stored transposed.
__device__ __forceinline__ void copy_LBA(const __bf16* sLt, __bf16* Tt, const float* fr, int lane) {
    lane = opaque(lane);
    const int m = lane / 2, c = 32 + 16 * (lane % 2);
    float f[16];
    row_factors<4>(f, fr, c);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sLt + m * TSTR + c + 8 * hf);
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (__bf16)((float)a[e] * f[8 * hf + e]);
        *reinterpret_cast<bf16x8*>(Tt + m * TSTR + c + 8 * hf) = o;
    }
}

// ------------------------------------------------------------------------------------------
// row waves: state chain and output of one chunk for 16 state rows, in registers.
// Across the barriers a row wave keeps S, the output accumulators of the chunk and U' (in the two
// operand orders the two sub-stages need); every other value is recomputed or read from LDS.
template <int DK>
struct RowRegs {
    static constexpr int DT = DK / 16, KS = DK / 32;
    fx4 S[DT];       // S^T tiles: lane (c = l%16, g) holds S[c][kcol(dt, 4g + e)]
    fx4 ot[4];       // O^T of the chunk, sub-stage A -> B
    bf16x8 ub[2];    // U' (tokens 0..31, 32..63) for the output products
    bf16x8 ut[2];    // U' diag(exp(gamma_C - gamma)) for the state update
};

// Sub-stage A: K S^T and S Q^T (S in bf16 is the same operand for both), then
// Y = beta rk V - beta Gamma rk^2 K S^T and U' = T' Y blockwise.
template <int DK, int BV, bool OUT = true>
__device__ __forceinline__ void row_A(RowRegs<DK>& st, unsigned char* sm, const unsigned char* raw,
                                      const unsigned char* qv, const unsigned char* gb, int wave, int lane) {
    lane = opaque(lane);
    using S = Smem<DK, BV>;
    constexpr int KS = DK / 32;
    const __bf16* K = reinterpret_cast<const __bf16*>(raw + S::rK);
    const __bf16* Q = reinterpret_cast<const __bf16*>(qv + S::rQ);
    const __bf16* V = reinterpret_cast<const __bf16*>(qv + S::rV);
    const __bf16* Tt = reinterpret_cast<const __bf16*>(sm + S::T);
    const float* gKK = reinterpret_cast<const float*>(gb + S::gKK);
    const float* gVB = reinterpret_cast<const float*>(gb + S::gVB);
    const float* gDR = reinterpret_cast<const float*>(gb + S::gDR);
    const int g = lane / 16, l16 = lane % 16, cbase = 16 * wave;

    // K S^T and S Q^T, k-step outer so that one k-step of K and Q fragments is live at a time
    fx4 ks_acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        ks_acc[t] = zero4();
        st.ot[t] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 sb = pack_chain(st.S[2 * ks], st.S[2 * ks + 1]);
        const int o = off_nat<DK>(ks, g, l16);
        bf16x8 kfr[4], qfr[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            kfr[t] = lds_at<bf16x8>(K, o + 16 * t * DK);
            if constexpr (OUT) qfr[t] = lds_at<bf16x8>(Q, o + 16 * t * DK);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            ks_acc[t] = mfma(kfr[t], sb, ks_acc[t]);                        // K S^T (M = token, N = c)
            if constexpr (OUT) st.ot[t] = mfma(sb, qfr[t], st.ot[t]);       // S Q^T (M = c, N = token)
        }
    }
    bf16x4 vv[4];
    fx4 bm[4], kk[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int m0 = 16 * t + 4 * g;
        vv[t] = str4<BV>(V, m0, cbase, l16);  // V[m0 .. +3][cbase + l16]
        bm[t] = *reinterpret_cast<const fx4*>(gVB + m0);
        kk[t] = *reinterpret_cast<const fx4*>(gKK + m0);
    }
    // T' blocks: T'_AA rows 0..31, L'_BA rows 32..63 (k over tokens 0..31), T'_BB rows 32..63
    const bf16x8 ta0 = frag_tr_chain(Tt, TSTR, 0, 0, g, l16), ta1 = frag_tr_chain(Tt, TSTR, 0, 16, g, l16);
    const bf16x8 la2 = frag_tr_chain(Tt, TSTR, 0, 32, g, l16), la3 = frag_tr_chain(Tt, TSTR, 0, 48, g, l16);
    const bf16x8 tb2 = frag_tr_chain(Tt, TSTR, 32, 32, g, l16), tb3 = frag_tr_chain(Tt, TSTR, 32, 48, g, l16);
    fx4 x[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[t][e] = bm[t][e] * (float)vv[t][e] - kk[t][e] * ks_acc[t][e];

    // X enters the solve as a bf16 pair (hi + lo): the value path V -> X -> U' -> O otherwise
    // rounds the rows that dominate their own outputs twice more to bf16 (each about 2^-9 of the
    // row), which with large convolved values comes close to the o tolerance
    const bf16x8 xa = pack_chain(x[0], x[1]), xal = pack_chain_lo(x[0], x[1], xa);
    fx4 u[4];
    u[0] = mfma(ta0, xal, mfma(ta0, xa, zero4()));
    u[1] = mfma(ta1, xal, mfma(ta1, xa, zero4()));
    st.ub[0] = pack_chain(u[0], u[1]);
    const fx4 y2 = mfma(la2, st.ub[0], zero4()), y3 = mfma(la3, st.ub[0], zero4());
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2][e] -= y2[e];
        x[3][e] -= y3[e];
    }
    const bf16x8 xb = pack_chain(x[2], x[3]), xbl = pack_chain_lo(x[2], x[3], xb);
    u[2] = mfma(tb2, xbl, mfma(tb2, xb, zero4()));
    u[3] = mfma(tb3, xbl, mfma(tb3, xb, zero4()));
    st.ub[1] = pack_chain(u[2], u[3]);

    fx4 ut[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const fx4 dr = *reinterpret_cast<const fx4*>(gDR + 16 * it + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) ut[it][e] = u[it][e] * dr[e];
    }
    st.ut[0] = pack_chain(ut[0], ut[1]);
    st.ut[1] = pack_chain(ut[2], ut[3]);
}

// Sub-stage B: S^T <- Gamma_C S^T + K^T diag(exp(gamma_C - gamma)) U', and
// O^T = (S Q^T) diag(Gamma rq) + U'^T Pm'^T with Pm' = diag(rq) lower(M o Q K^T) (lane: token
// 16 it + l16, state rows cbase + 4g .. +3), stored by row_store.
template <int DK, int BV, bool OUT = true>
__device__ __forceinline__ void row_B(RowRegs<DK>& st, unsigned char* sm, const unsigned char* raw,
                                      const unsigned char* gb, int lane) {
    lane = opaque(lane);
    using S = Smem<DK, BV>;
    constexpr int DT = DK / 16;
    // wide workgroups (three waves per SIMD) read K^T one token half at a time
    constexpr int NH = S::WIDE ? 1 : 2;
    const __bf16* K = reinterpret_cast<const __bf16*>(raw + S::rK);
    const __bf16* Pm = reinterpret_cast<const __bf16*>(sm + S::PM);
    const float* orq = reinterpret_cast<const float*>(sm + S::ORQ);  // Gamma rq per token
    const float gc = reinterpret_cast<const float*>(gb + S::gGC)[0];
    const int g = lane / 16, l16 = lane % 16;
    bf16x8 kt[DT][NH];
    auto read_kt = [&](int s2, int slot) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int o = off_trk<DK>(dt, g, l16) + 32 * s2 * DK;
            kt[dt][slot] = __builtin_shufflevector(tr_read(K + o), tr_read(K + o + 16 * DK), 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
#pragma unroll
    for (int s2 = 0; s2 < NH; ++s2) read_kt(s2, s2);
    bf16x8 pf[4][2];
    float r[4];
    if constexpr (OUT) {
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                if (s2 == 0 || it >= 2) pf[it][s2] = frag_chain(Pm + (16 * it + l16) * TSTR, 32 * s2, g);
#pragma unroll
        for (int it = 0; it < 4; ++it) r[it] = orq[16 * it + l16];
    }
    issue_fence();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) st.S[dt][e] *= gc;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.S[dt] = mfma(kt[dt][0], st.ut[0], st.S[dt]);
    if constexpr (NH == 1) read_kt(1, 0);
    // O^T = (S Q^T) diag(Gamma rq) + U'^T Pm'^T (rq already in Pm')
    if constexpr (OUT) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
#pragma unroll
            for (int e = 0; e < 4; ++e) st.ot[it][e] *= r[it];
            st.ot[it] = mfma(st.ub[0], pf[it][0], st.ot[it]);
            if (it >= 2) st.ot[it] = mfma(st.ub[1], pf[it][1], st.ot[it]);
        }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.S[dt] = mfma(kt[dt][NH - 1], st.ut[1], st.S[dt]);
}
// The chunk's output rows of this wave's state rows (after the wave's loads have been waited for:
// the stores would count in the same wait).
template <int DK, int BV>
__device__ __forceinline__ void row_store(const Params<DK>& p, const RowRegs<DK>& st, int wave, int lane, long t0,
                                          int len, int h, int vb) {
    lane = opaque(lane);
    const int g = lane / 16, l16 = lane % 16, cbase = 16 * wave;
    if (p.out != OUT_STORE) return;
    // Lane (g, l16) holds columns cbase + 4g .. + 3 of token 16 it + l16 in each tile.  Tiles it and
    // it + 1 trade rows of 16 lanes (v_permlane16_swap: rows 1, 3 of the first with rows 0, 2 of the
    // second), after which lane (g, l16) holds columns cbase + 8 (g / 2) .. + 7 of token
    // 16 (it + g % 2) + l16: one 16-byte store per lane and tile pair instead of two 8-byte ones.
#pragma unroll
    for (int it = 0; it < 4; it += 2) {
        bf16x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = (__bf16)(p.scale * st.ot[it][e]);
            b[e] = (__bf16)(p.scale * st.ot[it + 1][e]);
        }
        uint32_t ua[2], ub[2];
        __builtin_memcpy(ua, &a, 8);
        __builtin_memcpy(ub, &b, 8);
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const auto r = __builtin_amdgcn_permlane16_swap(ua[w], ub[w], false, false);
            ua[w] = r[0];
            ub[w] = r[1];
        }
        const int i = 16 * (it + g % 2) + l16;
        if (i < len) {
            uint4 v;
            v.x = ua[0];
            v.y = ua[1];
            v.z = ub[0];
            v.w = ub[1];
            *reinterpret_cast<uint4*>(p.o + ((size_t)(t0 + i) * p.H + h) * p.dv + vb * BV + cbase + 8 * (g / 2)) = v;
        }
    }
}

// ------------------------------------------------------------------------------------------
// Wide workgroups (dk = BV = 128: K, Q and V tiles of 16 slots of 16 bytes (8 channels) per row):
// the conv weights live in LDS as [8 channels][48 slots][4 taps] (slots 0..15 the K channels,
// 16..31 Q, 32..47 V), loaded once per workgroup and multiplied by -log2(e) (see silu_of_scaled).
// Channel-major, so that the lanes of a wave, which hold consecutive slots, read consecutive
// 16-byte words (slot-major would put the 64 lanes on a few banks).
constexpr float kNegLog2e = -1.44269504088896341f;
template <int DK, int BV>
__device__ void conv_weights_wide(const Params<DK>& p, unsigned char* sm, int tid, int h, int hk, int vb) {
    using S = Smem<DK, BV>;
    static_assert(DK == 128 && BV == 128, "wide conv layout");
    if (tid < 48 * 8) {
        const int sl = tid / 8, tile = sl / 16, c = (sl % 16) * 8 + tid % 8;  // channel within its tile
        const int row = tile == 0 ? (p.Hk + hk) * DK + c : (tile == 1 ? hk * DK + c : 2 * p.Hk * DK + h * p.dv + vb * BV + c);
        const float4 w = *reinterpret_cast<const float4*>(p.conv_w + (size_t)row * 4);
        *reinterpret_cast<float4*>(sm + S::CW + 16 * ((tid % 8) * 48 + sl)) =
            make_float4(w.x * kNegLog2e, w.y * kNegLog2e, w.z * kNegLog2e, w.w * kNegLog2e);
    }
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u128;
__device__ __forceinline__ u32x4 ld128(unsigned a) { return *reinterpret_cast<lds_u128*>(static_cast<uintptr_t>(a)); }
__device__ __forceinline__ void st128(unsigned a, u32x4 v) { *reinterpret_cast<lds_u128*>(static_cast<uintptr_t>(a)) = v; }
// SiLU(y) from t = -log2(e) y: y / (1 + e^-y) = t / (-log2(e) (1 + 2^t)), the factor folded into
// one fma (y -> -inf: 2^t = inf and the result -0; y -> +inf: 2^t = 0 and the result y).
__device__ __forceinline__ float silu_of_scaled(float t) {
    return t * __builtin_amdgcn_rcpf(__builtin_fmaf(__builtin_amdgcn_exp2f(t), kNegLog2e, kNegLog2e));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// The conv + SiLU of one chunk's tiles in a wide workgroup (the same operation as conv_chunk).
// Item = lane: 16-byte slot s (8 channels of one tile) and rows 4 rb .. 4 rb + 3.  Wave w owns
// slots 4w .. 4w + 3 (waves 0..3 the K tile, 4..7 Q, 8..11 V) in every row block: lane l takes slot
// 4w + l % 4 and block rb = l / 4.  An item reads its 4 raw rows and the 3 before them (the halo,
// for rb = 0 the previous chunk's last 3 raw rows), one 16-byte read each, then writes its 4
// results; the items of block 15 keep their raw rows 61..63 as the next chunk's halo ([3][48]
// slots of 16 bytes).  Every row an item reads but does not write belongs to an item of the same
// wave, so the wave's own ordering of its LDS accesses (all reads before any write) is enough: no
// workgroup barrier between the reads and the writes.  A 16-lane pass of the reads touches 4 rows
// 4 apart x 4 slots: 16 distinct swizzled slots, no bank conflict.  (Items of 4 channels x 8 rows
// with 8-byte accesses take fewer conversions but more LDS instructions, and measured slower.)
template <int DK, int BV>
__device__ void conv_chunk_wide(const Params<DK>& p, const unsigned char* sm, unsigned rawK, int lenK, unsigned rawQV,
                                int lenQV, unsigned halo, int parts, int tid) {
    using S = Smem<DK, BV>;
    static_assert(DK == 128 && BV == 128 && kernel_threads<BV>() == 48 * 16, "one item per lane");
    tid = opaque(tid);
    const int sl = 4 * (tid / 64) + tid % 4, rb = (tid % 64) / 4, tile = sl / 16, ts = sl % 16;
    const bool act = (parts & (tile == 0 ? 1 : 2)) && !(tile == 2 && p.v_zero);  // uniform per wave
    const unsigned base = tile == 0 ? rawK + S::rK : (tile == 1 ? rawQV + S::rQ : rawQV + S::rV);
    const int len = tile == 0 ? lenK : lenQV;
    auto at = [&](int r) { return base + 256u * r + 16u * (ts ^ (r & 15)); };  // swz<128>
    u32x4 x[7];
    if (act) {
#pragma unroll
        for (int j = 0; j < 3; ++j) x[j] = rb == 0 ? ld128(halo + 16u * (j * 48 + sl)) : ld128(at(4 * rb - 3 + j));
#pragma unroll
        for (int j = 0; j < 4; ++j) x[3 + j] = ld128(at(4 * rb + j));
    }
    wave_sync();  // every raw row this wave's items read has been read before any is written
    if (act) {
        float4 w[8];  // taps of channel c (scaled by -log2 e)
#pragma unroll
        for (int c = 0; c < 8; ++c) w[c] = *reinterpret_cast<const float4*>(sm + S::CW + 16 * (48 * c + sl));
        float lo[7][4], hi[7][4];
#pragma unroll
        for (int j = 0; j < 7; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                lo[j][q] = bf_lo(x[j][q]);
                hi[j][q] = bf_hi(x[j][q]);
            }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 a = w[2 * q], b = w[2 * q + 1];
                const float t0 = a.x * lo[r][q] + a.y * lo[r + 1][q] + a.z * lo[r + 2][q] + a.w * lo[r + 3][q];
                const float t1 = b.x * hi[r][q] + b.y * hi[r + 1][q] + b.z * hi[r + 2][q] + b.w * hi[r + 3][q];
                o[q] = pack_bf16(silu_of_scaled(t0), silu_of_scaled(t1));
            }
            if (4 * rb + r < len) st128(at(4 * rb + r), u32x4{o[0], o[1], o[2], o[3]});  // rows past the tail stay zero
        }
        if (rb == 15)
#pragma unroll
            for (int j = 0; j < 3; ++j) st128(halo + 16u * (j * 48 + sl), x[4 + j]);
    }
    lds_barrier();
}

// ------------------------------------------------------------------------------------------
// Output epilogue in a wide workgroup (page P2 section 4.2 reading: o <- o rsqrt(mean(o^2) + eps)
// (1 + w) sigmoid(z) over the dv outputs of a (token, head); a wide workgroup holds all dv = BV of
// them).  Sub-stage B: each row wave adds (scale o)^2 over its 16 rows for every token of the chunk
// and leaves the sum in LDS, while two prep waves load the chunk's z tile into the chunk's Q tile
// (read for the last time in sub-stage A); after the barrier (start of the next sub-stage A, or
// after the loop) epi_store adds the eight sums of a token and stores the gated, normalised rows.
// The Q tile of the next chunk, which shares the buffer parity with the one after it, is then
// also loaded in sub-stage B, so no load lands in a z tile before every row wave has read it.
template <int DK, int BV>
__device__ __forceinline__ void epi_sums(const Params<DK>& p, const RowRegs<DK>& st, unsigned char* sm, int wave,
                                         int lane) {
    using S = Smem<DK, BV>;
    lane = opaque(lane);
    const int g = lane / 16, l16 = lane % 16;
    float* ep = reinterpret_cast<float*>(sm + S::EP);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float o = p.scale * st.ot[it][e];
            a += o * o;
        }
        a += __shfl_xor(a, 16);
        a += __shfl_xor(a, 32);
        if (g == 0) ep[(16 * it + l16) * 8 + wave] = a;
    }
}
template <int DK, int BV>
__device__ __forceinline__ void epi_store(const Params<DK>& p, const RowRegs<DK>& st, const unsigned char* sm, int wave,
                                          int lane, long t0, int len, int h, int vb, const __bf16* zt) {
    using S = Smem<DK, BV>;
    lane = opaque(lane);
    const int g = lane / 16, l16 = lane % 16, cbase = 16 * wave;
    const float* ep = reinterpret_cast<const float*>(sm + S::EP);
    const fx4 w = *reinterpret_cast<const fx4*>(sm + S::NW + 4 * (cbase + 4 * g));
    // tiles it, it + 1 formed by every lane (rows past len too: in-bounds reads, never stored), then
    // paired as in row_store (v_permlane16_swap) for one 16-byte store per lane and tile pair
#pragma unroll
    for (int it = 0; it < 4; it += 2) {
        uint32_t u2[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = 16 * (it + u) + l16;
            const fx4 a = *reinterpret_cast<const fx4*>(ep + 8 * i), b = *reinterpret_cast<const fx4*>(ep + 8 * i + 4);
            const float ss = ((a[0] + a[1]) + (a[2] + a[3])) + ((b[0] + b[1]) + (b[2] + b[3]));
            const float rr = rsqrtf(ss * (1.f / BV) + p.norm_eps);
            const bf16x4 z = *reinterpret_cast<const bf16x4*>(zt + swz<BV>(i, cbase + 4 * g));
            bf16x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float zz = (float)z[e];
                out[e] = (__bf16)(p.scale * st.ot[it + u][e] * rr * (1.f + w[e]) * __builtin_amdgcn_rcpf(1.f + __expf(-zz)));
            }
            __builtin_memcpy(u2[u], &out, 8);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const auto r = __builtin_amdgcn_permlane16_swap(u2[0][q], u2[1][q], false, false);
            u2[0][q] = r[0];
            u2[1][q] = r[1];
        }
        const int i = 16 * (it + g % 2) + l16;
        if (i < len) {
            uint4 v;
            v.x = u2[0][0];
            v.y = u2[0][1];
            v.z = u2[1][0];
            v.w = u2[1][1];
            *reinterpret_cast<uint4*>(p.o + ((size_t)(t0 + i) * p.H + h) * p.dv + vb * BV + cbase + 8 * (g / 2)) = v;
        }
    }
}

// The conv after iteration k, once its loads have landed: narrow workgroups, chunk k+2; wide ones,
// K of chunk k+2 and Q, V of chunk k+1.
template <int DK, int BV>
__device__ __forceinline__ void conv_after(const Params<DK>& p, const ConvW<DK, BV>& cw, const unsigned char* sm,
                                           unsigned smb, int k, int len1, int len2, bool far, bool nxt, int tid) {
    using S = Smem<DK, BV>;
    if constexpr (S::WIDE) {
        if (far || nxt)
            conv_chunk_wide<DK, BV>(p, sm, smb + S::raw(k + 2), len2, smb + S::qv(k + 1), len1, smb + S::HB,
                                    (far ? 1 : 0) | (nxt ? 2 : 0), tid);
    } else {
        if (far) conv_chunk<DK, BV>(p, cw, smb + S::raw(k + 2), len2, smb + S::raw(k + 2), len2, smb + S::HB, 3, tid);
    }
}

// The sequence of rank r when sequences are ordered by length, longest first (ties: lower index
// first); called by every thread of the workgroup (it has barriers); N <= NT.  ws: N + 1 ints of LDS.
template <int NT>
__device__ int longest_first(const int32_t* cu, int N, int r, int tid, int* ws) {
    // every barrier is reached once by every wave (none sits in lane-dependent control flow)
    if (tid <= N) ws[tid] = cu[tid];
    __syncthreads();
    if (tid < N) {
        const int lm = ws[tid + 1] - ws[tid];
        int rank = 0;
        for (int j = 0; j < N; ++j) {
            const int lj = ws[j + 1] - ws[j];
            rank += (lj > lm || (lj == lm && j < tid)) ? 1 : 0;
        }
        if (rank == r) ws[N + 1] = tid;  // ranks are distinct: exactly one writer
    }
    __syncthreads();
    const int m = ws[N + 1];
    __syncthreads();  // ws is reused by the caller
    return m;
}

// exp(-27.73) = 2^-40: below this bound on the state transition since the start, whatever the
// state carried in, its remaining contribution is far under fp32 rounding.
constexpr float kExitLog = -27.7258872f;

// BYTES (a multiple of 16) from LDS byte offset `lds` to global dst, by thread t of NTH, 16 bytes
// at a time (a rolled loop: it sits inside the chunk loop, whose registers it must not take).
template <int BYTES, int NTH>
__device__ __forceinline__ void keep_to_global(const unsigned char* sm, int lds, unsigned char* dst, int t) {
#pragma unroll 1
    for (int i = t; i < BYTES / 16; i += NTH)
        *reinterpret_cast<u32x4*>(dst + 16 * i) = *reinterpret_cast<const u32x4*>(sm + lds + 16 * i);
}

// E_j = E_{j-1} A_j + B_j for j = j0+1 .. j1 (E_{j0} = B_{j0}, or E_{j1} = B_{j1} when A_{j1} is
// negligible), rows [vb BV, +BV) of sequence n, head h, in fp32: E in the row waves' registers in
// the state-tile layout, A_j staged transposed in LDS by every wave, the product on the fp32 MFMA
// (16x16x4) as D^T = A_j^T E^T so that D lands in the same layout.  E_{mid} (mid < j1, if mid >= j0)
// is stored to dmid and E_{j1} to dend (row blocks [BV][DK], either may be null).  Every thread of
// the workgroup calls this (it has barriers); it uses all of LDS.
template <int DK, int BV>
__device__ void chain_states(const Params<DK>& p, unsigned char* sm, int n, int h, int vb, int j0, int j1, int mid,
                             float* dmid, float* dend, int tid) {
    constexpr int DT = DK / 16, NT = kernel_threads<BV>(), ATS = DK + 4;  // At row stride (floats)
    static_assert(DK * ATS * 4 <= 160 * 1024, "A_j^T in LDS");
    const int wid = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64, g = lane / 16, l16 = lane % 16;
    const bool is_row = wid < BV / 16;
    const int row = vb * BV + 16 * wid + l16;
    float* At = reinterpret_cast<float*>(sm);
    auto slot = [&](int j) { return (size_t)(n * p.P + j) * p.H + h; };
    auto ld_rows = [&](const float* base, fx4 (&x)[DT]) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const float4 v = *reinterpret_cast<const float4*>(base + (size_t)row * DK + kcol(dt, 4 * g));
            x[dt] = fx4{v.x, v.y, v.z, v.w};
        }
    };
    auto st_rows = [&](float* base, const fx4 (&x)[DT]) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<float4*>(base + (size_t)row * DK + kcol(dt, 4 * g)) = make_float4(x[dt][0], x[dt][1], x[dt][2], x[dt][3]);
    };
    // B_j (B_{P-1} is in the final state's place, see Params::fin)
    auto bj = [&](int j) {
        return p.fin && !p.fin_in_slot && j == p.P - 1 ? p.fin + ((size_t)n * p.H + h) * p.dv * DK
                                                         : p.s0 + slot(j) * p.dv * DK;
    };
    fx4 E[DT];
    int lazy = j0;  // E_lazy = B_lazy, not yet loaded (-1: E is in the registers)
    auto held = [&]() {
        if (lazy >= 0 && is_row) ld_rows(bj(lazy), E);
        lazy = -1;
    };
    if (dmid && mid == j0) {
        held();
        if (is_row) st_rows(dmid, E);
    }
    for (int j = j0 + 1; j <= j1; ++j) {
        const float* Bj = bj(j);
        if (mark_negligible(p.marks[slot(j)])) {  // A_j negligible
            lazy = j;
        } else {
            held();
            const float* Aj = p.trans + slot(j) * DK * DK;
            lds_barrier();  // the previous product's reads of At are done
            for (int i = tid; i < DK * DK / 4; i += NT) {
                const float4 v = *reinterpret_cast<const float4*>(Aj + 4 * i);
                const int r = 4 * i / DK, c = 4 * i % DK;
                At[(c + 0) * ATS + r] = v.x;
                At[(c + 1) * ATS + r] = v.y;
                At[(c + 2) * ATS + r] = v.z;
                At[(c + 3) * ATS + r] = v.w;
            }
            lds_barrier();
            if (is_row) {
                fx4 acc[DT];
                ld_rows(Bj, acc);
#pragma unroll
                for (int dp = 0; dp < DT; ++dp)
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        // lane (m = l16, k = g): A_j[kcol(dp, 4g + e)][kcol(dt, m)], e = 0..3
                        const fx4 a = *reinterpret_cast<const fx4*>(At + kcol(dt, l16) * ATS + kcol(dp, 4 * g));
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], E[dp][e], acc[dt], 0, 0, 0);
                    }
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) E[dt] = acc[dt];
            }
        }
        if (dmid && j == mid) {
            held();
            if (is_row) st_rows(dmid, E);
        }
    }
    if (dend) {
        held();
        if (is_row) st_rows(dend, E);
    }
    lds_barrier();  // LDS is free again
}


// Spin bound of wait_transitions: each poll sleeps ~1,000 clocks, so about 10-20 s in all.
constexpr unsigned kWaitSpins = 1u << 23;

// A rerun in the launch of the transitions (Params::tr_wait) waits for the transitions A_j, j <= j1,
// that its entering state may need: each is formed by the workgroup of segment j's pair, whose
// block index lies below this one's (same head, earlier segment), before that workgroup waits for
// anything (at most the one-chunk rerun, which never waits, comes first).  The workgroups of a
// launch start in index order on each XCD, so every transition that a rerun waits for runs to its
// end.  Wave 0 polls the marks (lane j - 1 that of segment j) until each is 1 (negligible by the
// first pass: no transition runs) or at least tr_wait (every workgroup of its transition has
// counted itself), then its acquire fence invalidates the caches that could hold stale lines of the
// transitions; the verdict goes to the other waves through LDS word 0, so that all take the same
// path.  False if a mark did not get there within the spin bound.  Called by every thread, with
// LDS free.
template <int DK>
__device__ bool wait_transitions(const Params<DK>& p, unsigned char* sm, int n, int h, int j1, int tid) {
    int* verdict = reinterpret_cast<int*>(sm);
    if (tid < 64) {
        bool late = false;
        for (int j = 1 + tid; j <= j1; j += 64) {
            int* m = const_cast<int*>(p.marks) + (size_t)(n * p.P + j) * p.H + h;
            for (unsigned spin = 0;; ++spin) {
                const int v = __hip_atomic_load(m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v == 1 || v >= p.tr_wait) break;
                if (spin >= kWaitSpins) {
                    late = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(16);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        const bool ok = __ballot(late) == 0;
        if (tid == 0) *verdict = ok ? 1 : 0;
    }
    lds_barrier();
    const bool ok = *reinterpret_cast<volatile int*>(verdict) != 0;
    lds_barrier();  // LDS free again
    return ok;
}

// A rerun whose wait ran out: NaN in its outputs (and the final state's rows, for the last
// segment) instead of a result formed from unfinished transitions.
template <int DK, int BV>
__device__ void poison_segment(const Params<DK>& p, int n, int h, int vb, long bos, long eos, bool last, int tid) {
    constexpr int NT = kernel_threads<BV>();
    const __bf16 qnan = __builtin_bit_cast(__bf16, (unsigned short)0x7fc0);
    for (long i = tid; i < (eos - bos) * BV; i += NT)
        p.o[((bos + i / BV) * p.H + h) * p.dv + vb * BV + i % BV] = qnan;
    if (last)
        for (int i = tid; i < BV * DK; i += NT)
            p.fin[((size_t)n * p.H + h) * p.dv * DK + (size_t)vb * BV * DK + i] = __builtin_nanf("");
}

// Rerun of segment p >= 1 when the bound on the transition of its first chunk is already below
// 2^-40: from the state entering the segment (E_{p-1}, rows at ein), only that chunk's outputs change,
// and the first pass's o stands after it.  The chunk's prepared operands (T', Pm, rq, the gates)
// are the ones the first pass formed from the same tokens, kept in the workspace, so nothing is
// prepared here: one load phase (state, K, Q, V, the kept operands; z for the epilogue), then the
// row waves' two sub-stages on the chunk.  go() (uniform) is asked once the loads are in flight:
// false drops them (waited for, so that LDS is free again) and returns false.
template <int DK, int BV, bool EPI, typename Go>
__device__ bool rerun_first_chunk(const Params<DK>& p, unsigned char* sm, const unsigned char* kept, long bos, int len,
                                  int h, int hk, int vb, const float* ein, int tid, Go go) {
    using S = Smem<DK, BV>;
    constexpr bool WIDE = S::WIDE;
    constexpr int NT = kernel_threads<BV>(), PW0 = NT / 64 - 4;
    const int wid = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, g = lane / 16, l16 = lane % 16;
    const bool is_row = wid < BV / 16, is_prep = wid >= PW0;
    const int pw = wid - PW0;
    const unsigned smb = lds_base(sm);
    RowRegs<DK> st;
    if (is_row) {
        const float* src = ein + (size_t)(vb * BV + 16 * wid + l16) * DK;
#pragma unroll
        for (int dt = 0; dt < RowRegs<DK>::DT; ++dt) {
            const float4 v = *reinterpret_cast<const float4*>(src + kcol(dt, 4 * g));
            st.S[dt] = fx4{v.x, v.y, v.z, v.w};
        }
    }
    if constexpr (WIDE) {
        if (is_prep) {
            dma_k<DK, 16>(p, smb + S::raw(0) + S::rK, bos, len, hk, 16 * pw, lane);
            // z of the epilogue into the spare Q/V buffer
            if (EPI && pw >= 2) dma_z<DK, BV, 32>(p, smb + S::qv(1) + S::rQ, bos, len, h, vb, 32 * (pw - 2), lane);
        }
        if (is_row) {
            dma_q<DK, 8>(p, smb + S::qv(0) + S::rQ, bos, len, hk, 8 * wid, lane);
            dma_v<DK, BV, 8>(p, smb + S::qv(0) + S::rV, bos, len, h, vb, 8 * wid, lane);
        }
    } else if (is_prep) {
        dma_chunk<DK, BV>(p, smb, S::raw(0), bos, len, h, hk, vb, pw, lane);
    }
    if constexpr (EPI)
        if (tid < BV) reinterpret_cast<float*>(sm + S::NW)[tid] = p.norm_weight[vb * BV + tid];
    // the kept operands, by plain loads
    constexpr int NU = PRE_BYTES / 16, IT = (NU + NT - 1) / NT;
    u32x4 kv[IT];
#pragma unroll
    for (int j = 0; j < IT; ++j)
        if (tid + j * NT < NU) kv[j] = *reinterpret_cast<const u32x4*>(kept + 16 * (tid + j * NT));
    if (!go()) {
        wait_loads();
        lds_barrier();
        return false;
    }
#pragma unroll
    for (int j = 0; j < IT; ++j) {
        const int b = 16 * (tid + j * NT);
        if (b < PRE_BYTES) {
            const int dst = b < PRE_PM ? S::T + b
                                       : (b < PRE_RQ ? S::PM + (b - PRE_PM)
                                                     : (b < PRE_G ? S::ORQ + (b - PRE_RQ) : S::gates(0) + (b - PRE_G)));
            *reinterpret_cast<u32x4*>(sm + dst) = kv[j];
        }
    }
    wait_loads();
    if (len < C) {
        if constexpr (WIDE) {
            if (is_prep) zero_rows<DK, 16>(reinterpret_cast<__bf16*>(sm + S::raw(0) + S::rK), len, 16 * pw, opaque(lane));
            if (is_row) {
                zero_rows<DK, 8>(reinterpret_cast<__bf16*>(sm + S::qv(0) + S::rQ), len, 8 * wid, opaque(lane));
                zero_rows<BV, 8>(reinterpret_cast<__bf16*>(sm + S::qv(0) + S::rV), len, 8 * wid, opaque(lane));
            }
        } else if (is_prep) {
            zero_tail<DK, BV>(sm + S::raw(0), len, pw, lane);
        }
    }
    lds_barrier();
    if (is_row) {
        row_A<DK, BV>(st, sm, sm + S::raw(0), sm + S::qv(0), sm + S::gates(0), wid, lane);
        row_B<DK, BV>(st, sm, sm + S::raw(0), sm + S::gates(0), lane);
        if constexpr (EPI)
            epi_sums<DK, BV>(p, st, sm, wid, lane);
        else
            row_store<DK, BV>(p, st, wid, lane, bos, len, h, vb);
    }
    if constexpr (EPI) {
        lds_barrier();
        if (is_row)
            epi_store<DK, BV>(p, st, sm, wid, lane, bos, len, h, vb,
                              reinterpret_cast<const __bf16*>(sm + S::qv(1) + S::rQ));
    }
    return true;
}

// BV: state rows of the workgroup: BV / 16 row waves.  Narrow (BV = 64, or 32 for a 32-row
// state): 8 waves, waves 2 and 3 load the chunks, waves 4..7 prepare them.  Wide (BV = 128): 12
// waves, every row wave loads an eighth of each chunk, waves 8..11 prepare them; the preparation of
// a chunk (L, T, Pm, the gates) is shared by all 128 rows.
// RAW: g and beta hold the raw gate inputs (a separate instantiation, so that the plain one carries
// no trace of the gate transform).  EPI: the output epilogue.  LEAN: without the rerun pass's code
// (entering states, the one-chunk rerun); the first and transition passes without the epilogue
// run this one: the chunk loop schedules better without that code beside it.
// What chunk_body runs of a rerun (Params::init = INIT_PREV) and what it reports: BODY_FAST tries
// only the one-chunk rerun of the usual case, BODY_REST skips that attempt; the result has BODY_DONE
// once the segment's outputs are final, and BODY_TRANS where the pair's own transition may still
// be needed (the transition pass itself decides).
enum BodyPhase { BODY_ALL = 0, BODY_FAST = 1, BODY_REST = 2 };
enum BodyResult { BODY_DONE = 1, BODY_TRANS = 2 };

template <int DK, int BV, bool RAW, bool EPI, bool LEAN, bool TRANS>
__device__ __forceinline__ int chunk_body(const Params<DK>& p, const int b, const int phase = BODY_ALL) {
    using S = Smem<DK, BV>;
    // TRANS: the transition pass (no output): nothing of Q, Pm' or O is formed
    constexpr bool OUT = !TRANS;
    constexpr bool WIDE = S::WIDE;
    static_assert(!EPI || WIDE, "the fused output epilogue needs the whole row of a head");
    constexpr int NT = kernel_threads<BV>(), PW0 = NT / 64 - 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
    const int tid = threadIdx.x;
    const int wid = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;
    const int g = lane / 16, l16 = lane % 16;
    const bool is_row = wid < BV / 16, is_load = !WIDE && (wid == 2 || wid == 3), is_prep = wid >= PW0;
    const int pw = wid - PW0;  // prep wave index

    // XCD-aware order: the grp * nv workgroups that read one (segment, query/key head) -- its
    // value heads times their row blocks -- share blockIdx mod 8 (same XCD, same L2) when the
    // group count allows it.
    const int ngroups = p.N * p.P * p.Hk, wpg = p.grp * p.nv;
    int group, within;
    if (ngroups % 8 == 0) {
        group = (b / (8 * wpg)) * 8 + b % 8;
        within = (b / 8) % wpg;
    } else {
        group = b / wpg;
        within = b % wpg;
    }
    const int vb = within % p.nv;
    int pair = group * p.grp + within / p.nv;  // (segment, value head)
    const int h = pair % p.H, hk = h / p.grp;
    int n = pair / p.H / p.P;
    const int seg = pair / p.H % p.P;
    if (p.P == 1 && p.cu && p.N <= NT) {
        // Packed sequences of unequal lengths in one pass: the workgroups that start first (low
        // block index) take the longest sequences, so no long sequence starts last.
        n = longest_first<NT>(p.cu, p.N, n, tid, reinterpret_cast<int*>(sm + S::T));
        pair = n * p.H + h;
    }
    const int nseg = pair / p.H;
    if (p.skip_first && seg == 0) return BODY_DONE;
    if (p.negl_mode == NEGL_SKIP && p.negl[pair]) return BODY_DONE;  // the segment's transition is negligible
    long bos, eos;
    if (p.cu) {
        bos = p.cu[n];
        eos = p.cu[n + 1];
    } else {
        const long Ls = p.T_tot / p.N;
        bos = (long)n * Ls;
        eos = bos + Ls;
    }
    if (p.P > 1) {  // segment seg: ceil(chunks / P) whole chunks of the sequence
        const long per = (((eos - bos + C - 1) / C + p.P - 1) / p.P) * C;
        const long sb = min(eos, bos + seg * per);
        eos = min(eos, sb + per);
        bos = sb;
    }
    const int nchunks = (int)((eos - bos + C - 1) / C);
    auto clen = [&](int c) { return (int)min((long)C, eos - (bos + (long)c * C)); };
    // The state entering this segment (rerun: [rows][DK] block): E_{seg-1} = E_{seg-2} A_{seg-1} +
    // B_{seg-1}, E_0 = B_0, and E_j = B_j where A_j is negligible -- B_{seg-1} itself in the usual
    // case, else chained here from the last negligible link.  The last segment's workgroups also
    // form the final state E_{P-1}.
    // The last segment's workgroups chain the final state E_{P-1} over B_{P-1} where A_{P-1} is not
    // negligible.
    const float* ein = p.s0 + (size_t)((nseg - 1) * p.H + h) * p.dv * DK;
    const bool fast_ok = !LEAN && p.pre_mode == PRE_USE && seg > 0 && nchunks > 0 && p.early_exit && !p.conv_w;
    const unsigned char* kept = p.pre + (size_t)pair * PRE_BYTES;
    auto kept_bound = [&]() {  // the bound of the first chunk's transition, from the kept gates
        return __builtin_bit_cast(
            float, __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(kept + PRE_G + S::gGC + 4)));
    };
    if constexpr (!LEAN) {
        // The usual case, taken on trust while its loads are in flight: E_{seg-1} = B_{seg-1} in
        // place, no final state to chain, and the first chunk reaches the bound.
        if (phase != BODY_REST && fast_ok && p.marks) {
            bool own_negl = false;  // this segment's own transition negligible by the first pass
            auto usual = [&]() {
                own_negl = mark_negligible(p.marks[pair]);
                const bool mprev = mark_negligible(p.marks[(size_t)(n * p.P + seg - 1) * p.H + h]);
                const bool mlast = p.fin && seg == p.P - 1 ? (!p.fin_in_slot && mark_negligible(p.marks[pair])) : true;
                const float b0 = kept_bound();
                return (seg == 1 || mprev) && mlast && b0 <= kExitLog;
            };
            if (rerun_first_chunk<DK, BV, EPI>(p, sm, kept, bos, clen(0), h, hk, vb, ein, tid, usual))
                return BODY_DONE | (own_negl ? 0 : BODY_TRANS);
        }
        if (phase == BODY_FAST) return BODY_TRANS;
    }
    if (!LEAN && p.marks && seg > 0) {
        // the loads this choice needs, issued together
        const bool last = p.fin && seg == p.P - 1;
        if (p.tr_wait && !wait_transitions<DK>(p, sm, n, h, last ? seg : seg - 1, tid)) {
            poison_segment<DK, BV>(p, n, h, vb, bos, eos, last, tid);
            return BODY_DONE;
        }
        const bool mprev = mark_negligible(p.marks[(size_t)(n * p.P + seg - 1) * p.H + h]);
        const bool mlast = last ? (!p.fin_in_slot && mark_negligible(p.marks[pair])) : true;
        int j0 = seg - 1;
        if (j0 > 0 && !mprev)
            do --j0;
            while (j0 > 0 && !mark_negligible(p.marks[(size_t)(n * p.P + j0) * p.H + h]));
        const bool fin = !mlast;  // else B_{P-1}, in place, is the final state
        // (with fin_in_slot the chain to the final state runs even where A_{P-1} is negligible:
        // it then copies B_{P-1} from its slot)
        if (j0 < seg - 1 || fin) {
            float* own = p.ein + (size_t)pair * p.dv * DK;
            if constexpr (!LEAN)
                chain_states<DK, BV>(p, sm, n, h, vb, j0, fin ? seg : seg - 1, seg - 1, j0 < seg - 1 ? own : nullptr,
                                     fin ? p.fin + ((size_t)n * p.H + h) * p.dv * DK : nullptr, tid);
            if (j0 < seg - 1) ein = own;
        }
    }
    if (fast_ok && kept_bound() <= kExitLog) {
        if constexpr (!LEAN) rerun_first_chunk<DK, BV, EPI>(p, sm, kept, bos, clen(0), h, hk, vb, ein, tid, [] { return true; });
        return BODY_DONE;
    }
    // the first pass keeps its first chunk's prepared operands for the rerun (one copy per head)
    const bool keep = p.pre_mode == PRE_KEEP && seg > 0 && vb == 0;

    // T^T blocks above the diagonal blocks and Pm tiles above the diagonal are read as zeros but
    // never written: clear both once.  Zero values: clear V in every buffer that holds it.
    for (int i = tid; i < C * TSTR; i += NT) {
        reinterpret_cast<__bf16*>(sm + S::T)[i] = (__bf16)0.f;
        reinterpret_cast<__bf16*>(sm + S::PM)[i] = (__bf16)0.f;
    }
    if (p.v_zero) {
        for (int i = tid; i < C * BV; i += NT)
#pragma unroll
            for (int r = 0; r < (WIDE ? 2 : 3); ++r) reinterpret_cast<__bf16*>(sm + S::qv(r) + S::rV)[i] = (__bf16)0.f;
    }

    const unsigned smb = lds_base(sm);
    const bool conv = p.conv_w != nullptr;
    ConvW<DK, BV> cw;  // narrow: the weights of the lane's items (wide: in LDS)
    if (conv) {
        if constexpr (WIDE)
            conv_weights_wide<DK, BV>(p, sm, tid, h, hk, vb);
        else
            conv_weights<DK, BV>(cw, p, tid, h, hk, vb);
        const int from = seg > 0 ? (nchunks > 0 ? HALO_TOKENS : HALO_ZERO) : (p.conv_state ? HALO_STATE : HALO_ZERO);
        conv_halo_init<DK, BV>(p, smb + S::HB, tid, n, h, hk, vb, bos, from);
    }
    if constexpr (EPI)
        if (tid < BV) reinterpret_cast<float*>(sm + S::NW)[tid] = p.norm_weight[vb * BV + tid];
    // chunk 0 (wide: its K, g and beta, and without the epilogue its Q and V; with the epilogue
    // Q and V come with the first iteration's loads)
    if (nchunks > 0 && is_prep) {
        if constexpr (WIDE) {
            dma_k<DK, 16>(p, smb + S::raw(0) + S::rK, bos, clen(0), hk, 16 * pw, lane);
            if (pw < 2) dma_gates_in<DK>(p, smb + S::raw(0) + (pw == 0 ? S::rG : S::rB), bos, clen(0), h, pw, lane);
            if constexpr (!EPI) {
                if constexpr (OUT) dma_q<DK, 16>(p, smb + S::qv(0) + S::rQ, bos, clen(0), hk, 16 * pw, lane);
                if (!p.v_zero) dma_v<DK, BV, 16>(p, smb + S::qv(0) + S::rV, bos, clen(0), h, vb, 16 * pw, lane);
            }
            wait_loads();
            if constexpr (RAW) raw_gates<DK, BV>(p, sm + S::raw(0), clen(0), pw, lane, h);
            if (clen(0) < C) {
                zero_rows<DK, 16>(reinterpret_cast<__bf16*>(sm + S::raw(0) + S::rK), clen(0), 16 * pw, opaque(lane));
                if (pw < 2 && lane >= clen(0)) reinterpret_cast<float*>(sm + S::raw(0) + (pw == 0 ? S::rG : S::rB))[lane] = 0.f;
                if constexpr (!EPI) {
                    zero_rows<DK, 16>(reinterpret_cast<__bf16*>(sm + S::qv(0) + S::rQ), clen(0), 16 * pw, opaque(lane));
                    zero_rows<BV, 16>(reinterpret_cast<__bf16*>(sm + S::qv(0) + S::rV), clen(0), 16 * pw, opaque(lane));
                }
            }
        } else {
            dma_chunk<DK, BV>(p, smb, S::raw(0), bos, clen(0), h, hk, vb, pw, lane);
            wait_loads();
            if constexpr (RAW) raw_gates<DK, BV>(p, sm + S::raw(0), clen(0), pw, lane, h);
            zero_tail<DK, BV>(sm + S::raw(0), clen(0), pw, lane);
        }
    }
    lds_barrier();
    // conv of chunk 0 (wide: its K; Q and V with the first iteration's conv)
    if (conv && nchunks > 0) {
        if constexpr (WIDE)
            conv_chunk_wide<DK, BV>(p, sm, smb + S::raw(0), clen(0), smb + S::raw(0), clen(0), smb + S::HB, 1, tid);
        else
            conv_chunk<DK, BV>(p, cw, smb + S::raw(0), clen(0), smb + S::raw(0), clen(0), smb + S::HB, 3, tid);
    }

    // Iteration k: state and output on chunk k, Pm of chunk k, L and T of chunk k+1, loads of k+2
    // (wide: K, g, beta of k+2 and Q, V of k+1).  The row/load waves and the prep waves run separate copies of the loop with the same barrier
    // sequence, so that each role's registers are allocated for its own code only.  Every wave
    // reads the same transition bounds in the same order, so an early exit is uniform.
    float decay = 0.f;  // log bound of the transition over the chunks the state has passed
    auto bound = [&](int k) {
        if (p.early_exit || p.negl_mode == NEGL_MARK)
            decay += __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(
                                                   int, reinterpret_cast<const float*>(sm + S::gates(k) + S::gGC)[1])));
    };
    int stopped = 0;  // the chain stopped at the decay bound (row waves)
    if (!is_prep) {
        RowRegs<DK> st;
        const int row = vb * BV + 16 * wid + l16;  // state row of this lane (row waves)
        if (is_row) {
            const float* src = nullptr;
            if (p.init == INIT_S0 && p.s0 && seg == 0)
                src = p.s0 + (((size_t)n * p.H + h) * p.dv + row) * DK;
            else if (p.init == INIT_PREV)
                src = ein + (size_t)row * DK;
#pragma unroll
            for (int dt = 0; dt < RowRegs<DK>::DT; ++dt) {
                if (src) {
                    const float4 v = *reinterpret_cast<const float4*>(src + kcol(dt, 4 * g));
                    st.S[dt] = fx4{v.x, v.y, v.z, v.w};
                } else if (p.init == INIT_IDENTITY) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) st.S[dt][e] = (kcol(dt, 4 * g + e) == row) ? 1.f : 0.f;
                } else {
                    st.S[dt] = zero4();
                }
            }
        }
        int pend = -1;  // epilogue: the chunk whose outputs st.ot holds, stored after the next barrier
        for (int k = -1; k < nchunks; ++k) {
            const bool cur = k >= 0, nxt = k + 1 < nchunks, far = k + 2 < nchunks;
            const long tk = bos + (long)k * C;
            // ---- A
            if constexpr (EPI) {
                if (pend >= 0)
                    epi_store<DK, BV>(p, st, sm, wid, lane, bos + (long)pend * C, clen(pend), h, vb,
                                      reinterpret_cast<const __bf16*>(sm + S::qv(pend) + S::rQ));
                pend = -1;
            }
            if (cur && is_row) row_A<DK, BV, OUT>(st, sm, sm + S::raw(k), sm + S::qv(k), sm + S::gates(k), wid, lane);
            if constexpr (WIDE && !EPI) {
                // rows [16w, 16w + 16) of K of chunk k+2 (with g, beta: waves 0, 1), on waves 0..3,
                // which finish their row work first.  K's buffer held chunk k-1 (last read in the
                // previous sub-stage B).  Q and V come from the prep waves, a chunk further ahead.
                if (far && wid < 4) {
                    dma_k<DK, 16>(p, smb + S::raw(k + 2) + S::rK, tk + 2 * C, clen(k + 2), hk, 16 * wid, lane);
                    if (wid < 2)
                        dma_gates_in<DK>(p, smb + S::raw(k + 2) + (wid == 0 ? S::rG : S::rB), tk + 2 * C, clen(k + 2), h,
                                         wid, lane);
                }
            } else if constexpr (WIDE) {
                // rows [8w, 8w + 8) of K of chunk k+2 (with g, beta: waves 0, 1) and of V of chunk
                // k+1.  K's buffer held chunk k-1 (last read in the previous sub-stage B), the Q/V
                // buffer chunk k-1 (last read in the previous sub-stage A; its Q tile then held z).
                if (far) {
                    dma_k<DK, 8>(p, smb + S::raw(k + 2) + S::rK, tk + 2 * C, clen(k + 2), hk, 8 * wid, lane);
                    if (wid < 2)
                        dma_gates_in<DK>(p, smb + S::raw(k + 2) + (wid == 0 ? S::rG : S::rB), tk + 2 * C, clen(k + 2), h,
                                         wid, lane);
                }
                if (nxt && !p.v_zero)
                    dma_v<DK, BV, 8>(p, smb + S::qv(k + 1) + S::rV, tk + C, clen(k + 1), h, vb, 8 * wid, lane);
            } else if (far && is_load) {
                // the loads of chunk k+2 from waves 2 and 3 (rows 32 (w - 2) .. + 31), after their row
                // work: waves 0 and 1 share their SIMDs with the solve of the next sub-stage and wait
                // for nothing.  The buffer held chunk k-1, whose last reads were before the previous
                // barrier.
                dma_chunk<DK, BV>(p, smb, S::raw(k + 2), tk + 2 * C, clen(k + 2), h, hk, vb, 2 * (wid - 2), lane);
                dma_chunk<DK, BV>(p, smb, S::raw(k + 2), tk + 2 * C, clen(k + 2), h, hk, vb, 2 * (wid - 2) + 1, lane);
            }
            lds_barrier();
            // ---- B
            if (cur) {
                if (is_row) {
                    row_B<DK, BV, OUT>(st, sm, sm + S::raw(k), sm + S::gates(k), lane);
                    if constexpr (EPI) epi_sums<DK, BV>(p, st, sm, wid, lane);
                }
                bound(k);
            }
            if constexpr (WIDE && !EPI) {
                if (far && wid < 4) {
                    wait_loads();
                    if (RAW && wid < 2) raw_gates<DK, BV>(p, sm + S::raw(k + 2), clen(k + 2), wid, lane, h);
                    if (clen(k + 2) < C) {
                        zero_rows<DK, 16>(reinterpret_cast<__bf16*>(sm + S::raw(k + 2) + S::rK), clen(k + 2), 16 * wid,
                                          opaque(lane));
                        if (wid < 2 && lane >= clen(k + 2))
                            reinterpret_cast<float*>(sm + S::raw(k + 2) + (wid == 0 ? S::rG : S::rB))[lane] = 0.f;
                    }
                }
            } else if constexpr (WIDE) {
                if (far || nxt) {
                    wait_loads();
                    if (far) {
                        if (RAW && wid < 2) raw_gates<DK, BV>(p, sm + S::raw(k + 2), clen(k + 2), wid, lane, h);
                        if (clen(k + 2) < C) {
                            zero_rows<DK, 8>(reinterpret_cast<__bf16*>(sm + S::raw(k + 2) + S::rK), clen(k + 2), 8 * wid,
                                             opaque(lane));
                            if (wid < 2 && lane >= clen(k + 2))
                                reinterpret_cast<float*>(sm + S::raw(k + 2) + (wid == 0 ? S::rG : S::rB))[lane] = 0.f;
                        }
                    }
                    if (nxt && clen(k + 1) < C)
                        zero_rows<BV, 8>(reinterpret_cast<__bf16*>(sm + S::qv(k + 1) + S::rV), clen(k + 1), 8 * wid,
                                         opaque(lane));
                }
            } else if (far && is_load) {
                wait_loads();
                if (RAW && wid == 2) {
                    raw_gates<DK, BV>(p, sm + S::raw(k + 2), clen(k + 2), 0, lane, h);
                    raw_gates<DK, BV>(p, sm + S::raw(k + 2), clen(k + 2), 1, lane, h);
                }
                zero_tail<DK, BV>(sm + S::raw(k + 2), clen(k + 2), 2 * (wid - 2), lane);
                zero_tail<DK, BV>(sm + S::raw(k + 2), clen(k + 2), 2 * (wid - 2) + 1, lane);
            }
            if (cur && is_row) {
                if constexpr (EPI)
                    pend = k;
                else
                    row_store<DK, BV>(p, st, wid, lane, tk, clen(k), h, vb);
            }
            lds_barrier();
            if (p.early_exit && decay <= kExitLog) {
                stopped = 1;
                break;
            }
            // ---- C (conv only): the prologue on the chunks whose loads landed in this iteration
            if (conv) conv_after<DK, BV>(p, cw, sm, smb, k, clen(k + 1), clen(k + 2), far, nxt, tid);
        }
        if constexpr (EPI)
            if (pend >= 0)
                epi_store<DK, BV>(p, st, sm, wid, lane, bos + (long)pend * C, clen(pend), h, vb,
                                  reinterpret_cast<const __bf16*>(sm + S::qv(pend) + S::rQ));
        if (is_row && p.sfin) {
            // first pass, last segment: B_{P-1} into the final state (see Params::fin)
            float* dst = (p.fin && !p.fin_in_slot && seg == p.P - 1 ? p.fin + ((size_t)n * p.H + h) * p.dv * DK
                                                  : p.sfin + (size_t)pair * p.dv * DK) +
                         (size_t)row * DK;
#pragma unroll
            for (int dt = 0; dt < RowRegs<DK>::DT; ++dt) {
                const fx4 v = st.S[dt];
                *reinterpret_cast<float4*>(dst + kcol(dt, 4 * g)) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
        if (p.negl && vb == 0 && tid == 0 && !p.tr_signal)
            p.negl[pair] = p.negl_mode == NEGL_MARK ? (decay <= kExitLog) : stopped;
        // this wave's stores of A_j have reached L2 (vmcnt counts stores) before the workgroup
        // counts itself; the count's release then writes L2 back once for the whole workgroup
        if (p.tr_signal) wait_loads();
    } else {
        for (int k = -1; k < nchunks; ++k) {
            const bool cur = k >= 0, nxt = k + 1 < nchunks, far = k + 2 < nchunks;
            const long tk = bos + (long)k * C;
            // ---- A
            // the prep waves end sub-stage A last (each shares its SIMD with two row waves, which
            // reach the barrier early): their instructions go first until the barrier
            __builtin_amdgcn_s_setprio(1);
            if (cur && OUT) {
                unsigned char* rawk = sm + S::raw(k);
                if (pw == 1) prep_P<DK, BV, 0>(rawk, sm + S::qv(k), sm, lane, clen(k), p.l2norm);
                if (pw == 2) prep_P<DK, BV, 1>(rawk, sm + S::qv(k), sm, lane, clen(k), p.l2norm);
            }
            if (nxt && pw == 0) prep_L<DK, BV, 0>(sm + S::raw(k + 1), sm, lane, clen(k + 1), p.l2norm);
            if (nxt && pw == 3) prep_L<DK, BV, 1>(sm + S::raw(k + 1), sm, lane, clen(k + 1), p.l2norm);
            // T' and the gates of chunk 0, complete since the previous barrier (T' is rewritten in
            // this iteration's sub-stage B)
            if (keep && k == 0 && pw < 2) {
                unsigned char* kd = p.pre + (size_t)pair * PRE_BYTES;
                keep_to_global<C * TSTR * 2, 128>(sm, S::T, kd + PRE_T, tid - 64 * PW0);
                keep_to_global<Smem<DK, BV>::gBytes, 128>(sm, S::gates(0), kd + PRE_G, tid - 64 * PW0);
            }
            __builtin_amdgcn_s_setprio(0);
            lds_barrier();
            // ---- B
            if (cur) bound(k);
            if constexpr (WIDE && !EPI) {
                // first thing in sub-stage B, while the row waves issue no memory instructions: Q, V of
                // chunk k+1 (loaded at the start of the previous sub-stage B) have landed: their tail rows
                // set to zero; then Q, V of chunk k+2 into the buffer of chunk k, whose last reads were
                // in this iteration's sub-stage A.  Rows [16 pw, 16 pw + 16) each: the loads have an
                // iteration and a half to land, where the row waves' wait would be on the chain.
                if (nxt) {
                    wait_loads();
                    if (clen(k + 1) < C) {
                        zero_rows<DK, 16>(reinterpret_cast<__bf16*>(sm + S::qv(k + 1) + S::rQ), clen(k + 1), 16 * pw,
                                          opaque(lane));
                        zero_rows<BV, 16>(reinterpret_cast<__bf16*>(sm + S::qv(k + 1) + S::rV), clen(k + 1), 16 * pw,
                                          opaque(lane));
                    }
                }
                if (far) {
                    if constexpr (OUT)
                        dma_q<DK, 16>(p, smb + S::qv(k + 2) + S::rQ, tk + 2 * C, clen(k + 2), hk, 16 * pw, lane);
                    if (!p.v_zero)
                        dma_v<DK, BV, 16>(p, smb + S::qv(k + 2) + S::rV, tk + 2 * C, clen(k + 2), h, vb, 16 * pw, lane);
                }
            }
            if constexpr (EPI) {
                // waves 10, 11: rows [32 (pw - 2), + 32) of z of chunk k (into its Q tile) and of Q of
                // chunk k+1
                if (pw >= 2) {
                    if (cur) dma_z<DK, BV, 32>(p, smb + S::qv(k) + S::rQ, tk, clen(k), h, vb, 32 * (pw - 2), lane);
                    if (nxt) dma_q<DK, 32>(p, smb + S::qv(k + 1) + S::rQ, tk + C, clen(k + 1), hk, 32 * (pw - 2), lane);
                }
            }
            if (nxt && (pw == 0 || pw == 1)) {
                // the solve is this sub-stage's longest chain: its instructions go first on the SIMD
                __builtin_amdgcn_s_setprio(3);
                const __bf16* sLt = reinterpret_cast<const __bf16*>(sm + S::L);
                __bf16* Tt = reinterpret_cast<__bf16*>(sm + S::T);
                const float* fr = reinterpret_cast<const float*>(sm + S::WL) + 2 * C;  // f of L'
                solve_diag(sLt, Tt, fr, 2 * pw, lane);
                wave_sync();  // the level-1 products read the diagonal blocks other lanes wrote
                solve_level1(sLt, Tt, fr, 2 * pw, lane);
                __builtin_amdgcn_s_setprio(0);
            }
            if (nxt && pw == 2)
                copy_LBA(reinterpret_cast<const __bf16*>(sm + S::L), reinterpret_cast<__bf16*>(sm + S::T),
                         reinterpret_cast<const float*>(sm + S::WL) + 2 * C, lane);
            if (nxt && pw == 3) make_gates<DK, BV>(sm + S::raw(k + 1), sm + S::gates(k + 1), sm, lane, p.l2norm);
            // Pm and rq of chunk 0, formed in sub-stage A (rewritten in the next iteration's), by
            // the solve waves, which have time to spare here and never wait for their stores
            if (keep && k == 0 && pw < 2) {
                unsigned char* kd = p.pre + (size_t)pair * PRE_BYTES;
                keep_to_global<C * TSTR * 2, 128>(sm, S::PM, kd + PRE_PM, tid - 64 * PW0);
                keep_to_global<C * 4, 128>(sm, S::ORQ, kd + PRE_RQ, tid - 64 * PW0);
            }
            if constexpr (EPI) {
                if (pw >= 2 && (cur || nxt)) {
                    wait_loads();
                    if (nxt && clen(k + 1) < C)
                        zero_rows<DK, 32>(reinterpret_cast<__bf16*>(sm + S::qv(k + 1) + S::rQ), clen(k + 1),
                                          32 * (pw - 2), opaque(lane));
                }
            }
            lds_barrier();
            if (p.early_exit && decay <= kExitLog) break;
            if (conv) conv_after<DK, BV>(p, cw, sm, smb, k, clen(k + 1), clen(k + 2), far, nxt, tid);
        }
        // an early exit can leave Q, V loads of a later chunk in flight: none may land in LDS after
        // the workgroup has ended
        wait_loads();
    }
    if (p.tr_signal) {
        // every row wave's rows of A_j are in L2 (above): count this workgroup into the mark
        lds_barrier();
        if (tid == 0)
            __hip_atomic_fetch_add(p.negl + pair, 4 + (vb == 0 ? stopped : 0), __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    return BODY_DONE;
}

template <int DK, int BV, bool RAW, bool EPI, bool LEAN, bool TRANS = false>
__global__ __launch_bounds__(kernel_threads<BV>()) void chunk_bf16_kernel(Params<DK> p) {
    chunk_body<DK, BV, RAW, EPI, LEAN, TRANS>(p, blockIdx.x);
}

// The transition and rerun passes of the segmented path in one launch (d_k = d_v, so both passes
// map a block to the same (segment, head, row block)).  A block first tries the one-chunk rerun of
// the usual case (nothing to wait for); then, where the first pass left its pair's transition marked
// not negligible, it forms that transition and counts itself into the mark; then, if the first try
// did not apply, it reruns its segment, waiting where that needs a transition of an earlier segment
// (wait_transitions).  In the usual case, where the first pass marked every transition negligible,
// a block reads the marks with the rerun's loads in flight and forms no transition.
template <int DK, int BV, bool RAW, bool EPI>
__global__ __launch_bounds__(kernel_threads<BV>()) void chunk_bf16_tail_kernel(Params<DK> pt, Params<DK> pr) {
    const int r = chunk_body<DK, BV, RAW, EPI, false, false>(pr, blockIdx.x, BODY_FAST);
    if (r & BODY_TRANS) {
        lds_barrier();  // LDS free for the transition
        chunk_body<DK, BV, RAW, false, true, true>(pt, blockIdx.x);
    }
    if (!(r & BODY_DONE)) {
        lds_barrier();  // LDS free for the rerun
        chunk_body<DK, BV, RAW, EPI, false, false>(pr, blockIdx.x, BODY_REST);
    }
}

template <int DK, int BV, bool RAW, bool EPI, bool LEAN, bool TRANS>
hipError_t launch_one(const Params<DK>& p, const ChunkArgs& a, int grid, int smem) {
    hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(&chunk_bf16_kernel<DK, BV, RAW, EPI, LEAN, TRANS>), smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_bf16_kernel<DK, BV, RAW, EPI, LEAN, TRANS>), dim3(grid), dim3(kernel_threads<BV>()), smem,
                       a.stream, p);
    return hipGetLastError();
}

template <int DK, int BV, bool EPI>
hipError_t launch_k(const Params<DK>& p, const ChunkArgs& a, int grid, int smem) {
    // the lean instantiation (no rerun code) for every pass but the rerun, unless the epilogue is on;
    // the transition pass (no output) has one of its own
    constexpr bool L = !EPI;
    const bool lean = L && p.init != INIT_PREV;
    if constexpr (L) {
        if (lean && p.out == OUT_NONE)
            return a.gate_params ? launch_one<DK, BV, true, EPI, true, true>(p, a, grid, smem)
                                 : launch_one<DK, BV, false, EPI, true, true>(p, a, grid, smem);
    }
    if (a.gate_params)
        return lean ? launch_one<DK, BV, true, EPI, L, false>(p, a, grid, smem)
                    : launch_one<DK, BV, true, EPI, false, false>(p, a, grid, smem);
    return lean ? launch_one<DK, BV, false, EPI, L, false>(p, a, grid, smem)
                : launch_one<DK, BV, false, EPI, false, false>(p, a, grid, smem);
}

// One pass of the kernel.  rows = state rows (dv, or dk for the transition pass).
struct Pass {
    int P, init, out, v_zero, early_exit, skip_first, negl_mode, rows;
    const float* s0;
    float* sfin;
    int* negl;
    unsigned char* pre;
    int pre_mode;
    const int* marks;
    const float* trans;
    float* ein;
    float* fin;
    int fin_in_slot;
};

template <int DK, int BV>
Params<DK> make_params(const ChunkArgs& a, const Pass& c) {
    Params<DK> p;
    p.q = static_cast<const __bf16*>(a.q);
    p.k = static_cast<const __bf16*>(a.k);
    p.v = static_cast<const __bf16*>(a.v);
    p.g = a.g;
    p.beta = a.beta;
    p.s0 = c.s0;
    p.conv_w = a.conv_w;
    p.gate_params = a.gate_params;
    p.conv_state = static_cast<const __bf16*>(a.conv_state);
    p.cu = a.cu;
    p.o = static_cast<__bf16*>(a.o);
    p.sfin = c.sfin;
    p.negl = c.negl;
    p.N = a.N;
    p.T_tot = a.T_tot;
    p.H = a.H;
    p.Hk = a.Hk;
    p.grp = a.H / a.Hk;
    p.dv = c.rows;
    p.nv = c.rows / BV;
    p.P = c.P;
    p.init = c.init;
    p.out = c.out;
    p.v_zero = c.v_zero;
    p.early_exit = c.early_exit;
    p.skip_first = c.skip_first;
    p.negl_mode = c.negl_mode;
    p.pre = c.pre;
    p.pre_mode = c.pre_mode;
    p.marks = c.marks;
    p.trans = c.trans;
    p.ein = c.ein;
    p.fin = c.fin;
    p.fin_in_slot = c.fin_in_slot;
    p.tr_signal = 0;
    p.tr_wait = 0;
    p.scale = a.scale;
    p.l2norm = a.l2norm;
    p.out_gate = static_cast<const __bf16*>(a.out_gate);
    p.norm_weight = a.norm_weight;
    p.norm_eps = a.norm_eps;
    return p;
}

// the LDS a workgroup of this width needs (160 KiB on gfx950)
template <int DK, int BV>
hipError_t check_lds() {
    DeviceInfo dinfo;
    const hipError_t e = current_device_info(&dinfo);
    if (e != hipSuccess) return e;
    return dinfo.lds_max < Smem<DK, BV>::bytes ? hipErrorInvalidConfiguration : hipSuccess;
}

template <int DK, int BV>
hipError_t launch_t(const ChunkArgs& a, const Pass& c) {
    const Params<DK> p = make_params<DK, BV>(a, c);
    const int smem = Smem<DK, BV>::bytes;
    const hipError_t e = check_lds<DK, BV>();
    if (e != hipSuccess) return e;
    const int grid = a.N * c.P * a.H * p.nv;
    // the output epilogue in the kernel: wide workgroups of a pass that stores o
    const bool epi = Smem<DK, BV>::WIDE && a.out_gate && c.out == OUT_STORE;
    if (epi) {
        if constexpr (Smem<DK, BV>::WIDE) return launch_k<DK, BV, true>(p, a, grid, smem);
        return hipErrorInvalidValue;
    }
    return launch_k<DK, BV, false>(p, a, grid, smem);
}

template <int DK, int BV, bool RAW, bool EPI>
hipError_t launch_tail_one(const Params<DK>& pt, const Params<DK>& pr, const ChunkArgs& a, int grid) {
    const int smem = Smem<DK, BV>::bytes;
    hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(&chunk_bf16_tail_kernel<DK, BV, RAW, EPI>), smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_bf16_tail_kernel<DK, BV, RAW, EPI>), dim3(grid), dim3(kernel_threads<BV>()), smem,
                       a.stream, pt, pr);
    return hipGetLastError();
}

// The transition pass ct and the rerun pass cr in one launch (d_k = d_v: the same workgroups).
template <int DK, int BV>
hipError_t launch_tail_t(const ChunkArgs& a, const Pass& ct, const Pass& cr) {
    Params<DK> pt = make_params<DK, BV>(a, ct), pr = make_params<DK, BV>(a, cr);
    pt.tr_signal = 1;
    pr.tr_wait = 4 * pt.nv;
    const hipError_t e = check_lds<DK, BV>();
    if (e != hipSuccess) return e;
    const int grid = a.N * cr.P * a.H * pr.nv;
    if constexpr (Smem<DK, BV>::WIDE) {
        if (a.out_gate)
            return a.gate_params ? launch_tail_one<DK, BV, true, true>(pt, pr, a, grid)
                                 : launch_tail_one<DK, BV, false, true>(pt, pr, a, grid);
    }
    return a.gate_params ? launch_tail_one<DK, BV, true, false>(pt, pr, a, grid)
                         : launch_tail_one<DK, BV, false, false>(pt, pr, a, grid);
}

// 128 state rows per workgroup where chunk_rows_per_workgroup allows, else 64, or 32 when the
// pass has a 32-row state
template <int DK>
int width_for(int rows) {
    if (DK == 128 && chunk_rows_per_workgroup(DK, rows) == BVW) return BVW;
    return rows >= 64 ? 64 : 32;
}

template <int DK>
hipError_t launch_rows(const ChunkArgs& a, const Pass& c) {
    if constexpr (DK == 128)
        if (width_for<DK>(c.rows) == BVW) return launch_t<DK, BVW>(a, c);
    return c.rows >= 64 ? launch_t<DK, 64>(a, c) : launch_t<DK, 32>(a, c);
}

// The transition pass and the rerun: one launch where d_k = d_v (the two passes then have the same
// workgroups), else one launch each.
template <int DK>
hipError_t launch_tail(const ChunkArgs& a, const Pass& ct, const Pass& cr) {
    const int w = width_for<DK>(ct.rows);
    if (ct.rows == cr.rows) {
        if constexpr (DK == 128) {
            if (w == BVW) return launch_tail_t<DK, BVW>(a, ct, cr);
        } else {
            return w == 64 ? launch_tail_t<DK, 64>(a, ct, cr) : launch_tail_t<DK, 32>(a, ct, cr);
        }
    }
    hipError_t e = launch_rows<DK>(a, ct);
    if (e == hipSuccess) e = launch_rows<DK>(a, cr);
    return e;
}

template <int DK>
hipError_t run(const ChunkArgs& a, int P) {
    if (P <= 1) return launch_rows<DK>(a, Pass{1, INIT_S0, OUT_STORE, 0, 0, 0, NEGL_NONE, a.dv, a.s0, a.sfin, nullptr});
    // Segmented path for long sequences (each sequence cut into P segments of whole chunks).
    // The chunk map is affine in the state: S_out = S_in A_p + B_p.
    //  1. every segment from its own start: B_p (zero state in, the true initial state for p = 0)
    //     and o without the contribution of the state entering the segment; from the gates alone,
    //     whether the bound on the whole segment's transition is below 2^-40 (negligible);
    //  2. A_p = the transition of segment p (identity in, zero values), for the segments not marked
    //     negligible, stopped once its norm bound is below 2^-40 (then marked negligible);
    //  3. rerun: E_{p-1} (E_0 = B_0, E_j = E_{j-1} A_j + B_j, B_j itself where A_j is negligible),
    //     formed in segment p's own workgroups (final = E_{P-1} in the last segment's), then
    //     segment p again from E_{p-1}, overwriting o, until the bound on the transition
    //     since the segment start is <= 2^-40; from there on the state of step 1 differs from the
    //     true one by less than that factor of |E_{p-1}|, so step 1's o stands.  Where the first
    //     chunk alone reaches the bound (the usual case), step 1 keeps that chunk's prepared
    //     operands and the rerun only redoes the chunk's state and output products.
    const SegLayout L = seg_layout(a.N, a.H, a.dk, a.dv, P);
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    float* E = reinterpret_cast<float*>(ws + L.off_E);
    float* A = reinterpret_cast<float*>(ws + L.off_A);
    int* negl = reinterpret_cast<int*>(ws + L.off_negl);
    const int ex = a.l2norm ? 1 : 0;
    // the kept operands serve only a rerun that stops early and has no conv inside the kernel
    const bool keep = ex && !a.conv_w;
    unsigned char* pre = keep ? ws + L.off_pre : nullptr;
    // final_state == initial_state: segment 0 of the first pass reads the initial state while its
    // last segment would write B_{P-1} to the same buffer in the same launch, in no guaranteed
    // order.  B_{P-1} then stays in its slot and the rerun (after the first pass has finished
    // reading the initial state) writes the final state.
    const int in_slot = a.sfin && a.sfin == a.s0 ? 1 : 0;
    hipError_t e = launch_rows<DK>(a, Pass{P, INIT_S0, OUT_STORE, 0, 0, 0, NEGL_MARK, a.dv, a.s0, E, negl, pre,
                                           keep ? PRE_KEEP : PRE_NONE, nullptr, nullptr, nullptr,
                                           in_slot ? nullptr : a.sfin, 0});
    if (e == hipSuccess)
        e = launch_tail<DK>(a, Pass{P, INIT_IDENTITY, OUT_NONE, 1, ex, 1, NEGL_SKIP, a.dk, nullptr, A, negl},
                            Pass{P, INIT_PREV, OUT_STORE, 0, ex, 1, NEGL_NONE, a.dv, E, nullptr, nullptr, pre,
                                 keep ? PRE_USE : PRE_NONE, negl, A, reinterpret_cast<float*>(ws + L.off_ein), a.sfin,
                                 in_slot});
    return e;
}

}  // namespace

hipError_t launch_chunk_bf16(const ChunkArgs& a) {
    switch (a.dk) {
        case 32: return run<32>(a, a.segments);
        case 64: return run<64>(a, a.segments);
        case 128: return run<128>(a, a.segments);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
