// gemm_tiled.hip -- expert projections for larger batches: grouped bf16 GEMM
// on the CDNA4 matrix cores.
//
// Each expert's rows form one contiguous segment of the sorted activations, so
// the layer is a grouped GEMM C_e = X_e W_e^T with both operands K-contiguous
// (Mixtral of Experts, notion page "Implementation": SwiGLU experts with K = 2;
// the sparse-matmul kernels the pages cite are prior art, this is a plain
// grouped GEMM over the per-expert segments).
//
// Tile: 256 weight rows (MFMA M side) x BT tokens (MFMA N side) x 64 k, BT = 64,
// 128 or 256 by the rows an expert holds (chosen on the host).
//  * BT = 256: 8 wavefronts (2 per SIMD) in a 2 x 4 grid; each owns 128 weight
//    rows x 64 tokens as 8 x 4 accumulators of v_mfma_f32_16x16x32_bf16. Two
//    wavefronts per SIMD keep the matrix pipe fed while the other waits on LDS
//    or a barrier. The LDS holds three weight stages, so weight tiles are
//    fetched two k-blocks ahead of their use.
//  * BT = 64, 128: 8 wavefronts in a 4 x 2 grid of v_mfma_f32_32x32x16_bf16
//    tiles (the 32 x 32 shape needs fewer fragment registers per token).
//  * Global memory goes straight to LDS (global_load_lds_dwordx4: a wavefront
//    instruction fills one contiguous kilobyte, lane L the bytes [16L, 16L+16));
//    one barrier per k-block.
//  * LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled by swz() of
//    the row's position in its 32-row group, so that the fragment reads of both
//    MFMA shapes hit distinct banks in every pass of the LDS (measured: zero
//    bank conflicts); the DMA writes are contiguous kilobytes.
//  * Gate-up: the 256 weight rows are W1 and W3 rows of the same 128 output
//    columns, interleaved so that every wavefront holds g and u of the same
//    columns and applies silu(g) * u in registers; the result is rounded once to
//    bf16. Down: 256 W2 rows = 256 output columns, float32 out.
//  * Each of the 8 XCDs (workgroups are dealt to XCDs in turn) runs its tiles
//    with the token block fastest, so concurrently running tiles share weight
//    tiles in its own L2: the 256-token tiles take the (expert, column block)
//    groups round-robin over the XCDs, the narrower ones one contiguous range of
//    the (expert, column block, token block) order per XCD (see find_tile).
//    Token rows past a tile's end read a row of zeros (g_zero_row); their
//    results are never stored.
//  * Down can split the sum over h into `ksplit` parts: each part is a tile of
//    its own writing float32 partial sums that the combine step adds in a fixed
//    order, so that the last round of tiles fills the GPU.
//  * Every variant sums each output over k in the same order (64-wide k-blocks
//    in order, 16-wide halves of the MFMA steps within), so neither the tile
//    width nor the MFMA shape changes a bit of the result.
#include "kernels.h"

namespace moe {
namespace {

constexpr int kXCD = 8;
typedef __attribute__((address_space(3))) void lds_void;

// A row of zeros in device memory (static storage, zeroed when the code object
// loads). The rows of a token tile past its expert's end copy from it instead
// of duplicating a real row: their results are never stored, and matrix
// instructions on zero operands draw less power, which the power-limited clock
// returns as speed (0.2-3% per launch, most where tiles are mostly padding).
// Longer rows (K > kZeroK) fall back to the duplicates.
constexpr int kZeroK = 65536;
__device__ __attribute__((aligned(1024))) uint16_t g_zero_row[kZeroK];

// s_waitcnt immediates (vmcnt in bits 3:0, expcnt 6:4, lgkmcnt 11:8): vmcnt(n)
// with the other counters at their maximum, and vmcnt(n) with lgkmcnt(0).
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVm0Lgkm0 = 0x0070;
// vmcnt(n), n < 64 (its upper two bits go to bits 15:14)
constexpr int wait_vm(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }
constexpr int wait_vm_lgkm0(int n) { return ((n >> 4) << 14) | 0x0070 | (n & 15); }

// Workgroup barrier without the fence of __syncthreads() (which would wait for
// every copy in flight); the explicit vmcnt waits before it are the ones the
// pipeline needs, the empty asm keeps LDS accesses on their side of it.
#define TILED_BARRIER()                  \
  {                                      \
    asm volatile("" ::: "memory");       \
    __builtin_amdgcn_s_barrier();        \
    asm volatile("" ::: "memory");       \
  }

// ---- the main loop shared by the kernels below ---------------------------------
// A wavefront owns FA x FB accumulators of 32 x 32 (FA fragments of 32 weight rows,
// FB of 32 tokens). A 64-wide k-block is four 16-wide k-steps. Fragments of k-step
// kk are read from LDS one k-step ahead into the other of two register buffers.
// With copies into LDS in flight the compiler can only wait for every LDS read at
// once (lgkmcnt(0)), so the order within a k-step is fixed explicitly: the first
// MFMA, then the next k-step's reads, then the other MFMAs. The wait in front of
// a k-step's first MFMA then only covers reads issued a whole k-step earlier
// (measured on MI355X: with the reads issued before the first MFMA, or spread
// among the MFMAs, the last reads were still in flight at that wait).
#define TL_READ(SW, SX, KK, BUF)                                                           \
  {                                                                                        \
    const char *pa_ = reinterpret_cast<const char *>(SW) + baseA;                          \
    const char *pb_ = reinterpret_cast<const char *>(SX) + baseB;                          \
    _Pragma("unroll") for (int f = 0; f < FA; ++f) fa[BUF][f] =                            \
        *reinterpret_cast<const bf16x8 *>(pa_ + f * 4096 + offk[KK]);                      \
    _Pragma("unroll") for (int t = 0; t < FB; ++t) fb[BUF][t] =                            \
        *reinterpret_cast<const bf16x8 *>(pb_ + t * 4096 + offk[KK]);                      \
  }
#define TL_MFMA(BUF)                                                                       \
  _Pragma("unroll") for (int t = 0; t < FB; ++t)                                           \
    _Pragma("unroll") for (int f = 0; f < FA; ++f)                                         \
      acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[BUF][f], fb[BUF][t], acc[f][t], \
                                                          0, 0, 0);
// multiply the fragments in BUF while k-step KKN of (SW, SX) is read into BUFN
#define TL_KSTEP(SW, SX, KKN, BUFN, BUF)                                                   \
  TL_READ(SW, SX, KKN, BUFN)                                                               \
  TL_MFMA(BUF)                                                                             \
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                       \
  __builtin_amdgcn_sched_group_barrier(0x100, FA + FB, 0);                                 \
  __builtin_amdgcn_sched_group_barrier(0x008, FA * FB - 1, 0);                             \
  __builtin_amdgcn_sched_barrier(0);
// the last k-step of a k-block, no reads behind it
#define TL_KLAST(BUF)                                                                      \
  TL_MFMA(BUF)                                                                             \
  __builtin_amdgcn_sched_barrier(0);
// Three weight stages and two token stages (weights of k-block KB in slot KB % 3,
// tokens in KB % 2; WS/XS the slots of KB, WN/XN those of KB + 1). The barrier sits
// before the last k-step: k-steps 0-2 of KB are multiplied, the wavefront waits for
// its fragment reads and for the copies of KB + 1 (kStepWait: all but the weight
// copies of KB + 2, the youngest), the barrier makes every wavefront's copies visible and
// frees KB's slots, the copies of KB + 2 (tokens) and KB + 3 (weights) go into them,
// and k-step 3 of KB is multiplied from registers while k-step 0 of KB + 1 is read:
// the matrix cores do not drain at the barrier (5-8% faster than a barrier after
// the last k-step, bitwise the same sums). Weights are fetched about two k-blocks
// ahead, tokens one.
#define TL_STEP(KB, WS, XS, WN, XN)                                                        \
  TL_KSTEP(sW##WS, sX##XS, 1, 1, 0)                                                        \
  TL_KSTEP(sW##WS, sX##XS, 2, 0, 1)                                                        \
  TL_KSTEP(sW##WS, sX##XS, 3, 1, 0)                                                        \
  __builtin_amdgcn_s_waitcnt(kStepWait);                                                   \
  TILED_BARRIER()                                                                          \
  DMAX(sX##XS, (KB) + 2)                                                                   \
  DMAW(sW##WS, (KB) + 3)                                                                   \
  TL_KSTEP(sW##WN, sX##XN, 0, 0, 1)
// The whole k-loop over nk (even) k-blocks with that pipeline; unrolled by 6 so
// that every slot index is static.
#define TL_KLOOP(PROLOGUE_WAIT)                                                            \
  DMAW(sW0, 0)                                                                             \
  DMAX(sX0, 0)                                                                             \
  DMAW(sW1, 1)                                                                             \
  DMAX(sX1, 1)                                                                             \
  DMAW(sW2, 2)                                                                             \
  __builtin_amdgcn_s_waitcnt(PROLOGUE_WAIT); /* k-block 0 has landed */                    \
  TILED_BARRIER()                                                                          \
  TL_READ(sW0, sX0, 0, 0)                                                                  \
  {                                                                                        \
    int kt = 0;                                                                            \
    for (; kt + 6 <= nk; kt += 6) {                                                        \
      TL_STEP(kt + 0, 0, 0, 1, 1)                                                          \
      TL_STEP(kt + 1, 1, 1, 2, 0)                                                          \
      TL_STEP(kt + 2, 2, 0, 0, 1)                                                          \
      TL_STEP(kt + 3, 0, 1, 1, 0)                                                          \
      TL_STEP(kt + 4, 1, 0, 2, 1)                                                          \
      TL_STEP(kt + 5, 2, 1, 0, 0)                                                          \
    }                                                                                      \
    if (kt < nk) { /* 2 or 4 k-blocks remain */                                            \
      TL_STEP(kt + 0, 0, 0, 1, 1)                                                          \
      TL_STEP(kt + 1, 1, 1, 2, 0)                                                          \
      kt += 2;                                                                             \
    }                                                                                      \
    if (kt < nk) {                                                                         \
      TL_STEP(kt + 0, 2, 0, 0, 1)                                                          \
      TL_STEP(kt + 1, 0, 1, 1, 0)                                                          \
    }                                                                                      \
  }                                                                                        \
  /* no copy or read in flight past the loop (the last step read ahead) */                 \
  __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);

// Physical 16-byte chunk = logical chunk ^ swz(row); depends on row & 31 only.
// A wavefront's ds_read_b128 is served in four passes of 16 lanes; lane 0 shares
// its pass with lanes 1-3, 12-15, 20-23 and 24-27 (the 4-lane groups whose index
// bits XOR to the same parity within each half-wavefront), 64 banks of 4 bytes
// (measured on MI355X with single-wavefront address patterns). For both fragment
// shapes below (32 rows x 2 chunks per 32 x 32 operand, 16 rows x 4 chunks per
// 16 x 16 operand) this swizzle puts every pass on 16 distinct 4-bank groups;
// (r ^ r >> 3) & 7, which is conflict-free for the 32-row reads, costs 1.5x on the
// 16-row ones.
__host__ __device__ constexpr int swz(int r) { return (r & 7) ^ ((r >> 4) & 1); }
// the odd 16-row half of a 32-row group has the swizzle of the even half XOR this
// (as a byte offset)
constexpr int kOddXor = (swz(16) ^ swz(0)) * 16;
static_assert(((swz(16) ^ swz(0)) == (swz(31) ^ swz(15))), "odd-half swizzle is one XOR");

// One global -> LDS copy of 16 bytes per lane (a plain function: the builtin
// inside a kernel template can fail the template's host-side instantiation).
__device__ __forceinline__ void dma16(const uint16_t *g, lds_void *l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}
// The same copy with the non-temporal hint, for weight tiles that only one
// token tile reads.
__device__ __forceinline__ void dma16_nt(const uint16_t *g, lds_void *l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 2);
}

// The tile of this workgroup: expert e (rows row0 .. row0 + ne - 1), token
// rows m0 .. lim - 1 of it, output column c0 and, with ksplit > 1 (down only),
// the part ks of the sum over K: 64-wide k-blocks kb0 .. kb0 + nkp - 1. False
// when the workgroup has no tile.
struct Tile {
  int e, row0, ne, m0, lim, c0, ks, kb0, nkp;
};

constexpr int kCUsPerXCD = 32;  // MI355X: 256 compute units in 8 XCDs

// Where part 0 of a 2-way split of nkt k-blocks ends, for g tiles per part on each
// XCD. The workgroups of an XCD run part 0 of its g tiles first, then part 1, one
// per compute unit at a time. With g = q C + r (C compute units, 0 < r, q >= 1), an
// even split leaves C - r units idle through the last round; a longer part 0
// (q or q + 1 of them per unit) and a shorter part 1 that fills the units that
// finished part 0 a round early end together when part 0 holds the fraction
// g / (g + C - r) of the k-blocks (prefill_8x7b down: g = 72, C = 32, 168 of 224
// k-blocks). Rounded to an even count, clamped to [nkt / 2, nkt - 2].
__device__ __forceinline__ int split_point(int g, int nkt) {
  const int C = kCUsPerXCD, q = g / C, r = g % C;
  if (q == 0 || r == 0) return nkt / 2;
  const int64_t den = int64_t(g + C - r);
  const int a = int((int64_t(nkt) * g + den) / (2 * den)) * 2;  // nearest even
  return max(nkt / 2, min(nkt - 2, a));
}

// Column blocks c of expert e that XCD x takes under the round-robin order below:
// c = first, first + 8, ... < ct, where (e ct + c) % 8 == x.
__device__ __forceinline__ int rr_first(int e, int x, int ct) {
  return ((x - e * ct) % kXCD + kXCD) % kXCD;
}
__device__ __forceinline__ int rr_groups(int e, int x, int ct) {
  const int c0 = rr_first(e, x, ct);
  return c0 < ct ? (ct - 1 - c0) / kXCD + 1 : 0;
}

// EVEN: an expert's ceil(ne / BT) token tiles split its rows evenly (tile m holds
// rows m ne / mtiles .. (m + 1) ne / mtiles - 1, all within one row of each other)
// instead of BT rows each and the rest in the last; the tiles of different experts
// then differ in length, so the XCDs (workgroups are dealt to them in turn) take the
// (expert, column block) groups round-robin: XCD x runs the groups e ct + c = x mod 8,
// each with all its token blocks one after another, expert by expert, so that every
// XCD gets the same share of every expert (prefill_8x7b: 14 of each expert's 112
// gate-up column blocks) and the token blocks sharing a weight slice run on one XCD
// at one time. Otherwise the tiles of a part are ordered (expert, column block, token
// block) and each XCD takes one contiguous range of g of them. Either way an XCD runs
// all parts of its tiles, part-major.
template <int BT, int kCols, bool EVEN = false, bool UNEVEN = true>
__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offsets, int E, int N,
                                          int K, int ksplit, Tile &tl) {
  const int ct = (N + kCols - 1) / kCols;
  const int x = blockIdx.x % kXCD, i = blockIdx.x / kXCD;
  int g = 0;      // tiles per part on this XCD
  int total = 0;  // tiles per part (contiguous order)
  if constexpr (EVEN) {
    for (int q = 0; q < E; ++q)
      g += rr_groups(q, x, ct) * ((offsets[q + 1] - offsets[q] + BT - 1) / BT);
  } else {
    for (int q = 0; q < E; ++q) total += ct * ((offsets[q + 1] - offsets[q] + BT - 1) / BT);
    g = (total + kXCD - 1) / kXCD;
  }
  if (i >= g * ksplit) return false;
  tl.ks = i / g;
  int L = i % g;
  const int nkt = K / 64;
  // (kb0 and nkp are set once, from locals: with a store to each field in both arms
  // of the branch the compiler merged them into one store to a selected field, which
  // kept the whole tile in scratch memory and put a scratch load in every prologue)
  int kb0, nkp;
  if (ksplit == 2 && UNEVEN) {
    const int a = split_point(g, nkt);  // part 0 takes k-blocks [0, a), part 1 [a, nkt)
    kb0 = tl.ks ? a : 0;
    nkp = tl.ks ? nkt - a : a;
  } else {
    nkp = nkt / ksplit;
    kb0 = tl.ks * nkp;
  }
  tl.kb0 = kb0;
  tl.nkp = nkp;
  int e = 0, row0 = 0, ne = 0, mtiles = 0;
  if constexpr (EVEN) {
    int ng = 0;
    for (; e < E; ++e) {
      row0 = offsets[e];
      ne = offsets[e + 1] - row0;
      mtiles = (ne + BT - 1) / BT;
      ng = rr_groups(e, x, ct);
      if (L < ng * mtiles) break;
      L -= ng * mtiles;
    }
    // L < g, so some expert holds it: L = group index * mtiles + token block
    tl.c0 = (rr_first(e, x, ct) + kXCD * (L / mtiles)) * kCols;
  } else {
    L += x * g;
    if (L >= total) return false;
    for (; e < E; ++e) {
      row0 = offsets[e];
      ne = offsets[e + 1] - row0;
      mtiles = (ne + BT - 1) / BT;
      if (L < ct * mtiles) break;
      L -= ct * mtiles;
    }
    tl.c0 = (L / mtiles) * kCols;
  }
  tl.e = e;
  tl.row0 = row0;
  tl.ne = ne;
  const int m = L % mtiles;
  if constexpr (EVEN) {
    tl.m0 = int(int64_t(m) * ne / mtiles);
    tl.lim = int(int64_t(m + 1) * ne / mtiles);
  } else {
    tl.m0 = m * BT;
    tl.lim = min(ne, tl.m0 + BT);
  }
  return true;
}

// ---- BT = 256: the 16 x 16 x 32 body ---------------------------------------------
// 8 wavefronts (2 per SIMD) in a 2 x 4 grid; each owns 128 weight rows x 4 token
// fragments of 16 (every fourth fragment of the tile, so that a tile of fewer rows
// leaves every wavefront about the same work) as 8 x 4 accumulators of
// v_mfma_f32_16x16x32_bf16 (A: lane holds weight row
// lane & 15 and k 8 (lane >> 4) + 0..7 of a 32-wide k-step; B the same for a token;
// D: token lane & 15, weight rows 4 (lane >> 4) + 0..3). A 64-wide k-block is two
// 32-wide k-steps. On MI355X this shape runs the same tile 4-6% faster than the
// 32 x 32 x 16 one (the clock holds about 0.15 GHz higher at the same matrix work)
// and gives the same sums to the bit: both add the products of each 16-wide half of
// a 32-wide k-step into the accumulator in the same order.
//
// Weight fragment f (rows 16 f .. 16 f + 15 of the wavefront's block), k-step kk:
// logical chunk 4 kk + (lane >> 4) of row 16 f + (lane & 15) sits at physical chunk
// (lane >> 4) ^ swz(lane & 15) ^ 4 kk ^ (f & 1) kOddXor / 16, so every read address
// is lane_base ^ (64 kk | (f & 1) kOddXor) + 2048 f; token fragment t (tile rows
// 16 (4 t + wc) ..) is lane_base ^ 64 kk + 8192 t, its parity fixed by wc. The empty
// asm hands each k-step a fresh copy of the lane base, so that the compiler does not
// keep one address register per slot, k-step and parity live across the loop.
#define M16_READ_B(SX, KK, BUF)                                                            \
  {                                                                                        \
    uint32_t lb_ = laneB;                                                                  \
    asm volatile("" : "+v"(lb_));                                                          \
    const char *p_ = reinterpret_cast<const char *>(SX) + (lb_ ^ (64 * (KK)));             \
    _Pragma("unroll") for (int t = 0; t < NT; ++t) fb[BUF][t] =                            \
        *reinterpret_cast<const bf16x8 *>(p_ + t * 8192);                                  \
  }
#define M16_READ_A(SW, KK, BUF, H)                                                         \
  {                                                                                        \
    uint32_t la_ = laneA;                                                                  \
    asm volatile("" : "+v"(la_));                                                          \
    const char *p0_ = reinterpret_cast<const char *>(SW) + (la_ ^ (64 * (KK)));            \
    const char *p1_ = reinterpret_cast<const char *>(SW) + (la_ ^ (64 * (KK) + kOddXor));  \
    _Pragma("unroll") for (int f = 4 * (H); f < 4 * (H) + 4; ++f) fa[BUF][f] =             \
        *reinterpret_cast<const bf16x8 *>(((f & 1) ? p1_ : p0_) + f * 2048);               \
  }
#define M16_MFMA(BUF, H)                                                                   \
  _Pragma("unroll") for (int f = 4 * (H); f < 4 * (H) + 4; ++f)                           \
    _Pragma("unroll") for (int t = 0; t < NT; ++t)                                         \
      acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[BUF][f], fb[BUF][t], acc[f][t], \
                                                          0, 0, 0);
// Multiply the fragments in BUF while k-step KKN of (SW, SX) is read into BUFN, in
// two halves so that only half of the weight fragments are double-buffered (the
// registers hold 128 accumulators): the token fragments and weight fragments 0-3
// are read during the first half of the k-step, weight fragments 4-7 during its
// second half, once fragments 0-3 of this k-step have been consumed. The k-step
// behind a barrier also issues the copies into the slots the barrier freed
// (tokens of KB + 2 from DX in its first half, weights of KB + 3 from DW in its
// second). Every half starts with an MFMA, and the fragment reads and copies go
// out one or two at a time between MFMAs rather than in bursts, so that the LDS
// and the memory system see an even stream and each wavefront always has matrix
// work queued behind them: the gate-up reads two fragments after each of the first
// four MFMAs and then the copies after every second MFMA; the down projection,
// one read after every second MFMA, and a copy after every second read. On MI355X
// (prefill_8x7b routing, 16 interleaved rounds) this took the gate-up from 1.634 to
// 1.572 ms and the down projection from 0.896 to 0.837 ms against reads in one
// burst after the first MFMA and copies after every third; the other combinations
// of the two patterns, and reads after every fourth MFMA, landed in between.
// Bitwise the same sums: only the issue order of loads changes.
#define M16_G(M, N) __builtin_amdgcn_sched_group_barrier(M, N, 0);
#define M16_G4(X) X X X X
#define M16_MM(N) M16_G(0x008, N) /* N MFMAs */
#define M16_DS(N) M16_G(0x100, N) /* N LDS reads */
#define M16_VM(N) M16_G(0x010, N) /* N copies */
#define M16_KSTEP(SW, SX, KKN, BUFN, BUF)                                                  \
  M16_READ_B(SX, KKN, BUFN)                                                                \
  M16_READ_A(SW, KKN, BUFN, 0)                                                             \
  M16_MFMA(BUF, 0)                                                                         \
  if constexpr (GATEUP) { M16_G4(M16_MM(1) M16_DS(2)) M16_MM(12) }                         \
  else { M16_G4(M16_MM(2) M16_DS(1) M16_MM(2) M16_DS(1)) }                                 \
  __builtin_amdgcn_sched_barrier(0);                                                       \
  M16_READ_A(SW, KKN, BUFN, 1)                                                             \
  M16_MFMA(BUF, 1)                                                                         \
  if constexpr (GATEUP) { M16_G4(M16_MM(1) M16_DS(1)) M16_MM(12) }                         \
  else { M16_G4(M16_MM(2) M16_DS(1)) M16_MM(8) }                                           \
  __builtin_amdgcn_sched_barrier(0);
#define M16_KSTEP_COPY(SW, SX, KKN, BUFN, BUF, DX, DW, KB)                                 \
  M16_READ_B(SX, KKN, BUFN)                                                                \
  M16_READ_A(SW, KKN, BUFN, 0)                                                             \
  DMAX(DX, (KB) + 2)                                                                       \
  M16_MFMA(BUF, 0)                                                                         \
  if constexpr (GATEUP) { M16_G4(M16_MM(1) M16_DS(2)) M16_G4(M16_MM(2) M16_VM(1)) M16_MM(4) } \
  else { M16_G4(M16_MM(2) M16_DS(1) M16_MM(2) M16_DS(1) M16_VM(1)) }                       \
  __builtin_amdgcn_sched_barrier(0);                                                       \
  M16_READ_A(SW, KKN, BUFN, 1)                                                             \
  DMAW(DW, (KB) + 3)                                                                       \
  M16_MFMA(BUF, 1)                                                                         \
  if constexpr (GATEUP) { M16_G4(M16_MM(1) M16_DS(1)) M16_G4(M16_MM(2) M16_VM(1)) M16_MM(4) } \
  else { M16_G4(M16_MM(2) M16_DS(1) M16_VM(1)) M16_MM(8) }                                 \
  __builtin_amdgcn_sched_barrier(0);
// One k-block with the pipeline of TL_STEP: k-step 0 is multiplied while k-step 1
// is read, the wait and the barrier, then k-step 1 is multiplied while k-step 0 of
// KB + 1 is read and the copies of KB + 2 (tokens) and KB + 3 (weights) go out.
#define M16_STEP(KB, WS, XS, WN, XN)                                                       \
  M16_KSTEP(sW##WS, sX##XS, 1, 1, 0)                                                       \
  __builtin_amdgcn_s_waitcnt(kStepWait);                                                   \
  TILED_BARRIER()                                                                          \
  M16_KSTEP_COPY(sW##WN, sX##XN, 0, 0, 1, sX##XS, sW##WS, KB)
#define M16_KLOOP(PROLOGUE_WAIT)                                                           \
  DMAW(sW0, 0)                                                                             \
  DMAX(sX0, 0)                                                                             \
  DMAW(sW1, 1)                                                                             \
  DMAX(sX1, 1)                                                                             \
  DMAW(sW2, 2)                                                                             \
  __builtin_amdgcn_s_waitcnt(PROLOGUE_WAIT); /* k-block 0 has landed */                    \
  TILED_BARRIER()                                                                          \
  M16_READ_B(sX0, 0, 0)                                                                    \
  M16_READ_A(sW0, 0, 0, 0)                                                                 \
  M16_READ_A(sW0, 0, 0, 1)                                                                 \
  {                                                                                        \
    int kt = 0;                                                                            \
    for (; kt + 6 <= nk; kt += 6) {                                                        \
      M16_STEP(kt + 0, 0, 0, 1, 1)                                                         \
      M16_STEP(kt + 1, 1, 1, 2, 0)                                                         \
      M16_STEP(kt + 2, 2, 0, 0, 1)                                                         \
      M16_STEP(kt + 3, 0, 1, 1, 0)                                                         \
      M16_STEP(kt + 4, 1, 0, 2, 1)                                                         \
      M16_STEP(kt + 5, 2, 1, 0, 0)                                                         \
    }                                                                                      \
    if (kt < nk) { /* 2 or 4 k-blocks remain */                                            \
      M16_STEP(kt + 0, 0, 0, 1, 1)                                                         \
      M16_STEP(kt + 1, 1, 1, 2, 0)                                                         \
      kt += 2;                                                                             \
    }                                                                                      \
    if (kt < nk) {                                                                         \
      M16_STEP(kt + 0, 2, 0, 0, 1)                                                         \
      M16_STEP(kt + 1, 0, 1, 1, 0)                                                         \
    }                                                                                      \
  }                                                                                        \
  /* no copy or read in flight past the loop (the last step read ahead) */                 \
  __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);

// Three weight stages and two token stages (160 KiB of LDS). The weight tile of the
// first token block to reach a k-block is an HBM miss; about two k-blocks of lead
// hide more of that latency than one (measured 4-9% faster than two stages of both).
template <bool GATEUP>
__device__ __forceinline__ void body256(const Tile &tl, const uint16_t *__restrict__ X,
                                        const uint16_t *__restrict__ Wa,
                                        const uint16_t *__restrict__ Wb, void *__restrict__ out,
                                        int N, int K, int ksplit, int64_t part_stride,
                                        const int32_t *__restrict__ rowmap, uint16_t *sW0,
                                        uint16_t *sW1, uint16_t *sW2, uint16_t *sX0,
                                        uint16_t *sX1) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wavefront w takes weight rows 128 wr .. and the token fragments wc, wc + 4, ...;
  // with the wavefronts of a workgroup placed on the SIMDs in turn (w and w + 4 on
  // SIMD w % 4), the two of a SIMD hold wc and wc ^ 2, whose fragment counts add up
  // to the same on every SIMD when a tile has fewer than 16 fragments (other
  // assignments measured the same to within 1%)
  const int wr = wave >> 2, wc = (wave & 3) ^ (wr << 1);

  // ---- DMA assignment, 8 rows per instruction; lane p writes LDS bytes
  // [16p, 16p+16) of the instruction's kilobyte: row 8i + p/8 of its 8, physical
  // chunk p%8 = logical chunk ^ swz(row). Weights: wave w fills rows [32w, 32w+32).
  // Gate-up weight rows: 64 W1 rows, the W3 rows of the same columns, the next 64
  // W1 rows, their W3 rows. Weight offsets are bytes from the expert's matrix
  // (h d < 2^31, so they fit 32 bits), so the copies take a uniform base and a
  // 32-bit per-lane offset. Tokens: wave (wr, wc) fills the fragments wc + 8 wr and
  // wc + 8 wr + 4 (two instructions each), so the wavefront with wr = 0 copies the
  // first two fragments its column pair multiplies and the one with wr = 1 the
  // third and fourth. A tile whose column pair multiplies only 3 or 2 fragments
  // then leaves out the copies of the others: 4-6 of the 32 token copies per
  // k-block at prefill_8x7b (13-14 fragments of rows), 14 at T = 1024 (9), which
  // measured bitwise the same and 1% (prefill_8x7b), 10-11% (T = 1024 and a
  // ragged routing of 2200 rows) faster on the gate-up, up to 2% on the down
  // projection, against every wavefront copying 32 consecutive token rows.
  const size_t mat_elems = size_t(N) * K;
  const uint16_t *wmat = Wa + size_t(tl.e) * mat_elems;
  if (GATEUP && ((wave >> 1) & 1)) wmat = Wb + size_t(tl.e) * mat_elems;
  // token rows: x_perm rows row0 + m0 + r, or with a row map the rows
  // rowmap[...] of the unsorted input (one pointer per DMA instruction)
  uint32_t wofs[4];
  const uint16_t *xsrc[4];
  int xrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    int wrow;
    if constexpr (GATEUP) wrow = tl.c0 + ((r >> 7) << 6) + (r & 63);
    else wrow = min(tl.c0 + r, N - 1);
    wofs[i] = (uint32_t(wrow) * uint32_t(K) + c * 8) * 2u;
    const int rx = 16 * (wc + 8 * wr + 4 * (i >> 1)) + 8 * (i & 1) + (lane >> 3);
    xrow[i] = tl.row0 + tl.m0 + min(rx, tl.lim - 1 - tl.m0);
  }
  // The row map's four entries load together, so the first copies wait for one round
  // trip to the cache rather than four (with a load per branch the compiler waited for
  // each before the next; rows past the tile's end read the entry of its last row and
  // then take the zero row). With the tile kept out of scratch memory (find_tile):
  // bitwise the same, 0.5-1% faster on the gate-up.
  if (rowmap) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xrow[i] = rowmap[xrow[i]];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rx = 16 * (wc + 8 * wr + 4 * (i >> 1)) + 8 * (i & 1) + (lane >> 3);
    const int cx = (lane & 7) ^ swz(rx);
    xsrc[i] = (rx > tl.lim - 1 - tl.m0 && K <= kZeroK) ? g_zero_row + cx * 8
                                                        : X + size_t(xrow[i]) * K + cx * 8;
  }
  const int dma_row = wave * 32;
  // LDS row of token copy i: dma_xrow + 64 (i >> 1) + 8 (i & 1)
  const int dma_xrow = 16 * (wc + 8 * wr);

  // ---- fragment read bases (bytes): row lane & 15 of the wavefront's first
  // weight (token) fragment, physical chunk of logical chunk lane >> 4. Token
  // fragment t of the wavefront is tile rows 16 (4 t + wc) .., whose rows all have
  // the swizzle parity of wc: one base, 8 KiB (64 rows) apart.
  const uint32_t lchunk = uint32_t(((lane >> 4) ^ swz(lane & 15)) << 4);
  const uint32_t laneA = uint32_t((wr * 128 + (lane & 15)) * 128) | lchunk;
  const uint32_t laneB = uint32_t((wc * 16 + (lane & 15)) * 128) |
                         uint32_t(((lane >> 4) ^ swz(16 * (wc & 1) + (lane & 15))) << 4);

  f32x4 acc[8][4];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[f][t][i] = 0.f;
  bf16x8 fa[2][8], fb[2][4];

  // k-blocks of this part (an even count) and the first of them. Uniform values, but
  // the compiler cannot prove it through the tile lookup: without readfirstlane the
  // k-loop runs as a divergent loop under an exec mask, and at the loop's tail the
  // compiler waits for every copy in flight before the first LDS read (vmcnt(0) in
  // each of the five loops); scalar, the loop branches on SCC and those waits are
  // gone (bitwise the same sums, about 0.5-1% faster at prefill_8x7b and skew_8x7b)
  const int nk = __builtin_amdgcn_readfirstlane(tl.nkp);
  const int kb0 = __builtin_amdgcn_readfirstlane(tl.kb0);

#define DMAW(SW, KB)                                                                       \
  {                                                                                        \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                          \
      dma16(reinterpret_cast<const uint16_t *>(                                            \
                reinterpret_cast<const char *>(wmat + k0) + wofs[i]),                       \
            (lds_void *)(SW + (dma_row + i * 8) * 64));                                      \
  }
// NX of the 4 token copies: the fragments the loop multiplies
#define DMAX(SX, KB)                                                                       \
  {                                                                                        \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    _Pragma("unroll") for (int i = 0; i < NX; ++i)                                         \
      dma16(xsrc[i] + k0,                                                                  \
            (lds_void *)(SX + (dma_xrow + 64 * (i >> 1) + 8 * (i & 1)) * 64));             \
  }
  // 4 weight + NX token copies per wavefront and k-block, the weights issued last;
  // the prologue waits for k-block 0 with the weights of 1 and 2 and the tokens of
  // 1 in flight (8 + NX copies), each step for all but the last 4 (the weights of
  // KB + 3)
  constexpr int kStepWait = wait_vm_lgkm0(4);
  // Matrix work only for the token fragments that hold rows: the wavefront's
  // fragments below nf = ceil(rows / 16) (4, 3, or 2 and fewer, which take the
  // 2-fragment loop; rows past the tile are the zero row or a repeat, their sums
  // are not stored)
  const int nf = (tl.lim - tl.m0 + 15) >> 4;
  const int nt = (nf - wc + 3) >> 2;
  // (the wavefront with wr = 1 copies fragments wc + 8 and wc + 12: both for 4,
  // the first for 3, none for 2)
  if (nt >= 4) {
    constexpr int NT = 4, NX = 4;
    M16_KLOOP(wait_vm(8 + NX))
  } else if (nt == 3) {
    if (wr == 0) {
      constexpr int NT = 3, NX = 4;
      M16_KLOOP(wait_vm(8 + NX))
    } else {
      constexpr int NT = 3, NX = 2;
      M16_KLOOP(wait_vm(8 + NX))
    }
  } else {
    if (wr == 0) {
      constexpr int NT = 2, NX = 4;
      M16_KLOOP(wait_vm(8 + NX))
    } else {
      constexpr int NT = 2, NX = 0;
      M16_KLOOP(wait_vm(8 + NX))
    }
  }
#undef DMAW
#undef DMAX

  // ---- epilogue: lane holds token 16 (4 t + wc) + (lane & 15) and weight rows
  // 16 f + 4 (lane >> 4) + 0..3 of the wavefront's 128; for gate-up fragments 0-3
  // are g and 4-7 the u of the same 64 columns. Fragments t >= NT lie at or past
  // the tile's end.
  const int ih = 4 * (lane >> 4);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int tok = tl.m0 + 16 * (4 * t + wc) + (lane & 15);
    if (tok >= tl.lim) continue;
    const size_t orow = size_t(tl.row0 + tok) * N + size_t(tl.ks) * size_t(part_stride);
    if constexpr (GATEUP) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int col = tl.c0 + wr * 64 + f * 16 + ih;
        if (col >= N) continue;
        float v[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) v[s] = silu(acc[f][t][s]) * acc[f + 4][t][s];
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + orow + col) = pk;
      }
    } else {
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int col = tl.c0 + wr * 128 + f * 16 + ih;
        if (col >= N) continue;
        *reinterpret_cast<float4 *>(static_cast<float *>(out) + orow + col) =
            make_float4(acc[f][t][0], acc[f][t][1], acc[f][t][2], acc[f][t][3]);
      }
    }
  }
}

// Small batches (an expert holds a few dozen rows): the weight tiles are read
// from HBM once and the matrix work is mostly padding, so the tile narrows to
// BT = 64 or 128 tokens (256 weight rows as before). 8 wavefronts in a 4 x 2
// grid, each 64 weight rows x BT/2 tokens (2 x BT/64 accumulators); for gate-up
// a wavefront's 64 rows are 32 W1 and the same 32 W3 rows. BT = 64 uses two
// stages of both tiles (80 KiB of LDS), so two workgroups share a compute unit
// and keep more bytes in flight; BT = 128 has room for a third weight stage
// (128 KiB) and fetches the weights two k-blocks ahead, as tiled256_kernel.
// The weight copies carry the non-temporal hint: each weight tile is read by
// one token tile (an expert rarely holds more rows than one tile), and on
// MI355X this moved 8-13% more bytes per second at T = 128-384 (the 256-token
// kernel, whose weight tiles are shared by several token tiles, measured no
// better with it). The kernels below own the LDS (separate arrays per slot, so that the compiler
// sees the copies in flight cannot alias the slot being read) and run this body.
template <bool GATEUP, int BT, bool THREE_STAGE>
__device__ __forceinline__ void small_body(
    const Tile &tl, const uint16_t *__restrict__ X, const uint16_t *__restrict__ Wa,
    const uint16_t *__restrict__ Wb, void *__restrict__ out, int N, int K, int ksplit,
    int64_t part_stride, const int32_t *__restrict__ rowmap, uint16_t *sW0, uint16_t *sW1,
    uint16_t *sW2, uint16_t *sX0, uint16_t *sX1) {
  constexpr int NT = BT / 64;  // 32-token accumulator columns per wavefront
  constexpr int XI = BT / 64;  // token-row DMA instructions per wavefront
  const int e = tl.e, row0 = tl.row0, ne = tl.ne, m0 = tl.m0, c0 = tl.c0, ks = tl.ks;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;

  // ---- DMA assignment (8 rows per instruction, as in body256): wave w fills weight rows
  // [32w, 32w+32) (for gate-up: W1 rows if w is even, else the W3 rows of the
  // same 32 columns) and token rows [w*BT/8, (w+1)*BT/8).
  const size_t mat_elems = size_t(N) * K;
  const uint16_t *wmat = Wa + size_t(e) * mat_elems;
  if (GATEUP && (wave & 1)) wmat = Wb + size_t(e) * mat_elems;
  const int xlim = ne - 1 - m0;
  const int dma_row = wave * 32;
  const int dma_xrow = wave * (BT / 8);
  uint32_t wofs[4];
  const uint16_t *xsrc[XI];  // token rows (through the row map if given)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = lane >> 3;
    const int c = (lane & 7) ^ swz(8 * i + lr);
    int wrow;
    if constexpr (GATEUP) wrow = c0 + (wave >> 1) * 32 + 8 * i + lr;
    else wrow = min(c0 + dma_row + 8 * i + lr, N - 1);
    wofs[i] = uint32_t(wrow) * uint32_t(K) + c * 8;
  }
  // (row map entries loaded together, as in body256)
  int xrow[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) xrow[i] = row0 + m0 + min(dma_xrow + 8 * i + (lane >> 3), xlim);
  if (rowmap) {
#pragma unroll
    for (int i = 0; i < XI; ++i) xrow[i] = rowmap[xrow[i]];
  }
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int lr = lane >> 3;
    const int chunk = ((lane & 7) ^ swz(dma_xrow + 8 * i + lr)) << 3;
    xsrc[i] = (dma_xrow + 8 * i + lr > xlim && K <= kZeroK)
                  ? g_zero_row + chunk  // padding row
                  : X + size_t(xrow[i]) * K + chunk;
  }

  // ---- fragment read addresses (bytes): row (lane & 31) of a 32-row group,
  // logical chunk kk*2 + (lane >> 5)
  const int g = (lane >> 5) ^ swz(lane & 31);
  uint32_t offk[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) offk[kk] = uint32_t(((kk * 2) ^ g) * 16);
  const uint32_t baseA = uint32_t((wr * 64 + (lane & 31)) * 128);
  const uint32_t baseB = uint32_t((wc * (BT / 2) + (lane & 31)) * 128);

  constexpr int FA = 2, FB = NT;  // 64 weight rows x BT/2 tokens per wavefront
  f32x16 acc[FA][FB];
#pragma unroll
  for (int f = 0; f < FA; ++f)
#pragma unroll
    for (int t = 0; t < FB; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[f][t][i] = 0.f;
  bf16x8 fa[2][FA], fb[2][FB];

  // k-blocks of this part (an even count) and the first, made scalar as in body256
  const int nk = __builtin_amdgcn_readfirstlane(tl.nkp);
  const int kb0 = __builtin_amdgcn_readfirstlane(tl.kb0);

#define DMAW(SW, KB)                                                                       \
  {                                                                                        \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                          \
      dma16_nt(wmat + wofs[i] + k0, (lds_void *)(SW + (dma_row + i * 8) * 64));            \
  }
#define DMAX(SX, KB)                                                                       \
  {                                                                                        \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    _Pragma("unroll") for (int i = 0; i < XI; ++i)                                         \
      dma16(xsrc[i] + k0, (lds_void *)(SX + (dma_xrow + i * 8) * 64));                    \
  }
  if constexpr (!THREE_STAGE) {
    // two stages of both: the next k-block's copies are issued, the current one
    // is multiplied, then a wait for all copies and a barrier
#define TL_BLOCK(SW, SX)                                                                   \
  TL_READ(SW, SX, 0, 0)                                                                    \
  TL_KSTEP(SW, SX, 1, 1, 0)                                                                \
  TL_KSTEP(SW, SX, 2, 0, 1)                                                                \
  TL_KSTEP(SW, SX, 3, 1, 0)                                                                \
  TL_KLAST(1)
    DMAW(sW0, 0)
    DMAX(sX0, 0)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      DMAW(sW1, kt + 1)
      DMAX(sX1, kt + 1)
      TL_BLOCK(sW0, sX0)
      __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
      __syncthreads();
      DMAW(sW0, kt + 2)
      DMAX(sX0, kt + 2)
      TL_BLOCK(sW1, sX1)
      __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
      __syncthreads();
    }
#undef TL_BLOCK
  } else {
    // as the 256-token tile (4 weight and XI token copies per wavefront and
    // k-block)
    constexpr int kStepWait = wait_vm_lgkm0(4);
    TL_KLOOP(wait_vm(8 + XI))
  }
#undef DMAW
#undef DMAX

  // ---- epilogue: 32 x 32 accumulator layout, lane holds token (lane & 31) of its
  // 32-token column and weight rows 8 q + 4 (lane >> 5) + 0..3 of each 32-row fragment
  const int ih = 4 * (lane >> 5);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = m0 + wc * (BT / 2) + t * 32 + (lane & 31);
    if (tok >= ne) continue;
    const size_t orow = size_t(row0 + tok) * N + size_t(ks) * size_t(part_stride);
    if constexpr (GATEUP) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = c0 + wr * 32 + 8 * q + ih;
        if (col >= N) continue;
        float v[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) v[s] = silu(acc[0][t][4 * q + s]) * acc[1][t][4 * q + s];
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + orow + col) = pk;
      }
    } else {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = c0 + wr * 64 + f * 32 + 8 * q + ih;
          if (col >= N) continue;
          *reinterpret_cast<float4 *>(static_cast<float *>(out) + orow + col) =
              make_float4(acc[f][t][4 * q], acc[f][t][4 * q + 1], acc[f][t][4 * q + 2],
                          acc[f][t][4 * q + 3]);
        }
      }
    }
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(512) void tiled64_kernel(
    const uint16_t *__restrict__ X, const int32_t *__restrict__ offsets, int E,
    const uint16_t *__restrict__ Wa, const uint16_t *__restrict__ Wb, void *__restrict__ out,
    int N, int K, int ksplit, int64_t part_stride, const int32_t *__restrict__ rowmap) {
  __shared__ __attribute__((aligned(1024))) uint16_t sW0[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sW1[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX0[64 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX1[64 * 64];
  Tile tl;
  if (!find_tile<64, GATEUP ? 128 : 256>(offsets, E, N, K, ksplit, tl)) return;
  small_body<GATEUP, 64, false>(tl, X, Wa, Wb, out, N, K, ksplit, part_stride, rowmap, sW0, sW1,
                                nullptr, sX0, sX1);
}

template <bool GATEUP>
__global__ __launch_bounds__(512) void tiled128_kernel(
    const uint16_t *__restrict__ X, const int32_t *__restrict__ offsets, int E,
    const uint16_t *__restrict__ Wa, const uint16_t *__restrict__ Wb, void *__restrict__ out,
    int N, int K, int ksplit, int64_t part_stride, const int32_t *__restrict__ rowmap) {
  __shared__ __attribute__((aligned(1024))) uint16_t sW0[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sW1[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sW2[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX0[128 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX1[128 * 64];
  Tile tl;
  if (!find_tile<128, GATEUP ? 128 : 256>(offsets, E, N, K, ksplit, tl)) return;
  small_body<GATEUP, 128, true>(tl, X, Wa, Wb, out, N, K, ksplit, part_stride, rowmap, sW0, sW1,
                                sW2, sX0, sX1);
}

// Experts of more than a few hundred rows: up to 256 tokens per tile (body256),
// an expert's ceil(rows / 256) tiles splitting its rows evenly (an expert of 1062
// rows: 5 tiles of 212-213 rows, 14 fragments, instead of 4 x 256 and 38), and
// each wavefront multiplying only its fragments that hold rows. The tiles of one
// expert and column block then run the same length and stay in step through the
// k-loop, so that the weight slices they share are fetched once. On MI355X in one
// process, interleaved: gate-up 1.565 -> 1.520 ms and down 0.864 -> 0.849 ms at
// the prefill_8x7b routing (matrix work 12.5% -> 3.7% above the algorithmic), 1%
// at skew_8x7b, 8% at a ragged routing of 2200 rows, bitwise the same outputs.
// Narrowing only the last tile to 64 or 128 tokens was no faster and doubled the
// HBM reads (3.1 -> 5.9 GB per gate-up launch): a narrow tail runs ahead of its
// expert's full tiles and fetches the shared weight slices first, which the full
// tiles then find evicted from L2; running all tails after the full tiles cut that
// to 4.7 GB and was slower.
template <bool GATEUP>
__global__ __launch_bounds__(512) void tiled256_kernel(
    const uint16_t *__restrict__ X, const int32_t *__restrict__ offsets, int E,
    const uint16_t *__restrict__ Wa, const uint16_t *__restrict__ Wb, void *__restrict__ out,
    int N, int K, int ksplit, int64_t part_stride, const int32_t *__restrict__ rowmap) {
  __shared__ __attribute__((aligned(1024))) uint16_t sW0[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sW1[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sW2[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX0[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX1[256 * 64];
  Tile tl;
  if (!find_tile<256, GATEUP ? 128 : 256, true>(offsets, E, N, K, ksplit, tl)) return;
  body256<GATEUP>(tl, X, Wa, Wb, out, N, K, ksplit, part_stride, rowmap, sW0, sW1, sW2, sX0, sX1);
}

// Upper bound of the tile count for any split of S rows over E experts.
// (per part, an XCD gets at most ceil(tiles / 8) tiles in the contiguous order and
// at most ceil(ct / 8) column blocks of every token block in the round-robin order
// of the 256-token tiles)
inline unsigned tiled_grid(int64_t S, int E, int N, int cols, int bt, int ksplit) {
  const int64_t ct = (N + cols - 1) / cols;
  const int64_t mt = (S + bt - 1) / bt + E;  // token blocks, at most
  const int64_t per_xcd = bt == 256 ? (ct + kXCD - 1) / kXCD * mt : (ct * mt + kXCD - 1) / kXCD;
  return unsigned(per_xcd * kXCD * ksplit);
}

template <bool GATEUP>
void launch_bt(int bt, const void *x, const int32_t *rowmap, const int32_t *offsets,
               const void *wa, const void *wb, void *out, int E, int64_t S, int N, int K,
               int ksplit, int64_t part_stride, hipStream_t s) {
  const dim3 grid(tiled_grid(S, E, N, GATEUP ? 128 : 256, bt, ksplit));
  const auto *xp = static_cast<const uint16_t *>(x);
  const auto *ap = static_cast<const uint16_t *>(wa);
  const auto *bp = static_cast<const uint16_t *>(wb);
  if (bt == 128)
    hipLaunchKernelGGL((tiled128_kernel<GATEUP>), grid, dim3(512), 0, s, xp, offsets, E, ap, bp,
                       out, N, K, ksplit, part_stride, rowmap);
  else if (bt == 64)
    hipLaunchKernelGGL((tiled64_kernel<GATEUP>), grid, dim3(512), 0, s, xp, offsets, E, ap, bp,
                       out, N, K, ksplit, part_stride, rowmap);
  else
    hipLaunchKernelGGL((tiled256_kernel<GATEUP>), grid, dim3(512), 0, s, xp, offsets, E, ap, bp,
                       out, N, K, ksplit, part_stride, rowmap);
}

}  // namespace

hipError_t launch_tiled_gate_up(const void *x_perm, const int32_t *rowmap, const int32_t *offsets,
                                const void *w1, const void *w3, void *act, int E, int64_t S,
                                int d, int h, int bt, hipStream_t s) {
  launch_bt<true>(bt, x_perm, rowmap, offsets, w1, w3, act, E, S, h, d, 1, 0, s);
  return hipGetLastError();
}

hipError_t launch_tiled_down(const void *act, const int32_t *offsets, const void *w2,
                             float *o_perm, int E, int64_t S, int d, int h, int bt, int parts,
                             hipStream_t s) {
  launch_bt<false>(bt, act, nullptr, offsets, w2, nullptr, o_perm, E, S, d, h, parts, S * d, s);
  return hipGetLastError();
}

}  // namespace moe
