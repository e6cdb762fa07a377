// gemm_tiled.hip -- expert projections for large batches: grouped bf16 GEMM on
// the CDNA4 matrix cores.
//
// Each expert's rows form one contiguous segment of the sorted activations, so
// the layer is a grouped GEMM C_e = X_e W_e^T with both operands K-contiguous
// (Mixtral of Experts, notion page "Implementation": SwiGLU experts with K = 2;
// the sparse-matmul kernels the pages cite are prior art, this is a plain
// grouped GEMM over the per-expert segments).
//
// Tile: 256 weight rows (MFMA M side) x BT tokens (MFMA N side, BT = 256 or
// 384) x 64 k.
//  * 8 wavefronts (2 per SIMD) in a 2 x 4 grid; each owns 128 weight rows x
//    BT/4 tokens as 4 x BT/128 accumulators of v_mfma_f32_32x32x16_bf16. Two
//    wavefronts per SIMD keep the matrix pipe fed while the other waits on LDS
//    or a barrier. BT = 384 is the largest tile whose accumulators (192
//    registers) fit two wavefronts per SIMD; it moves 17% fewer bytes from L2
//    per flop than BT = 256, which it replaces once experts hold >= 256 rows
//    on average (with fewer rows the wider tile only adds padding).
//  * Global memory goes straight to LDS (global_load_lds_dwordx4: a wavefront
//    instruction fills one contiguous kilobyte, lane L the bytes [16L, 16L+16)),
//    two stages (64 or 80 KiB each); the k-block after the current one is in
//    flight while the current one is multiplied; one barrier per k-block.
//  * LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled by
//    (r ^ r >> 3) & 7 of the row's position in its 32-row group, so both the
//    DMA writes and the fragment reads of 8 or 16 consecutive rows hit distinct
//    banks (measured: zero bank conflicts).
//  * Gate-up: the 256 weight rows are W1 and W3 rows of the same 128 output
//    columns, interleaved in blocks of 64 so that every wavefront holds g and u
//    of the same columns and applies silu(g) * u in registers; the result is
//    rounded once to bf16. Down: 256 W2 rows = 256 output columns, float32 out.
//  * Tiles are ordered (expert, column block, token block) with the token block
//    fastest, so concurrently running tiles share weight tiles; the linear tile
//    id is remapped so that each of the 8 XCDs (workgroups are dealt to XCDs
//    round-robin) owns one contiguous range of tiles and its own L2 sees the
//    reuse. Token rows past an expert's end are clamped duplicates whose results
//    are never stored.
//  * Down can split the sum over h into `ksplit` parts: each part is a tile of
//    its own writing float32 partial sums that the combine step adds in a fixed
//    order, so that the last round of tiles fills the GPU.
#include "kernels.h"

namespace moe {
namespace {

constexpr int kXCD = 8;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate with vmcnt(0) and the other counters at their maximum.
constexpr int kWaitVm0 = 0x0F70;

// Physical 16-byte chunk = logical chunk ^ swz(row); depends on row & 31 only.
__device__ __forceinline__ int swz(int r) { return ((r & 31) ^ ((r & 31) >> 3)) & 7; }

template <bool GATEUP, int BT>
__global__ __launch_bounds__(512) void tiled_kernel(const uint16_t *__restrict__ X,
                                                     const int32_t *__restrict__ offsets, int E,
                                                     const uint16_t *__restrict__ Wa,
                                                     const uint16_t *__restrict__ Wb,
                                                     void *__restrict__ out, int N, int K,
                                                     int ksplit, int64_t part_stride) {
  constexpr int NT = BT / 128;        // 32-token accumulator columns per wavefront
  constexpr int XI = BT / 64;         // token-row DMA instructions per wavefront
  constexpr int kCols = GATEUP ? 128 : 256;
  const int ct = (N + kCols - 1) / kCols;
  int total = 0;
  for (int q = 0; q < E; ++q) total += ct * ((offsets[q + 1] - offsets[q] + BT - 1) / BT);
  // ksplit > 1 (down only): the sum over K is cut into ksplit ranges, part ks
  // writing its float32 partial sums to out + ks * part_stride
  const int g8 = (total * ksplit + kXCD - 1) / kXCD;
  const int b = blockIdx.x;
  if (b >= g8 * kXCD) return;
  int L = (b % kXCD) * g8 + b / kXCD;
  if (L >= total * ksplit) return;
  const int ks = L / total;
  L -= ks * total;
  int e = 0, row0 = 0, ne = 0, mtiles = 0;
  for (; e < E; ++e) {
    row0 = offsets[e];
    ne = offsets[e + 1] - row0;
    mtiles = (ne + BT - 1) / BT;
    if (L < ct * mtiles) break;
    L -= ct * mtiles;
  }
  const int cb = L / mtiles;
  const int m0 = (L % mtiles) * BT;
  const int c0 = cb * kCols;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // (BT = 384 keeps wave-uniform values in scalar registers: the vector
  // registers are all but taken by its accumulators)
  const int wave = BT == 384 ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int wr = wave >> 2, wc = wave & 3;

  __shared__ __attribute__((aligned(1024))) uint16_t sW0[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sW1[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX0[BT * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX1[BT * 64];

  // ---- DMA assignment: wave w fills weight rows [32w, 32w+32) and token rows
  // [w*BT/8, (w+1)*BT/8), 8 rows per instruction; lane p writes LDS bytes
  // [16p, 16p+16) of the instruction's kilobyte: row 8i + p/8, physical chunk
  // p%8 = logical chunk ^ swz(row). Instruction i of a share starting at row s
  // covers position 8 * ((s/8 + i) & 3) + p/8 of a 32-row group.
  const size_t mat_elems = size_t(N) * K;
  const uint16_t *wmat = Wa + size_t(e) * mat_elems;
  if (GATEUP && ((wave >> 1) & 1)) wmat = Wb + size_t(e) * mat_elems;
  const uint16_t *x_t = X + size_t(row0 + m0) * K;
  const int wrow0 = GATEUP ? c0 + (wave >> 2) * 64 + (wave & 1) * 32 : c0 + wave * 32;
  const int xlim = ne - 1 - m0;
  const int dma_row = wave * 32;
  const int dma_xrow = wave * (BT / 8);
  // BT = 256: the per-lane DMA offsets are computed once (registers to spare)
  uint32_t wofs[4], xofs[4];
  if constexpr (BT == 256) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 32 + i * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      int wrow;
      if constexpr (GATEUP) wrow = c0 + ((r >> 7) << 6) + (r & 63);
      else wrow = min(c0 + r, N - 1);
      wofs[i] = uint32_t(wrow) * uint32_t(K) + c * 8;
      xofs[i] = uint32_t(min(r, xlim)) * uint32_t(K) + c * 8;
    }
  }

  // ---- fragment read addresses (bytes): row (lane & 31) of a 32-row group,
  // logical chunk kk*2 + (lane >> 5)
  const int g = (lane >> 5) ^ swz(lane & 31);
  uint32_t offk0[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) offk0[kk] = uint32_t(((kk * 2) ^ g) * 16);
  const uint32_t baseA = uint32_t((wr * 128 + (lane & 31)) * 128);
  const uint32_t baseB = uint32_t((wc * (BT / 4) + (lane & 31)) * 128);

  f32x16 acc[4][NT];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[f][t][i] = 0.f;

  const int nk = K / 64 / ksplit;  // k-blocks of this part (an even count)
  const int kb0 = ks * nk;

  // BT = 384: the DMA and fragment addresses are recomputed from opaque
  // copies of the lane values at each use, so that they hold no registers
  // across the main loop (its accumulators leave almost none).
#define DMA(SW, SX, KB)                                                                    \
  if constexpr (BT == 256) {                                                               \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                        \
      __builtin_amdgcn_global_load_lds(wmat + wofs[i] + k0,                                \
                                       (lds_void *)(SW + (dma_row + i * 8) * 64), 16, 0, 0); \
      __builtin_amdgcn_global_load_lds(x_t + xofs[i] + k0,                                 \
                                       (lds_void *)(SX + (dma_row + i * 8) * 64), 16, 0, 0); \
    }                                                                                      \
  } else {                                                                                 \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    int ln = lane;                                                                         \
    asm volatile("" : "+v"(ln));                                                           \
    const int lr = ln >> 3, lc = ln & 7;                                                   \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                        \
      const int wrow = GATEUP ? wrow0 + 8 * i + lr : min(wrow0 + 8 * i + lr, N - 1);      \
      const uint32_t o = uint32_t(wrow) * uint32_t(K) + ((lc ^ lr ^ i) << 3) + k0;         \
      __builtin_amdgcn_global_load_lds(wmat + o, (lds_void *)(SW + (dma_row + i * 8) * 64), \
                                       16, 0, 0);                                          \
    }                                                                                      \
    _Pragma("unroll") for (int i = 0; i < XI; ++i) {                                       \
      const int xrow = min(dma_xrow + 8 * i + lr, xlim);                                   \
      const int q = (dma_xrow / 8 + i) & 3;                                                \
      const uint32_t o = uint32_t(xrow) * uint32_t(K) + ((lc ^ lr ^ q) << 3) + k0;         \
      __builtin_amdgcn_global_load_lds(x_t + o, (lds_void *)(SX + (dma_xrow + i * 8) * 64), \
                                       16, 0, 0);                                          \
    }                                                                                      \
  }
  // NT = 2: both fragment sets double-buffered, the next kk's six reads issued
  // ahead of the current kk's eight MFMAs. NT = 3 (no registers for that): the
  // token fragments double-buffered, each weight fragment reloaded for the next
  // kk as soon as its three MFMAs are issued.
#define COMPUTE(SW, SX)                                                                    \
  {                                                                                        \
    const char *pa = reinterpret_cast<const char *>(SW) + baseA;                           \
    const char *pb = reinterpret_cast<const char *>(SX) + baseB;                           \
    if constexpr (NT == 2) {                                                               \
      const uint32_t *offk = offk0;                                                        \
      bf16x8 fa[2][4], fb[2][2];                                                           \
      _Pragma("unroll") for (int f = 0; f < 4; ++f)                                        \
        fa[0][f] = *reinterpret_cast<const bf16x8 *>(pa + f * 4096 + offk[0]);             \
      _Pragma("unroll") for (int t = 0; t < 2; ++t)                                        \
        fb[0][t] = *reinterpret_cast<const bf16x8 *>(pb + t * 4096 + offk[0]);             \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                                   \
        const int cur = kk & 1;                                                            \
        if (kk + 1 < 4) {                                                                  \
          _Pragma("unroll") for (int f = 0; f < 4; ++f) fa[cur ^ 1][f] =                   \
              *reinterpret_cast<const bf16x8 *>(pa + f * 4096 + offk[kk + 1]);             \
          _Pragma("unroll") for (int t = 0; t < 2; ++t) fb[cur ^ 1][t] =                   \
              *reinterpret_cast<const bf16x8 *>(pb + t * 4096 + offk[kk + 1]);             \
        }                                                                                  \
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);                                 \
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);                                 \
        _Pragma("unroll") for (int t = 0; t < 2; ++t)                                      \
          _Pragma("unroll") for (int f = 0; f < 4; ++f)                                    \
            acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][f], fb[cur][t],    \
                                                                acc[f][t], 0, 0, 0);       \
        __builtin_amdgcn_sched_barrier(0);                                                 \
      }                                                                                    \
    } else {                                                                               \
      int gg = g;                                                                          \
      asm volatile("" : "+v"(gg));                                                         \
      uint32_t offk[4];                                                                    \
      _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) offk[kk] = uint32_t(((kk * 2) ^ gg) * 16); \
      bf16x8 fa[4], fb[2][NT];                                                             \
      _Pragma("unroll") for (int t = 0; t < NT; ++t)                                       \
        fb[0][t] = *reinterpret_cast<const bf16x8 *>(pb + t * 4096 + offk[0]);             \
      _Pragma("unroll") for (int f = 0; f < 4; ++f)                                        \
        fa[f] = *reinterpret_cast<const bf16x8 *>(pa + f * 4096 + offk[0]);                \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                                   \
        const int cur = kk & 1;                                                            \
        if (kk + 1 < 4) {                                                                  \
          _Pragma("unroll") for (int t = 0; t < NT; ++t) fb[cur ^ 1][t] =                  \
              *reinterpret_cast<const bf16x8 *>(pb + t * 4096 + offk[kk + 1]);             \
          __builtin_amdgcn_sched_group_barrier(0x100, NT, 0);                              \
        }                                                                                  \
        _Pragma("unroll") for (int f = 0; f < 4; ++f) {                                    \
          _Pragma("unroll") for (int t = 0; t < NT; ++t)                                   \
            acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f], fb[cur][t],         \
                                                                acc[f][t], 0, 0, 0);       \
          __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);                              \
          if (kk + 1 < 4) {                                                                \
            fa[f] = *reinterpret_cast<const bf16x8 *>(pa + f * 4096 + offk[kk + 1]);       \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                             \
          }                                                                                \
        }                                                                                  \
        __builtin_amdgcn_sched_barrier(0);                                                 \
      }                                                                                    \
    }                                                                                      \
  }

  DMA(sW0, sX0, 0)
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    DMA(sW1, sX1, kt + 1)
    COMPUTE(sW0, sX0)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    DMA(sW0, sX0, kt + 2)
    COMPUTE(sW1, sX1)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  }
#undef DMA
#undef COMPUTE

  // ---- epilogue: lane holds token column j = lane & 31 and weight rows
  // i = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4) of each 32x32 fragment.
  const int ih = 4 * (lane >> 5);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = m0 + wc * (BT / 4) + t * 32 + (lane & 31);
    if (tok >= ne) continue;
    const size_t orow = size_t(row0 + tok) * N + size_t(ks) * size_t(part_stride);
    if constexpr (GATEUP) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = c0 + wr * 64 + f * 32 + 8 * q + ih;
          if (col >= N) continue;
          float v[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) v[s] = silu(acc[f][t][4 * q + s]) * acc[f + 2][t][4 * q + s];
          uint2 pk;
          pk.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
          pk.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
          *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + orow + col) = pk;
        }
      }
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = c0 + wr * 128 + f * 32 + 8 * q + ih;
          if (col >= N) continue;
          *reinterpret_cast<float4 *>(static_cast<float *>(out) + orow + col) =
              make_float4(acc[f][t][4 * q], acc[f][t][4 * q + 1], acc[f][t][4 * q + 2],
                          acc[f][t][4 * q + 3]);
        }
      }
    }
  }
}

// One global -> LDS copy of 16 bytes per lane (a plain function: the builtin
// inside a kernel template can fail the template's host-side instantiation).
__device__ __forceinline__ void dma16(const uint16_t *g, lds_void *l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

// Small batches (an expert holds a few dozen rows): the weight tiles are read
// from HBM once and the matrix work is mostly padding, so the tile narrows to
// BT = 64 or 128 tokens (256 weight rows as before). 8 wavefronts in a 4 x 2
// grid, each 64 weight rows x BT/2 tokens (2 x BT/64 accumulators); for gate-up
// a wavefront's 64 rows are 32 W1 and the same 32 W3 rows. BT = 64 needs 80 KiB
// of LDS, so two workgroups share a compute unit and keep more bytes in flight.
template <bool GATEUP, int BT>
__global__ __launch_bounds__(512) void tiled_small_kernel(
    const uint16_t *__restrict__ X, const int32_t *__restrict__ offsets, int E,
    const uint16_t *__restrict__ Wa, const uint16_t *__restrict__ Wb, void *__restrict__ out,
    int N, int K, int ksplit, int64_t part_stride) {
  constexpr int NT = BT / 64;  // 32-token accumulator columns per wavefront
  constexpr int XI = BT / 64;  // token-row DMA instructions per wavefront
  constexpr int kCols = GATEUP ? 128 : 256;
  const int ct = (N + kCols - 1) / kCols;
  int total = 0;
  for (int q = 0; q < E; ++q) total += ct * ((offsets[q + 1] - offsets[q] + BT - 1) / BT);
  const int g8 = (total * ksplit + kXCD - 1) / kXCD;
  const int b = blockIdx.x;
  if (b >= g8 * kXCD) return;
  int L = (b % kXCD) * g8 + b / kXCD;
  if (L >= total * ksplit) return;
  const int ks = L / total;
  L -= ks * total;
  int e = 0, row0 = 0, ne = 0, mtiles = 0;
  for (; e < E; ++e) {
    row0 = offsets[e];
    ne = offsets[e + 1] - row0;
    mtiles = (ne + BT - 1) / BT;
    if (L < ct * mtiles) break;
    L -= ct * mtiles;
  }
  const int cb = L / mtiles;
  const int m0 = (L % mtiles) * BT;
  const int c0 = cb * kCols;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  __shared__ __attribute__((aligned(1024))) uint16_t sW0[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sW1[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX0[BT * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX1[BT * 64];

  // ---- DMA assignment as in tiled_kernel: wave w fills weight rows
  // [32w, 32w+32) (for gate-up: W1 rows if w is even, else the W3 rows of the
  // same 32 columns) and token rows [w*BT/8, (w+1)*BT/8).
  const size_t mat_elems = size_t(N) * K;
  const uint16_t *wmat = Wa + size_t(e) * mat_elems;
  if (GATEUP && (wave & 1)) wmat = Wb + size_t(e) * mat_elems;
  const uint16_t *x_t = X + size_t(row0 + m0) * K;
  const int xlim = ne - 1 - m0;
  const int dma_row = wave * 32;
  const int dma_xrow = wave * (BT / 8);
  uint32_t wofs[4], xofs[XI];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = lane >> 3;
    const int c = (lane & 7) ^ lr ^ i;  // swz of row 8i + lr in its 32-row group
    int wrow;
    if constexpr (GATEUP) wrow = c0 + (wave >> 1) * 32 + 8 * i + lr;
    else wrow = min(c0 + dma_row + 8 * i + lr, N - 1);
    wofs[i] = uint32_t(wrow) * uint32_t(K) + c * 8;
  }
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int lr = lane >> 3;
    const int q = (dma_xrow / 8 + i) & 3;
    xofs[i] = uint32_t(min(dma_xrow + 8 * i + lr, xlim)) * uint32_t(K) +
              (((lane & 7) ^ lr ^ q) << 3);
  }

  // ---- fragment read addresses (bytes): row (lane & 31) of a 32-row group,
  // logical chunk kk*2 + (lane >> 5)
  const int g = (lane >> 5) ^ swz(lane & 31);
  uint32_t offk[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) offk[kk] = uint32_t(((kk * 2) ^ g) * 16);
  const uint32_t baseA = uint32_t((wr * 64 + (lane & 31)) * 128);
  const uint32_t baseB = uint32_t((wc * (BT / 2) + (lane & 31)) * 128);

  f32x16 acc[2][NT];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[f][t][i] = 0.f;

  const int nk = K / 64 / ksplit;  // k-blocks of this part (an even count)
  const int kb0 = ks * nk;

#define DMA(SW, SX, KB)                                                                    \
  {                                                                                        \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                          \
      dma16(wmat + wofs[i] + k0, (lds_void *)(SW + (dma_row + i * 8) * 64));              \
    _Pragma("unroll") for (int i = 0; i < XI; ++i)                                         \
      dma16(x_t + xofs[i] + k0, (lds_void *)(SX + (dma_xrow + i * 8) * 64));              \
  }
#define COMPUTE(SW, SX)                                                                    \
  {                                                                                        \
    const char *pa = reinterpret_cast<const char *>(SW) + baseA;                           \
    const char *pb = reinterpret_cast<const char *>(SX) + baseB;                           \
    bf16x8 fa[2][2], fb[2][NT];                                                            \
    _Pragma("unroll") for (int f = 0; f < 2; ++f)                                          \
      fa[0][f] = *reinterpret_cast<const bf16x8 *>(pa + f * 4096 + offk[0]);               \
    _Pragma("unroll") for (int t = 0; t < NT; ++t)                                         \
      fb[0][t] = *reinterpret_cast<const bf16x8 *>(pb + t * 4096 + offk[0]);               \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                                     \
      const int cur = kk & 1;                                                              \
      if (kk + 1 < 4) {                                                                    \
        _Pragma("unroll") for (int f = 0; f < 2; ++f) fa[cur ^ 1][f] =                     \
            *reinterpret_cast<const bf16x8 *>(pa + f * 4096 + offk[kk + 1]);               \
        _Pragma("unroll") for (int t = 0; t < NT; ++t) fb[cur ^ 1][t] =                    \
            *reinterpret_cast<const bf16x8 *>(pb + t * 4096 + offk[kk + 1]);               \
      }                                                                                    \
      __builtin_amdgcn_sched_group_barrier(0x100, 2 + NT, 1);                              \
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NT, 1);                              \
      _Pragma("unroll") for (int t = 0; t < NT; ++t)                                       \
        _Pragma("unroll") for (int f = 0; f < 2; ++f)                                      \
          acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][f], fb[cur][t],      \
                                                              acc[f][t], 0, 0, 0);         \
      __builtin_amdgcn_sched_barrier(0);                                                   \
    }                                                                                      \
  }

  DMA(sW0, sX0, 0)
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    DMA(sW1, sX1, kt + 1)
    COMPUTE(sW0, sX0)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    DMA(sW0, sX0, kt + 2)
    COMPUTE(sW1, sX1)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  }
#undef DMA
#undef COMPUTE

  // ---- epilogue (fragment layout as in tiled_kernel)
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
        pk.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
        pk.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
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

// Upper bound of the tile count for any split of S rows over E experts.
inline unsigned tiled_grid(int64_t S, int E, int N, int cols, int bt, int ksplit) {
  const int64_t ct = (N + cols - 1) / cols;
  const int64_t tiles = ksplit * ct * ((S + bt - 1) / bt + E);
  return unsigned((tiles + kXCD - 1) / kXCD * kXCD);
}

template <bool GATEUP, int BT>
void launch_t(const void *x, const int32_t *offsets, const void *wa, const void *wb, void *out,
              int E, int64_t S, int N, int K, int ksplit, int64_t part_stride, hipStream_t s) {
  hipLaunchKernelGGL((tiled_kernel<GATEUP, BT>),
                     dim3(tiled_grid(S, E, N, GATEUP ? 128 : 256, BT, ksplit)), dim3(512), 0, s,
                     static_cast<const uint16_t *>(x), offsets, E,
                     static_cast<const uint16_t *>(wa), static_cast<const uint16_t *>(wb), out, N,
                     K, ksplit, part_stride);
}

template <bool GATEUP, int BT>
void launch_small(const void *x, const int32_t *offsets, const void *wa, const void *wb,
                  void *out, int E, int64_t S, int N, int K, int ksplit, int64_t part_stride,
                  hipStream_t s) {
  hipLaunchKernelGGL((tiled_small_kernel<GATEUP, BT>),
                     dim3(tiled_grid(S, E, N, GATEUP ? 128 : 256, BT, ksplit)), dim3(512), 0, s,
                     static_cast<const uint16_t *>(x), offsets, E,
                     static_cast<const uint16_t *>(wa), static_cast<const uint16_t *>(wb), out, N,
                     K, ksplit, part_stride);
}

}  // namespace

hipError_t launch_tiled_gate_up(const void *x_perm, const int32_t *offsets, const void *w1,
                                const void *w3, void *act, int E, int64_t S, int d, int h,
                                int bt, hipStream_t s) {
  if (bt == 384)
    launch_t<true, 384>(x_perm, offsets, w1, w3, act, E, S, h, d, 1, 0, s);
  else if (bt == 128)
    launch_small<true, 128>(x_perm, offsets, w1, w3, act, E, S, h, d, 1, 0, s);
  else if (bt == 64)
    launch_small<true, 64>(x_perm, offsets, w1, w3, act, E, S, h, d, 1, 0, s);
  else
    launch_t<true, 256>(x_perm, offsets, w1, w3, act, E, S, h, d, 1, 0, s);
  return hipGetLastError();
}

hipError_t launch_tiled_down(const void *act, const int32_t *offsets, const void *w2,
                             float *o_perm, int E, int64_t S, int d, int h, int bt, int parts,
                             hipStream_t s) {
  if (bt == 384)
    launch_t<false, 384>(act, offsets, w2, nullptr, o_perm, E, S, d, h, parts, S * d, s);
  else if (bt == 128)
    launch_small<false, 128>(act, offsets, w2, nullptr, o_perm, E, S, d, h, parts, S * d, s);
  else if (bt == 64)
    launch_small<false, 64>(act, offsets, w2, nullptr, o_perm, E, S, d, h, parts, S * d, s);
  else
    launch_t<false, 256>(act, offsets, w2, nullptr, o_perm, E, S, d, h, parts, S * d, s);
  return hipGetLastError();
}

}  // namespace moe
