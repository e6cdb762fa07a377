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
//    rows x 64 tokens as 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16. Two
//    wavefronts per SIMD keep the matrix pipe fed while the other waits on LDS
//    or a barrier. The LDS holds three weight stages, so weight tiles are
//    fetched two k-blocks ahead of their use.
//  * Global memory goes straight to LDS (global_load_lds_dwordx4: a wavefront
//    instruction fills one contiguous kilobyte, lane L the bytes [16L, 16L+16));
//    one barrier per k-block.
//  * LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled by
//    (r ^ r >> 3) & 7 of the row's position in its 32-row group, so both the
//    DMA writes and the fragment reads of 8 or 16 consecutive rows hit distinct
//    banks (measured: zero bank conflicts).
//  * Gate-up: the 256 weight rows are W1 and W3 rows of the same 128 output
//    columns, interleaved so that every wavefront holds g and u of the same
//    columns and applies silu(g) * u in registers; the result is rounded once to
//    bf16. Down: 256 W2 rows = 256 output columns, float32 out.
//  * Tiles are ordered (expert, column block, token block) with the token block
//    fastest, so concurrently running tiles share weight tiles; the linear tile
//    id is remapped so that each of the 8 XCDs (workgroups are dealt to XCDs
//    round-robin) owns one contiguous range of tiles and its own L2 sees the
//    reuse. Token rows past an expert's end read a row of zeros (g_zero_row);
//    their results are never stored.
//  * Down can split the sum over h into `ksplit` parts: each part is a tile of
//    its own writing float32 partial sums that the combine step adds in a fixed
//    order, so that the last round of tiles fills the GPU.
//  * Every variant sums each output over k in the same order (64-wide k-blocks
//    in order, 16-wide MFMA steps within), so the tile width changes no bit of
//    the result.
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

// s_waitcnt immediates: vmcnt(0) / vmcnt(4) with the other counters at their maximum.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVm4 = 0x0F74;

// Workgroup barrier without the fence of __syncthreads() (which would wait for
// every copy in flight); the explicit vmcnt waits before it are the ones the
// pipeline needs, the empty asm keeps LDS accesses on their side of it.
#define TILED_BARRIER()                  \
  {                                      \
    asm volatile("" ::: "memory");       \
    __builtin_amdgcn_s_barrier();        \
    asm volatile("" ::: "memory");       \
  }

// Physical 16-byte chunk = logical chunk ^ swz(row); depends on row & 31 only.
__device__ __forceinline__ int swz(int r) { return ((r & 31) ^ ((r & 31) >> 3)) & 7; }

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
// block m0, output column c0 and, with ksplit > 1 (down only), the part ks of
// the sum over K. False when the workgroup has no tile.
struct Tile {
  int e, row0, ne, m0, c0, ks;
};
template <int BT, int kCols>
__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offsets, int E, int N,
                                          int ksplit, Tile &tl) {
  const int ct = (N + kCols - 1) / kCols;
  int total = 0;
  for (int q = 0; q < E; ++q) total += ct * ((offsets[q + 1] - offsets[q] + BT - 1) / BT);
  const int g8 = (total * ksplit + kXCD - 1) / kXCD;
  const int b = blockIdx.x;
  if (b >= g8 * kXCD) return false;
  int L = (b % kXCD) * g8 + b / kXCD;
  if (L >= total * ksplit) return false;
  tl.ks = L / total;
  L -= tl.ks * total;
  int e = 0, row0 = 0, ne = 0, mtiles = 0;
  for (; e < E; ++e) {
    row0 = offsets[e];
    ne = offsets[e + 1] - row0;
    mtiles = (ne + BT - 1) / BT;
    if (L < ct * mtiles) break;
    L -= ct * mtiles;
  }
  tl.e = e;
  tl.row0 = row0;
  tl.ne = ne;
  tl.m0 = (L % mtiles) * BT;
  tl.c0 = (L / mtiles) * kCols;
  return true;
}

// Epilogue of the 2 x 4 wavefront grid (BT = 256): lane holds token column j = lane & 31
// and weight rows i = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4) of each 32x32
// fragment; gate-up fragments 0, 1 are g and 2, 3 the u of the same columns.
template <bool GATEUP, int BT>
__device__ __forceinline__ void store_2x4(const f32x16 (&acc)[4][BT / 128], const Tile &tl,
                                          int lane, int wr, int wc, int N,
                                          int64_t part_stride, void *__restrict__ out) {
  constexpr int NT = BT / 128;
  const int ih = 4 * (lane >> 5);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = tl.m0 + wc * (BT / 4) + t * 32 + (lane & 31);
    if (tok >= tl.ne) continue;
    const size_t orow = size_t(tl.row0 + tok) * N + size_t(tl.ks) * size_t(part_stride);
    if constexpr (GATEUP) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = tl.c0 + wr * 64 + f * 32 + 8 * q + ih;
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
          const int col = tl.c0 + wr * 128 + f * 32 + 8 * q + ih;
          if (col >= N) continue;
          *reinterpret_cast<float4 *>(static_cast<float *>(out) + orow + col) =
              make_float4(acc[f][t][4 * q], acc[f][t][4 * q + 1], acc[f][t][4 * q + 2],
                          acc[f][t][4 * q + 3]);
        }
      }
    }
  }
}

// BT = 256: three weight stages and two token stages (160 KiB of LDS). Per
// k-block: the token tile one k-block ahead and the weight tile two k-blocks
// ahead are issued, the current k-block is multiplied, then a wait for all but
// the 4 youngest copies (the weights two ahead) and a barrier. The weight tile
// of the first token block to reach a k-block is an HBM miss; two k-blocks of
// lead hide more of that latency than one (measured 4-9% faster than two
// stages of both).
template <bool GATEUP>
__global__ __launch_bounds__(512) void tiled256_kernel(const uint16_t *__restrict__ X,
                                                       const int32_t *__restrict__ offsets, int E,
                                                       const uint16_t *__restrict__ Wa,
                                                       const uint16_t *__restrict__ Wb,
                                                       void *__restrict__ out, int N, int K,
                                                       int ksplit, int64_t part_stride,
                                                       const int32_t *__restrict__ rowmap) {
  constexpr int BT = 256;
  Tile tl;
  if (!find_tile<BT, GATEUP ? 128 : 256>(offsets, E, N, ksplit, tl)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 2, wc = wave & 3;

  __shared__ __attribute__((aligned(1024))) uint16_t sW0[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sW1[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sW2[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX0[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX1[256 * 64];

  // ---- DMA assignment: wave w fills rows [32w, 32w+32) of both tiles, 8 rows
  // per instruction; lane p writes LDS bytes [16p, 16p+16) of the
  // instruction's kilobyte: row 8i + p/8, physical chunk p%8 = logical chunk ^
  // swz(row). Gate-up weight rows: 64 W1 rows, the W3 rows of the same
  // columns, the next 64 W1 rows, their W3 rows.
  const size_t mat_elems = size_t(N) * K;
  const uint16_t *wmat = Wa + size_t(tl.e) * mat_elems;
  if (GATEUP && ((wave >> 1) & 1)) wmat = Wb + size_t(tl.e) * mat_elems;
  // token rows: x_perm rows row0 + m0 + r, or with a row map the rows
  // rowmap[...] of the unsorted input (one pointer per DMA instruction)
  uint32_t wofs[4];
  const uint16_t *xsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    int wrow;
    if constexpr (GATEUP) wrow = tl.c0 + ((r >> 7) << 6) + (r & 63);
    else wrow = min(tl.c0 + r, N - 1);
    wofs[i] = uint32_t(wrow) * uint32_t(K) + c * 8;
    if (r > tl.ne - 1 - tl.m0 && K <= kZeroK) {
      xsrc[i] = g_zero_row + c * 8;
    } else {
      const int xr = tl.row0 + tl.m0 + min(r, tl.ne - 1 - tl.m0);
      xsrc[i] = X + size_t(rowmap ? rowmap[xr] : xr) * K + c * 8;
    }
  }
  const int dma_row = wave * 32;

  // ---- fragment read addresses (bytes): row (lane & 31) of a 32-row group,
  // logical chunk kk*2 + (lane >> 5)
  const int g = (lane >> 5) ^ swz(lane & 31);
  uint32_t offk[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) offk[kk] = uint32_t(((kk * 2) ^ g) * 16);
  const uint32_t baseA = uint32_t((wr * 128 + (lane & 31)) * 128);
  const uint32_t baseB = uint32_t((wc * 64 + (lane & 31)) * 128);

  f32x16 acc[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[f][t][i] = 0.f;

  const int nk = K / 64 / ksplit;  // k-blocks of this part (an even count)
  const int kb0 = tl.ks * nk;

#define DMAW(SW, KB)                                                                       \
  {                                                                                        \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                          \
      dma16(wmat + wofs[i] + k0, (lds_void *)(SW + (dma_row + i * 8) * 64));               \
  }
#define DMAX(SX, KB)                                                                       \
  {                                                                                        \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                          \
      dma16(xsrc[i] + k0, (lds_void *)(SX + (dma_row + i * 8) * 64));                      \
  }
  // both fragment sets double-buffered: the next kk's six reads are issued
  // ahead of the current kk's eight MFMAs
#define COMPUTE(SW, SX)                                                                    \
  {                                                                                        \
    const char *pa = reinterpret_cast<const char *>(SW) + baseA;                           \
    const char *pb = reinterpret_cast<const char *>(SX) + baseB;                           \
    bf16x8 fa[2][4], fb[2][2];                                                             \
    _Pragma("unroll") for (int f = 0; f < 4; ++f)                                          \
      fa[0][f] = *reinterpret_cast<const bf16x8 *>(pa + f * 4096 + offk[0]);               \
    _Pragma("unroll") for (int t = 0; t < 2; ++t)                                          \
      fb[0][t] = *reinterpret_cast<const bf16x8 *>(pb + t * 4096 + offk[0]);               \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                                     \
      const int cur = kk & 1;                                                              \
      if (kk + 1 < 4) {                                                                    \
        _Pragma("unroll") for (int f = 0; f < 4; ++f) fa[cur ^ 1][f] =                     \
            *reinterpret_cast<const bf16x8 *>(pa + f * 4096 + offk[kk + 1]);               \
        _Pragma("unroll") for (int t = 0; t < 2; ++t) fb[cur ^ 1][t] =                     \
            *reinterpret_cast<const bf16x8 *>(pb + t * 4096 + offk[kk + 1]);               \
      }                                                                                    \
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);                                   \
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);                                   \
      _Pragma("unroll") for (int t = 0; t < 2; ++t)                                        \
        _Pragma("unroll") for (int f = 0; f < 4; ++f)                                      \
          acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][f], fb[cur][t],      \
                                                              acc[f][t], 0, 0, 0);         \
      __builtin_amdgcn_sched_barrier(0);                                                   \
    }                                                                                      \
  }
  // k-block KB: weights in slot KB % 3, tokens in slot KB % 2; the copies
  // issued go to the slots the previous k-block has just released. Separate
  // LDS arrays per slot (not one indexed array) let the compiler see that the
  // copies in flight do not touch the slots being read.
#define STEP(KB, WS, XS, XN, WN)                                                           \
  DMAX(sX##XN, (KB) + 1)                                                                   \
  DMAW(sW##WN, (KB) + 2)                                                                   \
  COMPUTE(sW##WS, sX##XS)                                                                  \
  __builtin_amdgcn_s_waitcnt(kWaitVm4);                                                    \
  TILED_BARRIER()

  DMAW(sW0, 0)
  DMAX(sX0, 0)
  DMAW(sW1, 1)
  __builtin_amdgcn_s_waitcnt(kWaitVm4);
  TILED_BARRIER()
  int kt = 0;
  for (; kt + 6 <= nk; kt += 6) {  // unrolled by 6 so that every slot index is static
    STEP(kt + 0, 0, 0, 1, 2)
    STEP(kt + 1, 1, 1, 0, 0)
    STEP(kt + 2, 2, 0, 1, 1)
    STEP(kt + 3, 0, 1, 0, 2)
    STEP(kt + 4, 1, 0, 1, 0)
    STEP(kt + 5, 2, 1, 0, 1)
  }
  if (kt < nk) {  // nk is even: 2 or 4 k-blocks remain
    STEP(kt + 0, 0, 0, 1, 2)
    STEP(kt + 1, 1, 1, 0, 0)
    kt += 2;
  }
  if (kt < nk) {
    STEP(kt + 0, 2, 0, 1, 1)
    STEP(kt + 1, 0, 1, 0, 2)
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no copy in flight past the main loop
#undef STEP
#undef DMAW
#undef DMAX
#undef COMPUTE

  store_2x4<GATEUP, BT>(acc, tl, lane, wr, wc, N, part_stride, out);
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
template <bool GATEUP, int BT>
__device__ __forceinline__ void small_body(
    const uint16_t *__restrict__ X, const int32_t *__restrict__ offsets, int E,
    const uint16_t *__restrict__ Wa, const uint16_t *__restrict__ Wb, void *__restrict__ out,
    int N, int K, int ksplit, int64_t part_stride, const int32_t *__restrict__ rowmap,
    uint16_t *sW0, uint16_t *sW1, uint16_t *sW2, uint16_t *sX0, uint16_t *sX1) {
  constexpr int NT = BT / 64;  // 32-token accumulator columns per wavefront
  constexpr int XI = BT / 64;  // token-row DMA instructions per wavefront
  Tile tl;
  if (!find_tile<BT, GATEUP ? 128 : 256>(offsets, E, N, ksplit, tl)) return;
  const int e = tl.e, row0 = tl.row0, ne = tl.ne, m0 = tl.m0, c0 = tl.c0, ks = tl.ks;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  // ---- DMA assignment as in tiled_kernel: wave w fills weight rows
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
    const int chunk = ((lane & 7) ^ lr ^ q) << 3;
    if (dma_xrow + 8 * i + lr > xlim && K <= kZeroK) {
      xsrc[i] = g_zero_row + chunk;  // padding row
    } else {
      const int xr = row0 + m0 + min(dma_xrow + 8 * i + lr, xlim);
      xsrc[i] = X + size_t(rowmap ? rowmap[xr] : xr) * K + chunk;
    }
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

#define DMAW(SW, KB)                                                                       \
  {                                                                                        \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                          \
      dma16_nt(wmat + wofs[i] + k0, (lds_void *)(SW + (dma_row + i * 8) * 64));              \
  }
#define DMAX(SX, KB)                                                                       \
  {                                                                                        \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    _Pragma("unroll") for (int i = 0; i < XI; ++i)                                         \
      dma16(xsrc[i] + k0, (lds_void *)(SX + (dma_xrow + i * 8) * 64));                    \
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

  if constexpr (BT == 64) {
    DMAW(sW0, 0)
    DMAX(sX0, 0)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      DMAW(sW1, kt + 1)
      DMAX(sX1, kt + 1)
      COMPUTE(sW0, sX0)
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      DMAW(sW0, kt + 2)
      DMAX(sX0, kt + 2)
      COMPUTE(sW1, sX1)
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
    }
  } else {
    // as tiled256_kernel: tokens one k-block ahead, weights two
#define STEP(KB, WS, XS, XN, WN)                                                           \
  DMAX(sX##XN, (KB) + 1)                                                                   \
  DMAW(sW##WN, (KB) + 2)                                                                   \
  COMPUTE(sW##WS, sX##XS)                                                                  \
  __builtin_amdgcn_s_waitcnt(kWaitVm4);                                                    \
  TILED_BARRIER()
    DMAW(sW0, 0)
    DMAX(sX0, 0)
    DMAW(sW1, 1)
    __builtin_amdgcn_s_waitcnt(kWaitVm4);
    TILED_BARRIER()
    int kt = 0;
    for (; kt + 6 <= nk; kt += 6) {
      STEP(kt + 0, 0, 0, 1, 2)
      STEP(kt + 1, 1, 1, 0, 0)
      STEP(kt + 2, 2, 0, 1, 1)
      STEP(kt + 3, 0, 1, 0, 2)
      STEP(kt + 4, 1, 0, 1, 0)
      STEP(kt + 5, 2, 1, 0, 1)
    }
    if (kt < nk) {
      STEP(kt + 0, 0, 0, 1, 2)
      STEP(kt + 1, 1, 1, 0, 0)
      kt += 2;
    }
    if (kt < nk) {
      STEP(kt + 0, 2, 0, 1, 1)
      STEP(kt + 1, 0, 1, 0, 2)
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no copy in flight past the main loop
#undef STEP
  }
#undef DMAW
#undef DMAX
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

template <bool GATEUP>
__global__ __launch_bounds__(512) void tiled64_kernel(
    const uint16_t *__restrict__ X, const int32_t *__restrict__ offsets, int E,
    const uint16_t *__restrict__ Wa, const uint16_t *__restrict__ Wb, void *__restrict__ out,
    int N, int K, int ksplit, int64_t part_stride, const int32_t *__restrict__ rowmap) {
  __shared__ __attribute__((aligned(1024))) uint16_t sW0[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sW1[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX0[64 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX1[64 * 64];
  small_body<GATEUP, 64>(X, offsets, E, Wa, Wb, out, N, K, ksplit, part_stride, rowmap, sW0,
                         sW1, nullptr, sX0, sX1);
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
  small_body<GATEUP, 128>(X, offsets, E, Wa, Wb, out, N, K, ksplit, part_stride, rowmap, sW0,
                          sW1, sW2, sX0, sX1);
}

// Upper bound of the tile count for any split of S rows over E experts.
inline unsigned tiled_grid(int64_t S, int E, int N, int cols, int bt, int ksplit) {
  const int64_t ct = (N + cols - 1) / cols;
  const int64_t tiles = ksplit * ct * ((S + bt - 1) / bt + E);
  return unsigned((tiles + kXCD - 1) / kXCD * kXCD);
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
