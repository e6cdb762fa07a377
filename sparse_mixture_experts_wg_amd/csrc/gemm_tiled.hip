// gemm_tiled.hip -- expert projections for large batches: grouped bf16 GEMM on
// the CDNA4 matrix cores.
//
// Each expert's rows form one contiguous segment of the sorted activations, so
// the layer is a grouped GEMM C_e = X_e W_e^T with both operands K-contiguous
// (Mixtral of Experts, notion page "Implementation": SwiGLU experts with K = 2;
// the sparse-matmul kernels the pages cite are prior art, this is a plain
// grouped GEMM over the per-expert segments).
//
// Tile: 256 weight rows (MFMA M side) x BT tokens (MFMA N side) x 64 k.
//  * 4 wavefronts in a 2 x 2 grid; each owns 128 weight rows x BT/2 tokens as
//    4 x (BT/64) accumulators of v_mfma_f32_32x32x16_bf16 (16 fp32 each).
//  * Global -> VGPR -> LDS, two LDS stages (the next k-block's global loads are
//    in flight while the current one is multiplied), one barrier per k-block.
//    LDS rows are padded to 144 bytes so the 16-byte fragment reads of 8
//    consecutive rows hit distinct banks.
//  * Gate-up: the 256 weight rows are W1 and W3 rows of the same 128 output
//    columns, interleaved in blocks of 64 so that every wavefront holds g and u
//    of the same columns and applies silu(g) * u in registers; the result is
//    rounded once to bf16. Down: 256 W2 rows = 256 output columns, float32 out.
//  * Tiles are ordered (expert, column block, token block) with the token block
//    fastest, so concurrently running tiles share weight tiles; the linear tile
//    id is remapped so that each of the 8 XCDs (workgroups are dealt to XCDs
//    round-robin) owns one contiguous range of tiles and its own L2 sees the
//    reuse. Token blocks past an expert's last row skip their MFMAs.
#include "kernels.h"

namespace moe {
namespace {

constexpr int kBW = 256;        // weight rows per tile
constexpr int kBK = 64;         // k per stage
constexpr int kStride = 72;     // LDS row stride in bf16 (64 + 8 padding)
constexpr int kXCD = 8;

template <bool GATEUP>
__device__ __forceinline__ int weight_row(int r, int c0, int N, const uint16_t *Wa,
                                          const uint16_t *Wb, const uint16_t *&mat) {
  if constexpr (GATEUP) {
    // [0,64) W1 c0+[0,64) | [64,128) W3 c0+[0,64) | [128,192) W1 c0+64+[0,64) | [192,256) W3
    const int blk = r >> 6;
    mat = (blk & 1) ? Wb : Wa;
    return min(c0 + ((blk >> 1) << 6) + (r & 63), N - 1);
  } else {
    mat = Wa;
    return min(c0 + r, N - 1);
  }
}

template <bool GATEUP, int BT>
__global__ __launch_bounds__(256) void tiled_kernel(const uint16_t *__restrict__ X,
                                                    const int32_t *__restrict__ offsets, int E,
                                                    const uint16_t *__restrict__ Wa,
                                                    const uint16_t *__restrict__ Wb,
                                                    void *__restrict__ out, int N, int K) {
  constexpr int kCols = GATEUP ? kBW / 2 : kBW;  // output columns per tile
  constexpr int kTF = BT / 64;                   // token fragments (32 wide) per wavefront
  const int ct = (N + kCols - 1) / kCols;        // column blocks per expert

  // ---- which tile: total over experts, XCD-aware remap --------------------
  int total = 0;
  for (int q = 0; q < E; ++q) total += ct * ((offsets[q + 1] - offsets[q] + BT - 1) / BT);
  const int g8 = (total + kXCD - 1) / kXCD;
  const int b = blockIdx.x;
  if (b >= g8 * kXCD) return;
  int L = (b % kXCD) * g8 + b / kXCD;
  if (L >= total) return;
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

  __shared__ __attribute__((aligned(16))) uint16_t sW[2][kBW * kStride];
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][BT * kStride];

  // ---- global load assignment: thread owns 16-byte chunk (tid & 7) of rows
  //      (tid >> 3) + 32 j of both tiles. Addresses are 32-bit element offsets
  //      from wave-uniform bases (the expert's matrices, the tile's first row).
  const int kc = (tid & 7) * 8;
  const int rbase = tid >> 3;
  constexpr int kWL = kBW / 32;  // weight rows per thread
  constexpr int kXL = BT / 32;   // token rows per thread
  const size_t mat_elems = size_t(N) * K;
  const uint16_t *wa_e = Wa + size_t(e) * mat_elems;
  const uint16_t *wb_e = GATEUP ? Wb + size_t(e) * mat_elems : wa_e;
  const uint16_t *x_t = X + size_t(row0 + m0) * K;
  uint32_t woff[kWL], xoff[kXL];
#pragma unroll
  for (int j = 0; j < kWL; ++j) {
    const uint16_t *mat;
    const int row = weight_row<GATEUP>(rbase + 32 * j, c0, N, Wa, Wb, mat);
    woff[j] = uint32_t(row) * uint32_t(K) + kc;
  }
#pragma unroll
  for (int j = 0; j < kXL; ++j)
    xoff[j] = uint32_t(min(rbase + 32 * j, ne - 1 - m0)) * uint32_t(K) + kc;

  f32x16 acc[4][kTF];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < kTF; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[f][t][i] = 0.f;

  // fragment read offsets: lane reads row (lane & 31), k half (lane >> 5)
  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  const uint16_t *aW = &sW[0][(wr * 128 + frow) * kStride + fk];
  const uint16_t *aX = &sX[0][(wc * (BT / 2) + frow) * kStride + fk];
  uint16_t *dW = &sW[0][rbase * kStride + kc];
  uint16_t *dX = &sX[0][rbase * kStride + kc];

  // Software pipeline: k-block kt+2 is fetched into registers while k-block kt
  // is multiplied from LDS stage kt & 1 and k-block kt+1 (fetched one iteration
  // earlier) is written into the other stage; one barrier per k-block. Blocks
  // past the end are clamped re-reads of the last one, written to a stage that
  // is never read again. All 4 x kTF fragments are multiplied in every k-block
  // (no data-dependent branch touches the accumulators, so they stay in AGPRs);
  // token rows past the expert's end are clamped duplicates whose results are
  // never stored. K is a multiple of 128, so the k-block count is even.
  u32x4 r0w[kWL], r0x[kXL], r1w[kWL], r1x[kXL];
  const int nk = K / kBK;
#define MOE_GLOAD(RW, RX, KB)                                                                 \
  {                                                                                           \
    const uint32_t k0 = uint32_t(min(KB, nk - 1) * kBK);                                      \
    _Pragma("unroll") for (int j = 0; j < kWL; ++j) {                                         \
      const uint16_t *base = (GATEUP && ((j >> 1) & 1)) ? wb_e : wa_e;                        \
      RW[j] = *reinterpret_cast<const u32x4 *>(base + woff[j] + k0);                          \
    }                                                                                         \
    _Pragma("unroll") for (int j = 0; j < kXL; ++j)                                           \
      RX[j] = *reinterpret_cast<const u32x4 *>(x_t + xoff[j] + k0);                           \
  }
#define MOE_SSTORE(RW, RX, ST)                                                                \
  {                                                                                           \
    _Pragma("unroll") for (int j = 0; j < kWL; ++j)                                           \
      *reinterpret_cast<u32x4 *>(dW + (ST) * (kBW * kStride) + 32 * j * kStride) = RW[j];     \
    _Pragma("unroll") for (int j = 0; j < kXL; ++j)                                           \
      *reinterpret_cast<u32x4 *>(dX + (ST) * (BT * kStride) + 32 * j * kStride) = RX[j];      \
  }
// One k-block from LDS stage ST, in fenced blocks so that the order below is
// the order issued: (global loads for block kt+2, fragments of k-step 0),
// then per k-step: fragments of the next k-step, half of the LDS writes of
// block kt+1 (last two k-steps), and the 4 x kTF MFMAs of this k-step. A
// fragment read thus has a whole k-step of MFMAs to land, and the LDS writes
// come one iteration after their global loads were issued.
#define MOE_MMA_STAGE(ST, GLOAD_STMT, RW, RX, WST)                                            \
  {                                                                                           \
    const uint16_t *pw = aW + (ST) * (kBW * kStride);                                         \
    const uint16_t *px = aX + (ST) * (BT * kStride);                                          \
    bf16x8 fa[2][4], fb[2][kTF];                                                              \
    GLOAD_STMT                                                                                \
    _Pragma("unroll") for (int f = 0; f < 4; ++f)                                             \
      fa[0][f] = *reinterpret_cast<const bf16x8 *>(pw + f * 32 * kStride);                    \
    _Pragma("unroll") for (int t = 0; t < kTF; ++t)                                           \
      fb[0][t] = *reinterpret_cast<const bf16x8 *>(px + t * 32 * kStride);                    \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    _Pragma("unroll") for (int kk = 0; kk < kBK / 16; ++kk) {                                 \
      const int cur = kk & 1;                                                                 \
      if (kk + 1 < kBK / 16) {                                                                \
        _Pragma("unroll") for (int f = 0; f < 4; ++f) fa[cur ^ 1][f] =                        \
            *reinterpret_cast<const bf16x8 *>(pw + f * 32 * kStride + (kk + 1) * 16);         \
        _Pragma("unroll") for (int t = 0; t < kTF; ++t) fb[cur ^ 1][t] =                      \
            *reinterpret_cast<const bf16x8 *>(px + t * 32 * kStride + (kk + 1) * 16);         \
      }                                                                                       \
      if (kk == kBK / 16 - 2) {                                                               \
        _Pragma("unroll") for (int j = 0; j < kWL; ++j)                                       \
          *reinterpret_cast<u32x4 *>(dW + (WST) * (kBW * kStride) + 32 * j * kStride) = RW[j]; \
      }                                                                                       \
      if (kk == kBK / 16 - 1) {                                                               \
        _Pragma("unroll") for (int j = 0; j < kXL; ++j)                                       \
          *reinterpret_cast<u32x4 *>(dX + (WST) * (BT * kStride) + 32 * j * kStride) = RX[j]; \
      }                                                                                       \
      __builtin_amdgcn_sched_group_barrier(0x180, 64, 1);                                     \
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * kTF, 1);                                \
      _Pragma("unroll") for (int t = 0; t < kTF; ++t)                                         \
        _Pragma("unroll") for (int f = 0; f < 4; ++f)                                         \
          acc[f][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][f], fb[cur][t],         \
                                                              acc[f][t], 0, 0, 0);            \
      __builtin_amdgcn_sched_barrier(0);                                                      \
    }                                                                                         \
  }

  MOE_GLOAD(r0w, r0x, 0)
  MOE_GLOAD(r1w, r1x, 1)
  MOE_SSTORE(r0w, r0x, 0)
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    MOE_MMA_STAGE(0, MOE_GLOAD(r0w, r0x, kt + 2), r1w, r1x, 1)
    __syncthreads();
    MOE_MMA_STAGE(1, MOE_GLOAD(r1w, r1x, kt + 3), r0w, r0x, 0)
    __syncthreads();
  }
#undef MOE_GLOAD
#undef MOE_SSTORE
#undef MOE_MMA_STAGE

  // ---- epilogue. 32x32 accumulator: lane holds token column j = lane & 31 and
  // weight rows i = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4), r = 0..15.
  const int ih = 4 * (lane >> 5);
#pragma unroll
  for (int t = 0; t < kTF; ++t) {
    const int tok = m0 + wc * (BT / 2) + t * 32 + (lane & 31);
    if (tok >= ne) continue;
    const size_t orow = size_t(row0 + tok) * N;
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

constexpr int kBTGateUp = 256;
constexpr int kBTDown = 256;

// Upper bound of the tile count for any split of S rows over E experts.
inline unsigned tiled_grid(int64_t S, int E, int N, int cols, int BT) {
  const int64_t ct = (N + cols - 1) / cols;
  const int64_t tiles = ct * ((S + BT - 1) / BT + E);
  return unsigned((tiles + kXCD - 1) / kXCD * kXCD);
}

}  // namespace

hipError_t launch_tiled_gate_up(const void *x_perm, const int32_t *offsets, const void *w1,
                                const void *w3, void *act, int E, int64_t S, int d, int h,
                                hipStream_t s) {
  hipLaunchKernelGGL((tiled_kernel<true, kBTGateUp>), dim3(tiled_grid(S, E, h, kBW / 2, kBTGateUp)),
                     dim3(256), 0, s, static_cast<const uint16_t *>(x_perm), offsets, E,
                     static_cast<const uint16_t *>(w1), static_cast<const uint16_t *>(w3), act, h, d);
  return hipGetLastError();
}

hipError_t launch_tiled_down(const void *act, const int32_t *offsets, const void *w2,
                             float *o_perm, int E, int64_t S, int d, int h, hipStream_t s) {
  hipLaunchKernelGGL((tiled_kernel<false, kBTDown>), dim3(tiled_grid(S, E, d, kBW, kBTDown)),
                     dim3(256), 0, s, static_cast<const uint16_t *>(act), offsets, E,
                     static_cast<const uint16_t *>(w2), static_cast<const uint16_t *>(nullptr),
                     static_cast<void *>(o_perm), d, h);
  return hipGetLastError();
}

}  // namespace moe
