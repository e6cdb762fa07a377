// gemm_tiled.hip -- expert projections for large batches: grouped bf16 GEMM on
// the CDNA4 matrix cores.
//
// Each expert's rows form one contiguous segment of the sorted activations, so
// the layer is a grouped GEMM C_e = X_e W_e^T with both operands K-contiguous
// (Mixtral of Experts, notion page "Implementation": SwiGLU experts with K = 2;
// the sparse-matmul kernels the pages cite are prior art, this is a plain
// grouped GEMM over the per-expert segments).
//
// Tile: 256 weight rows (MFMA M side) x 256 tokens (MFMA N side) x 64 k.
//  * 8 wavefronts (2 per SIMD) in a 2 x 4 grid; each owns 128 weight rows x 64
//    tokens as 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16. Two wavefronts
//    per SIMD keep the matrix pipe fed while the other waits on LDS or a barrier
//    (one wavefront per SIMD tops out near 80% of the matrix peak on gfx950).
//  * Global memory goes straight to LDS (global_load_lds_dwordx4: a wavefront
//    instruction fills one contiguous kilobyte, lane L the bytes [16L, 16L+16)),
//    two stages of 64 KiB; the k-block after the current one is in flight while
//    the current one is multiplied; one barrier per k-block.
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
//  * Down with few row tiles can split the sum over h in two: each half is a
//    tile of its own writing float32 partial sums that the combine step adds
//    in a fixed order, so that the last round of tiles fills the GPU.
#include "kernels.h"

namespace moe {
namespace {

constexpr int kXCD = 8;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate with vmcnt(0) and the other counters at their maximum.
constexpr int kWaitVm0 = 0x0F70;

// Physical 16-byte chunk = logical chunk ^ swz(row); depends on row & 31 only.
__device__ __forceinline__ int swz(int r) { return ((r & 31) ^ ((r & 31) >> 3)) & 7; }

template <bool GATEUP>
__global__ __launch_bounds__(512) void tiled_kernel(const uint16_t *__restrict__ X,
                                                     const int32_t *__restrict__ offsets, int E,
                                                     const uint16_t *__restrict__ Wa,
                                                     const uint16_t *__restrict__ Wb,
                                                     void *__restrict__ out, int N, int K,
                                                     int ksplit, int64_t part_stride) {
  constexpr int BT = 256;
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
  const int wave = tid >> 6;
  const int wr = wave >> 2, wc = wave & 3;

  __shared__ __attribute__((aligned(1024))) uint16_t sW0[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sW1[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX0[256 * 64];
  __shared__ __attribute__((aligned(1024))) uint16_t sX1[256 * 64];

  // ---- DMA assignment: wave w fills rows [32w, 32w+32) of both tiles, 8 rows per
  // instruction; lane p writes LDS bytes [16p, 16p+16) of the instruction's
  // kilobyte: row 8i + p/8, physical chunk p%8 = logical chunk ^ swz(row).
  const size_t mat_elems = size_t(N) * K;
  const uint16_t *wmat = Wa + size_t(e) * mat_elems;
  if (GATEUP && ((wave >> 1) & 1)) wmat = Wb + size_t(e) * mat_elems;
  const uint16_t *x_t = X + size_t(row0 + m0) * K;
  uint32_t wofs[4], xofs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    int wrow;
    if constexpr (GATEUP) wrow = c0 + ((r >> 7) << 6) + (r & 63);
    else wrow = min(c0 + r, N - 1);
    wofs[i] = uint32_t(wrow) * uint32_t(K) + c * 8;
    xofs[i] = uint32_t(min(r, ne - 1 - m0)) * uint32_t(K) + c * 8;
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
  const int kb0 = ks * nk;

#define DMA(SW, SX, KB)                                                                    \
  {                                                                                        \
    const uint32_t k0 = uint32_t((kb0 + min(KB, nk - 1)) * 64);                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                        \
      __builtin_amdgcn_global_load_lds(wmat + wofs[i] + k0,                                \
                                       (lds_void *)(SW + (dma_row + i * 8) * 64), 16, 0, 0); \
      __builtin_amdgcn_global_load_lds(x_t + xofs[i] + k0,                                 \
                                       (lds_void *)(SX + (dma_row + i * 8) * 64), 16, 0, 0); \
    }                                                                                      \
  }
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
  for (int t = 0; t < 2; ++t) {
    const int tok = m0 + wc * 64 + t * 32 + (lane & 31);
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

// Upper bound of the tile count for any split of S rows over E experts.
inline unsigned tiled_grid(int64_t S, int E, int N, int cols, int ksplit) {
  const int64_t ct = (N + cols - 1) / cols;
  const int64_t tiles = ksplit * ct * ((S + 255) / 256 + E);
  return unsigned((tiles + kXCD - 1) / kXCD * kXCD);
}

}  // namespace

hipError_t launch_tiled_gate_up(const void *x_perm, const int32_t *offsets, const void *w1,
                                 const void *w3, void *act, int E, int64_t S, int d, int h,
                                 hipStream_t s) {
  hipLaunchKernelGGL((tiled_kernel<true>), dim3(tiled_grid(S, E, h, 128, 1)), dim3(512), 0, s,
                     static_cast<const uint16_t *>(x_perm), offsets, E,
                     static_cast<const uint16_t *>(w1), static_cast<const uint16_t *>(w3), act, h, d,
                     1, int64_t(0));
  return hipGetLastError();
}

hipError_t launch_tiled_down(const void *act, const int32_t *offsets, const void *w2,
                              float *o_perm, int E, int64_t S, int d, int h, int parts,
                              hipStream_t s) {
  hipLaunchKernelGGL((tiled_kernel<false>), dim3(tiled_grid(S, E, d, 256, parts)), dim3(512), 0, s,
                     static_cast<const uint16_t *>(act), offsets, E,
                     static_cast<const uint16_t *>(w2), static_cast<const uint16_t *>(nullptr),
                     static_cast<void *>(o_perm), d, h, parts, S * d);
  return hipGetLastError();
}

}  // namespace moe
