// gemm_stream.hip -- expert projections for small batches: weight streaming.
//
// With few tokens per expert (decode), every routed expert's W1/W3/W2 must be
// read once from HBM while the arithmetic is negligible: the pages stress that
// all expert weights have to be resident although only 2 of 8 run per token
// (ml-canon page, "Questions worth asking"), and a 32-token batch reaches all 8
// experts. This kernel is built to keep HBM busy:
//
//  * Weights are the MFMA A operand (16 weight rows x 32 k), the expert's
//    tokens the B operand (32 k x 16 tokens), v_mfma_f32_16x16x32_bf16. A lane
//    loads its 8 bf16 of a weight row straight from global memory with one
//    16-byte load; no LDS staging, so all VGPR room goes to loads in flight.
//  * A workgroup (4 wavefronts) owns 16*NT output columns of one expert; its
//    4 wavefronts split K into quarters (intra-workgroup split-K) so that a
//    column block is 4 independent load streams, and the 4 partial sums are
//    added in LDS in the fixed order 0+1+2+3 (deterministic, no atomics).
//  * Up to kMT token tiles of 16 (2 or 4, by batch size) stay in accumulators;
//    an expert with no rows exits before reading any weight. An expert with
//    more than 16*kMT rows is handled 16*kMT rows at a time (the weights stream
//    once per group: correct for any count, fast up to 16*kMT).
//  * Gate-up carries W1 and W3 rows of the same output columns, so the SwiGLU
//    epilogue silu(g) * u happens in registers before the single rounding to
//    bf16 (notion page, "Implementation").
#include "kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ bf16x8 ld16(const uint16_t *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

template <int NMAT, int NT, int U, int kMT>
__device__ __forceinline__ void stream_rows(const uint16_t *__restrict__ X,
                                            const uint16_t *__restrict__ Wa,
                                            const uint16_t *__restrict__ Wb,
                                            void *__restrict__ out, int N, int K, int e, int row0,
                                            int ne) {
  const int mt = (ne + 15) >> 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int kq = K >> 2;  // multiple of 32
  const int kbeg = wave * kq + g * 8;
  const int n0 = blockIdx.x * (16 * NT);

  const uint16_t *wp[NMAT][NT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      wp[m][nt] = (m == 0 ? Wa : Wb) + (size_t(e) * N + n0 + nt * 16 + r16) * size_t(K) + kbeg;
  const uint16_t *xp[kMT];
  bool xv[kMT];
#pragma unroll
  for (int mi = 0; mi < kMT; ++mi) {
    const int r = mi * 16 + r16;
    xv[mi] = r < ne;
    xp[mi] = X + size_t(row0 + (xv[mi] ? r : 0)) * K + kbeg;
  }

  f32x4 acc[NMAT][NT][kMT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mi = 0; mi < kMT; ++mi) acc[m][nt][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bf16x8 zero = {};
  int ks = 0;
  for (; ks + 32 * U <= kq; ks += 32 * U) {
    bf16x8 b[U][NMAT][NT];
    bf16x8 a[U][kMT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) b[u][m][nt] = ld16(wp[m][nt] + ks + u * 32);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mi = 0; mi < kMT; ++mi)
        a[u][mi] = (mi < mt && xv[mi]) ? ld16(xp[mi] + ks + u * 32) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mi = 0; mi < kMT; ++mi) {
        if (mi >= mt) continue;
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[m][nt][mi] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[u][m][nt], a[u][mi], acc[m][nt][mi], 0, 0, 0);
      }
  }
  for (; ks < kq; ks += 32) {
    bf16x8 b[NMAT][NT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) b[m][nt] = ld16(wp[m][nt] + ks);
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi) {
      if (mi >= mt) continue;
      const bf16x8 a = xv[mi] ? ld16(xp[mi] + ks) : zero;
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[m][nt][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[m][nt], a, acc[m][nt][mi], 0, 0, 0);
    }
  }

  // Split-K reduction: wavefronts 1..3 park their partial sums in LDS,
  // wavefront 0 adds them in the order 1, 2, 3.
  __shared__ f32x4 red[3][NMAT * NT * kMT][64];
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mi = 0; mi < kMT; ++mi)
          if (mi < mt) red[wave - 1][(m * NT + nt) * kMT + mi][lane] = acc[m][nt][mi];
  }
  __syncthreads();
  if (wave != 0) return;  // the caller's barrier is reached by all wavefronts
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mi = 0; mi < kMT; ++mi)
          if (mi < mt) acc[m][nt][mi] += red[w][(m * NT + nt) * kMT + mi][lane];

  // D[i][j] of a 16x16 tile: lane holds token j = lane % 16 and weight rows
  // (output columns) i = 4 * (lane / 16) + 0..3.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi) {
      const int tok = mi * 16 + r16;
      if (mi >= mt || tok >= ne) continue;
      const int col = n0 + nt * 16 + 4 * g;
      const size_t o = size_t(row0 + tok) * N + col;
      if constexpr (NMAT == 2) {
        const f32x4 gv = acc[0][nt][mi], uv = acc[1][nt][mi];
        uint2 q;
        q.x = f32_to_bf16_bits(silu(gv[0]) * uv[0]) | (f32_to_bf16_bits(silu(gv[1]) * uv[1]) << 16);
        q.y = f32_to_bf16_bits(silu(gv[2]) * uv[2]) | (f32_to_bf16_bits(silu(gv[3]) * uv[3]) << 16);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + o) = q;
      } else {
        const f32x4 v = acc[0][nt][mi];
        *reinterpret_cast<float4 *>(static_cast<float *>(out) + o) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
}

template <int NMAT, int NT, int U, int kMT>
__global__ __launch_bounds__(256) void stream_kernel(const uint16_t *__restrict__ X,
                                                     const int32_t *__restrict__ offsets,
                                                     const uint16_t *__restrict__ Wa,
                                                     const uint16_t *__restrict__ Wb,
                                                     void *__restrict__ out, int N, int K) {
  const int e = blockIdx.y;
  const int seg0 = offsets[e];
  const int seg_rows = offsets[e + 1] - seg0;
  // Rows are taken 16*kMT at a time; more rows re-stream the weights
  // (correct for any count, efficient up to 16*kMT).
  for (int rg = 0; rg < seg_rows; rg += 16 * kMT) {
    stream_rows<NMAT, NT, U, kMT>(X, Wa, Wb, out, N, K, e, seg0 + rg, min(seg_rows - rg, 16 * kMT));
    __syncthreads();
  }
}


constexpr int kNTGateUp = 2, kUGateUp = 4;
constexpr int kNTDown = 2, kUDown = 4;

}  // namespace

// max_rows: an upper bound of the rows of any expert (T for a routed batch);
// it only selects how many token tiles the accumulators hold.
hipError_t launch_stream_gate_up(const void *x_perm, const int32_t *offsets, const void *w1,
                                 const void *w3, void *act, int E, int d, int h, int64_t max_rows,
                                 hipStream_t s) {
  const dim3 grid(unsigned(h / (16 * kNTGateUp)), unsigned(E));
  auto X = static_cast<const uint16_t *>(x_perm);
  auto A = static_cast<const uint16_t *>(w1);
  auto B = static_cast<const uint16_t *>(w3);
  if (max_rows <= 32)
    hipLaunchKernelGGL((stream_kernel<2, kNTGateUp, kUGateUp, 2>), grid, dim3(256), 0, s, X,
                       offsets, A, B, act, h, d);
  else
    hipLaunchKernelGGL((stream_kernel<2, kNTGateUp, kUGateUp, 4>), grid, dim3(256), 0, s, X,
                       offsets, A, B, act, h, d);
  return hipGetLastError();
}

hipError_t launch_stream_down(const void *act, const int32_t *offsets, const void *w2,
                              float *o_perm, int E, int d, int h, int64_t max_rows, hipStream_t s) {
  const dim3 grid(unsigned(d / (16 * kNTDown)), unsigned(E));
  auto X = static_cast<const uint16_t *>(act);
  auto A = static_cast<const uint16_t *>(w2);
  if (max_rows <= 32)
    hipLaunchKernelGGL((stream_kernel<1, kNTDown, kUDown, 2>), grid, dim3(256), 0, s, X, offsets,
                       A, static_cast<const uint16_t *>(nullptr), static_cast<void *>(o_perm), d, h);
  else
    hipLaunchKernelGGL((stream_kernel<1, kNTDown, kUDown, 4>), grid, dim3(256), 0, s, X, offsets,
                       A, static_cast<const uint16_t *>(nullptr), static_cast<void *>(o_perm), d, h);
  return hipGetLastError();
}

}  // namespace moe
