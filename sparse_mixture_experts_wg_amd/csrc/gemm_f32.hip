// gemm_f32.hip -- expert projections for float32 problems (plain FMA tiles).
//
// Same grouped structure as the bf16 paths: the rows of expert e are
// x_perm[offsets[e] .. offsets[e+1]-1]; a workgroup computes a 64-row x
// 64-column tile of one expert, C[m, n] = sum_k A[m, k] * W[n, k], with both
// operands K-contiguous. The gate-up instance carries W1 and W3 together and
// applies the SwiGLU epilogue silu(g) * u in registers (notion page,
// "Implementation": SwiGLU experts). Accumulation is float32 FMA in ascending
// k order per output.
#include "kernels.h"

namespace moe {
namespace {

constexpr int kTile = 64;
constexpr int kBK = 16;

template <bool GATEUP>
__global__ __launch_bounds__(256) void f32_kernel(const float *__restrict__ X,
                                                  const int32_t *__restrict__ offsets, int E,
                                                  const float *__restrict__ Wa,
                                                  const float *__restrict__ Wb,
                                                  float *__restrict__ out, int N, int K) {
  // blockIdx.x: m-tile counted over all experts in order; blockIdx.y: n-tile
  int e = -1, m0 = 0, row0 = 0, ne = 0, seen = 0;
  for (int q = 0; q < E; ++q) {
    const int n = offsets[q + 1] - offsets[q];
    const int tq = (n + kTile - 1) / kTile;
    if (int(blockIdx.x) < seen + tq) {
      e = q;
      m0 = (int(blockIdx.x) - seen) * kTile;
      row0 = offsets[q];
      ne = n;
      break;
    }
    seen += tq;
  }
  if (e < 0) return;
  const int n0 = blockIdx.y * kTile;
  __shared__ float As[kBK][kTile + 1];
  __shared__ float Bs[kBK][kTile + 1];
  __shared__ float Cs[kBK][kTile + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4], acc2[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = acc2[i][j] = 0.f;

  const size_t wbase = size_t(e) * N;
  for (int k0 = 0; k0 < K; k0 += kBK) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      const int r = i >> 4, kk = i & 15;
      const int m = m0 + r;
      As[kk][r] = (m < ne) ? X[size_t(row0 + m) * K + k0 + kk] : 0.f;
      Bs[kk][r] = Wa[(wbase + n0 + r) * K + k0 + kk];
      if constexpr (GATEUP) Cs[kk][r] = Wb[(wbase + n0 + r) * K + k0 + kk];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; ++kk) {
      float a[4], b[4], c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[kk][tx * 4 + i];
        if constexpr (GATEUP) c[i] = Cs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if constexpr (GATEUP) acc2[i][j] = fmaf(a[i], c[j], acc2[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= ne) continue;
    float4 v;
    float *pv = reinterpret_cast<float *>(&v);
#pragma unroll
    for (int j = 0; j < 4; ++j) pv[j] = GATEUP ? silu(acc[i][j]) * acc2[i][j] : acc[i][j];
    *reinterpret_cast<float4 *>(out + size_t(row0 + m) * N + n0 + tx * 4) = v;
  }
}

inline dim3 f32_grid(int64_t S, int E, int N) {
  return dim3(unsigned((S + kTile - 1) / kTile + E), unsigned(N / kTile));
}

}  // namespace

hipError_t launch_f32_gate_up(const float *x_perm, const int32_t *offsets, const float *w1,
                              const float *w3, float *act, int E, int64_t S, int d, int h,
                              hipStream_t s) {
  hipLaunchKernelGGL(f32_kernel<true>, f32_grid(S, E, h), dim3(256), 0, s, x_perm, offsets, E, w1,
                     w3, act, h, d);
  return hipGetLastError();
}

hipError_t launch_f32_down(const float *act, const int32_t *offsets, const float *w2,
                           float *o_perm, int E, int64_t S, int d, int h, hipStream_t s) {
  hipLaunchKernelGGL(f32_kernel<false>, f32_grid(S, E, d), dim3(256), 0, s, act, offsets, E, w2,
                     nullptr, o_perm, d, h);
  return hipGetLastError();
}

}  // namespace moe
