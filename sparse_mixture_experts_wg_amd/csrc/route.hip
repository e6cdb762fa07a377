// route.hip -- router: logits x . W_g, top-K (K <= 2) and the softmax over the
// kept logits, one pass over x.
//
// Mixtral of Experts, crackai page "Top-2 Routing in Detail" (gate_logits =
// x . W_gate of shape [tokens, 8]; keep the top 2 and renormalise with a
// softmax) and notion page, sparse-gating equation G(x) = Softmax(TopK(x . W_g)).
//
// Layout of the work: a workgroup is 4 wavefronts, each wavefront owns TPW
// tokens. W_g is staged through LDS in slabs of 1024 rows, transposed to
// [expert][row] float32 so that a lane's 8 consecutive rows of one expert are
// two conflict-free 16-byte LDS reads. Each lane walks 8-element chunks of the
// token rows (one 16-byte load per token for bf16), keeps TPW x 8 float32
// partial sums, and a butterfly over the 64 lanes finishes the dot products.
// Logits stay float32 up to the top-K decision.
#include "kernels.h"

namespace moe {
namespace {

constexpr int kSlab = 1024;  // W_g rows per LDS slab (32 KiB as float32)
constexpr int kTPW = 8;      // tokens per wavefront
constexpr int kWaves = 4;

template <bool BF16>
__device__ __forceinline__ void load8(const void *base, int64_t elem, float v[8]) {
  if constexpr (BF16) {
    const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + elem);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem);
    const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void *base, int64_t elem) {
  if constexpr (BF16) return __uint_as_float(uint32_t(static_cast<const uint16_t *>(base)[elem]) << 16);
  else return static_cast<const float *>(base)[elem];
}

template <bool BF16>
__global__ __launch_bounds__(256) void route_kernel(const void *__restrict__ x,
                                                    const void *__restrict__ wg, int64_t T, int d,
                                                    int E, int K, int32_t *__restrict__ idx,
                                                    float *__restrict__ w,
                                                    float *__restrict__ logits) {
  __shared__ float wt[8][kSlab];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t tok0 = (int64_t(blockIdx.x) * kWaves + wave) * kTPW;

  float acc[kTPW][8];
#pragma unroll
  for (int t = 0; t < kTPW; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;

  for (int j0 = 0; j0 < d; j0 += kSlab) {
    const int rows = min(kSlab, d - j0);  // multiple of 128
    __syncthreads();
    for (int i = threadIdx.x; i < rows * 8; i += 256) {
      const int r = i >> 3, e = i & 7;
      wt[e][r] = e < E ? load1<BF16>(wg, int64_t(j0 + r) * E + e) : 0.f;
    }
    __syncthreads();
    for (int c = lane; c < (rows >> 3); c += 64) {
      float wv[8][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 a = *reinterpret_cast<const float4 *>(&wt[e][c * 8]);
        const float4 b = *reinterpret_cast<const float4 *>(&wt[e][c * 8 + 4]);
        wv[e][0] = a.x; wv[e][1] = a.y; wv[e][2] = a.z; wv[e][3] = a.w;
        wv[e][4] = b.x; wv[e][5] = b.y; wv[e][6] = b.z; wv[e][7] = b.w;
      }
#pragma unroll
      for (int t = 0; t < kTPW; ++t) {
        if (tok0 + t < T) {
          float xv[8];
          load8<BF16>(x, (tok0 + t) * d + j0 + c * 8, xv);
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[t][e] = fmaf(xv[i], wv[e][i], acc[t][e]);
        }
      }
    }
  }

  // Butterfly: every lane ends with the full sums.
#pragma unroll
  for (int t = 0; t < kTPW; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[t][e];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      acc[t][e] = v;
    }

#pragma unroll
  for (int t = 0; t < kTPW; ++t) {
    const int64_t tok = tok0 + t;
    if (lane != t || tok >= T) continue;
    const float *l = acc[t];
    // top-1 / top-2 by (logit desc, index asc); values tracked beside indices so
    // that no register array is indexed at run time
    int b0 = 0;
    float v0 = l[0];
#pragma unroll
    for (int e = 1; e < 8; ++e)
      if (e < E && l[e] > v0) { v0 = l[e]; b0 = e; }
    if (K == 1) {
      idx[tok] = b0;
      w[tok] = 1.0f;
    } else {
      int b1 = -1;
      float v1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < E && e != b0 && (b1 < 0 || l[e] > v1)) { v1 = l[e]; b1 = e; }
      // softmax over the two kept logits, v1 <= v0
      const float r = expf(v1 - v0);
      const float w0 = 1.0f / (1.0f + r);
      idx[tok * 2] = b0;
      idx[tok * 2 + 1] = b1;
      w[tok * 2] = w0;
      w[tok * 2 + 1] = r * w0;
    }
    if (logits) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < E) logits[tok * E + e] = l[e];
    }
  }
}

}  // namespace

hipError_t launch_route(bool bf16, const void *x, const void *wg, int64_t T, int d, int E, int K,
                        int32_t *idx, float *w, float *logits, hipStream_t s) {
  const int64_t per_block = int64_t(kWaves) * kTPW;
  const dim3 grid(unsigned((T + per_block - 1) / per_block));
  if (bf16)
    hipLaunchKernelGGL(route_kernel<true>, grid, dim3(256), 0, s, x, wg, T, d, E, K, idx, w, logits);
  else
    hipLaunchKernelGGL(route_kernel<false>, grid, dim3(256), 0, s, x, wg, T, d, E, K, idx, w, logits);
  return hipGetLastError();
}

}  // namespace moe
