// norm.hip -- RMSNorm of the block input, the normalisation in front of the
// MoE feed-forward layer in Mixtral's LLaMA-like blocks (ml-canon page
// "52 Mixtral", Connections: RMSNorm, RoPE, SwiGLU).
//
//   x[t, j] = h[t, j] * (1 / sqrt(mean_j' h[t, j']^2 + eps)) * g[j]
//
// One workgroup (4 wavefronts) per row. The mean square is accumulated in
// float32: each thread sums the squares of its 8-element chunks in chunk order,
// a butterfly finishes each wavefront and the 4 wavefront sums are added in the
// order 0+1+2+3, so every row is normalised the same way in every run. The
// second pass re-reads the row (L2-resident) and rounds x once to the layer's
// type. Memory-bound: T*d elements read twice (once from HBM) and written once.
#include "kernels.h"

namespace moe {
namespace {

template <bool BF16>
__device__ __forceinline__ void load8(const void *base, int64_t elem, float v[8]) {
  if constexpr (BF16) {
    const u32x4 q = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + elem);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + elem + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void store8(void *base, int64_t elem, const float v[8]) {
  if constexpr (BF16) {
    u32x4 q;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = f32_to_bf16_bits(v[2 * i]) | (f32_to_bf16_bits(v[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(base) + elem) = q;
  } else {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(base) + elem) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(static_cast<float *>(base) + elem + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void *__restrict__ h,
                                                      const void *__restrict__ g, float eps, int d,
                                                      void *__restrict__ x) {
  __shared__ float part[4];
  const int64_t row = int64_t(blockIdx.x) * d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunks = d >> 3;  // d is a multiple of 128
  float ss = 0.f;
  for (int c = threadIdx.x; c < chunks; c += 256) {
    float v[8];
    load8<BF16>(h, row + int64_t(c) * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  const float ms = (((part[0] + part[1]) + part[2]) + part[3]) / float(d);
  const float inv = 1.0f / sqrtf(ms + eps);
  for (int c = threadIdx.x; c < chunks; c += 256) {
    float v[8], gv[8];
    load8<BF16>(h, row + int64_t(c) * 8, v);
    load8<BF16>(g, int64_t(c) * 8, gv);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (v[i] * inv) * gv[i];
    store8<BF16>(x, row + int64_t(c) * 8, v);
  }
}

}  // namespace

hipError_t launch_rmsnorm(bool bf16, const void *h, const void *g, float eps, int64_t T, int d,
                          void *x, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(rmsnorm_kernel<true>, dim3(unsigned(T)), dim3(256), 0, s, h, g, eps, d, x);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<false>, dim3(unsigned(T)), dim3(256), 0, s, h, g, eps, d, x);
  return hipGetLastError();
}

}  // namespace moe
