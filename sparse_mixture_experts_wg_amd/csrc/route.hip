// route.hip -- router: logits x . W_g, top-K (K <= 2) and the softmax over the
// kept logits, one pass over x.
//
// Mixtral of Experts, crackai page "Top-2 Routing in Detail" (gate_logits =
// x . W_gate of shape [tokens, 8]; keep the top 2 and renormalise with a
// softmax) and notion page, sparse-gating equation G(x) = Softmax(TopK(x . W_g)).
//
// Layout of the work: a workgroup owns TPB tokens (1, 2 or 4 by batch size: a
// small batch gets more workgroups, measured faster on MI355X) and its 4
// wavefronts split the dot products into quarters of d, so that even a 1-token
// batch keeps 4 wavefronts of loads in flight. A lane walks chunks of 8 consecutive rows j:
// one 16-byte load of x per token (bf16) and the chunk's 8 rows of W_g (8 x 16
// bytes for bf16 with E = 8; W_g is 64 KiB for d = 4096 and stays in L2),
// reused by the TPB tokens; two chunks' loads are in flight before their FMAs.
// Partial sums (TPB tokens x 8 experts in float32) are finished by a butterfly
// over the 64 lanes and a fixed-order sum of the 4 quarters in LDS. Logits stay
// float32 up to the top-K decision.
#include "kernels.h"

namespace moe {
namespace {

constexpr int kWaves = 4;  // wavefronts per workgroup, each a quarter of d

// 8 consecutive elements as float.
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

// Row j of W_g as 8 floats (experts >= E read as 0).
template <bool BF16, bool E8>
__device__ __forceinline__ void load_wrow(const void *wg, int64_t j, int E, float v[8]) {
  if constexpr (E8) {
    load8<BF16>(wg, j * 8, v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e < E) {
        if constexpr (BF16)
          v[e] = __uint_as_float(uint32_t(static_cast<const uint16_t *>(wg)[j * E + e]) << 16);
        else
          v[e] = static_cast<const float *>(wg)[j * E + e];
      } else {
        v[e] = 0.f;
      }
    }
  }
}

template <bool BF16, bool E8, int kTPB>
__global__ __launch_bounds__(256) void route_kernel(const void *__restrict__ x,
                                                    const void *__restrict__ wg, int64_t T, int d,
                                                    int E, int K, int32_t *__restrict__ idx,
                                                    float *__restrict__ w,
                                                    float *__restrict__ logits) {
  __shared__ float part[kWaves][64];
  __shared__ float total[64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t tok0 = int64_t(blockIdx.x) * kTPB;
  const int ntok = int(min(int64_t(kTPB), T - tok0));

  float acc[kTPB][8];
#pragma unroll
  for (int t = 0; t < kTPB; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;

  const int quarter = d >> 5;  // chunks of 8 rows per wavefront (d multiple of 128)
  const int cbeg = wave * quarter, cend = cbeg + quarter;
#pragma unroll 2
  for (int c = cbeg + lane; c < cend; c += 64) {
    float wv[8][8];  // [row in chunk][expert]
#pragma unroll
    for (int r = 0; r < 8; ++r) load_wrow<BF16, E8>(wg, int64_t(c) * 8 + r, E, wv[r]);
#pragma unroll
    for (int t = 0; t < kTPB; ++t) {
      if (t >= ntok) continue;
      float xv[8];
      load8<BF16>(x, (tok0 + t) * d + int64_t(c) * 8, xv);
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[t][e] = fmaf(xv[r], wv[r][e], acc[t][e]);
    }
  }

  // Butterfly within the wavefront, then lane t*8+e keeps sum (t, e).
  float mine = 0.f;
#pragma unroll
  for (int t = 0; t < kTPB; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[t][e];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      if (lane == t * 8 + e) mine = v;
    }
  part[wave][lane] = mine;
  __syncthreads();
  if (wave == 0) total[lane] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
  __syncthreads();
  const int t = threadIdx.x;
  if (t >= ntok) return;
  const int64_t tok = tok0 + t;
  float l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) l[e] = total[t * 8 + e];
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

template <bool BF16, bool E8>
void launch(hipStream_t s, const void *x, const void *wg, int64_t T, int d, int E, int K,
            int32_t *idx, float *w, float *logits) {
  // tokens per workgroup by batch size (a sweep of T = 1 .. 16384 on MI355X)
  if (T <= 256)
    hipLaunchKernelGGL((route_kernel<BF16, E8, 1>), dim3(unsigned(T)), dim3(256), 0, s, x, wg, T,
                       d, E, K, idx, w, logits);
  else if (T <= 1024)
    hipLaunchKernelGGL((route_kernel<BF16, E8, 2>), dim3(unsigned((T + 1) / 2)), dim3(256), 0, s,
                       x, wg, T, d, E, K, idx, w, logits);
  else
    hipLaunchKernelGGL((route_kernel<BF16, E8, 4>), dim3(unsigned((T + 3) / 4)), dim3(256), 0, s,
                       x, wg, T, d, E, K, idx, w, logits);
}

}  // namespace

hipError_t launch_route(bool bf16, const void *x, const void *wg, int64_t T, int d, int E, int K,
                        int32_t *idx, float *w, float *logits, hipStream_t s) {
  const bool e8 = (E == 8);
  if (bf16 && e8) launch<true, true>(s, x, wg, T, d, E, K, idx, w, logits);
  else if (bf16) launch<true, false>(s, x, wg, T, d, E, K, idx, w, logits);
  else if (e8) launch<false, true>(s, x, wg, T, d, E, K, idx, w, logits);
  else launch<false, false>(s, x, wg, T, d, E, K, idx, w, logits);
  return hipGetLastError();
}

}  // namespace moe
