// route.hip -- router: logits x . W_g, top-K (K <= 2) and the softmax over the
// kept logits, one pass over x.
//
// Mixtral of Experts, crackai page "Top-2 Routing in Detail" (gate_logits =
// x . W_gate of shape [tokens, 8]; keep the top 2 and renormalise with a
// softmax) and notion page, sparse-gating equation G(x) = Softmax(TopK(x . W_g)).
//
// Layout of the work: a workgroup owns TPB tokens (1 up to 1024 tokens, else 2;
// bf16 batches of 8 experts from 2048 tokens on take route_wide_kernel below) and its 4
// wavefronts split the dot products into quarters of d, so that even a 1-token
// batch keeps 4 wavefronts of loads in flight. Within its quarter a wavefront
// takes 512 rows j at a time, lane L the rows j0 + 64 r + L (r = 0..7): each
// load instruction of W_g then reads one contiguous kilobyte (64 rows of
// 8 x bf16) and each load of x 128 contiguous bytes, the fewest cache lines per
// instruction (8 consecutive rows per lane would touch 64 lines per W_g
// instruction). W_g (64 KiB for d = 4096) stays in L2 and each row is reused by
// the TPB tokens. Partial sums (TPB tokens x 8 experts in float32) are finished
// by a butterfly over the 64 lanes and a fixed-order sum of the 4 quarters in
// LDS. Logits stay float32 up to the top-K decision.
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

// One element as float.
template <bool BF16>
__device__ __forceinline__ float load1(const void *base, int64_t elem) {
  if constexpr (BF16)
    return __uint_as_float(uint32_t(static_cast<const uint16_t *>(base)[elem]) << 16);
  else
    return static_cast<const float *>(base)[elem];
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

// Top-K of one token's logits l[e] = total[t * 8 + e]: by (logit desc, index
// asc), values tracked beside indices so that no register array is indexed at
// run time; then the softmax over the kept logits.
__device__ __forceinline__ void topk_out(const float *total, int t, int64_t tok, int E, int K,
                                         int32_t *__restrict__ idx, float *__restrict__ w,
                                         float *__restrict__ logits) {
  float l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) l[e] = total[t * 8 + e];
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

  // rows [rbeg, rend) of this wavefront (d a multiple of 128); rows past the
  // end of a 512-row block load row rend - 1 and count as x = 0
  const int rbeg = wave * (d >> 2), rend = rbeg + (d >> 2);
  for (int j0 = rbeg; j0 < rend; j0 += 512) {
    float wv[8][8];  // [r][expert]
    int jr[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      jr[r] = min(j0 + 64 * r + lane, rend - 1);
      load_wrow<BF16, E8>(wg, jr[r], E, wv[r]);
    }
#pragma unroll
    for (int t = 0; t < kTPB; ++t) {
      if (t >= ntok) continue;
      float xv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float v = load1<BF16>(x, (tok0 + t) * d + jr[r]);
        xv[r] = (j0 + 64 * r + lane < rend) ? v : 0.f;
      }
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
  topk_out(total, t, tok0 + t, E, K, idx, w, logits);
}

// Large batches, bf16 and 8 experts: route_kernel re-reads all of W_g (16 bytes
// per row of d) from L2 for every 1-2 tokens and loads x 2 bytes per lane, so at
// thousands of tokens it moves about five times the bytes of x through L2 and
// issues one load instruction per 128 bytes of x. Here a workgroup takes
// kWideTPB = 8 tokens and a lane 8 consecutive rows j .. j + 7 of its quarter of d:
// one 16-byte load per token and 512-row block brings x[t][j .. j + 7], and the
// 8 x 8 weights of those rows (8 loads of one W_g row each) serve all 8 tokens.
// The 64 partial sums per lane (8 tokens x 8 experts) are reduced over the
// wavefront by halving exchanges (at the exchange with lane ^ m a lane keeps the
// half of its values selected by bit m of its index and adds its partner's copy
// of that half; after m = 32 .. 1 lane L holds sum L = token L / 8, expert L % 8),
// then over the 4 quarters in LDS in the order 0+1+2+3.
constexpr int kWideTPB = 8;

__global__ __launch_bounds__(256) void route_wide_kernel(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ wg,
                                                        int64_t T, int d, int K,
                                                        int32_t *__restrict__ idx,
                                                        float *__restrict__ w,
                                                        float *__restrict__ logits) {
  __shared__ float part[kWaves][64];
  __shared__ float total[64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t tok0 = int64_t(blockIdx.x) * kWideTPB;
  const int ntok = int(min(int64_t(kWideTPB), T - tok0));

  float v[64];  // [token * 8 + expert]
#pragma unroll
  for (int i = 0; i < 64; ++i) v[i] = 0.f;

  // d / 4 is a multiple of 32, so a lane's 8 rows are all inside the quarter or
  // all outside it. The full 512-row blocks run as a uniform loop that issues the
  // next block's loads before the current block's arithmetic (two register
  // buffers); the lanes of a last, partial block run after it under a lane mask.
  // (With the lane test inside one loop the compiler ran the loop under an exec
  // mask and waited for every load at the top of each block.) The sums are those of
  // one block at a time, in the same order.
  const int rbeg = wave * (d >> 2), rend = rbeg + (d >> 2);
  const int nfull = (rend - rbeg) >> 9;
  u32x4 xq[2][kWideTPB], wq[2][8];
  auto load_block = [&](int j, u32x4 *xb, u32x4 *wb) {
#pragma unroll
    for (int t = 0; t < kWideTPB; ++t)  // a missing token re-reads the last one
      xb[t] = *reinterpret_cast<const u32x4 *>(x + (tok0 + min(t, ntok - 1)) * d + j);
#pragma unroll
    for (int r = 0; r < 8; ++r)
      wb[r] = *reinterpret_cast<const u32x4 *>(wg + int64_t(j + r) * 8);
  };
  // row by row (each accumulator still adds rows r = 0..7 in order), so that only one
  // row of weights is unpacked at a time
  auto mac_block = [&](const u32x4 *xb, const u32x4 *wb) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float wv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wv[2 * i] = __uint_as_float(wb[r][i] << 16);
        wv[2 * i + 1] = __uint_as_float(wb[r][i] & 0xFFFF0000u);
      }
#pragma unroll
      for (int t = 0; t < kWideTPB; ++t) {
        if (t >= ntok) continue;
        const uint32_t q = xb[t][r >> 1];
        const float xv = __uint_as_float((r & 1) ? (q & 0xFFFF0000u) : (q << 16));
#pragma unroll
        for (int e = 0; e < 8; ++e) v[t * 8 + e] = fmaf(xv, wv[e], v[t * 8 + e]);
      }
    }
  };
  if (nfull > 0) load_block(rbeg + 8 * lane, xq[0], wq[0]);
  int b = 0;
  for (; b + 2 <= nfull; b += 2) {
    load_block(rbeg + 512 * (b + 1) + 8 * lane, xq[1], wq[1]);  // (b + 1 < nfull)
    mac_block(xq[0], wq[0]);
    if (b + 2 < nfull) load_block(rbeg + 512 * (b + 2) + 8 * lane, xq[0], wq[0]);
    mac_block(xq[1], wq[1]);
  }
  if (b < nfull) mac_block(xq[0], wq[0]);  // odd count: the last full block
  {
    const int j = rbeg + 512 * nfull + 8 * lane;  // partial block, if any
    if (j < rend) {
      load_block(j, xq[1], wq[1]);
      mac_block(xq[1], wq[1]);
    }
  }

#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const bool hi = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < m; ++i) {
      const float send = hi ? v[i] : v[i + m];
      const float keep = hi ? v[i + m] : v[i];
      v[i] = keep + __shfl_xor(send, m, 64);
    }
  }
  part[wave][lane] = v[0];
  __syncthreads();
  if (wave == 0) total[lane] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
  __syncthreads();
  const int t = threadIdx.x;
  if (t >= ntok) return;
  topk_out(total, t, tok0 + t, 8, K, idx, w, logits);
}

// The pre-norm block's RMSNorm fused in front of the router: x = RMSNorm(h) * g
// is computed, written (the expert path reads it) and routed in one pass. The
// mean square of each token follows norm.hip's order exactly (thread i sums the
// squares of chunks i, i + 256, ... in order, a butterfly per wavefront, the 4
// wavefront sums added 0+1+2+3), and the logits follow route_kernel's order on
// the rounded x, so x, the logits and the routing are bitwise those of the two
// separate kernels.
template <bool BF16, bool E8, int kTPB>
__global__ __launch_bounds__(256) void norm_route_kernel(
    const void *__restrict__ h, const void *__restrict__ g, float eps,
    const void *__restrict__ wg, int64_t T, int d, int E, int K, void *__restrict__ x,
    int32_t *__restrict__ idx, float *__restrict__ w, float *__restrict__ logits) {
  __shared__ float part[kWaves][64];
  __shared__ float total[64];
  __shared__ float ssp[kTPB][kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t tok0 = int64_t(blockIdx.x) * kTPB;
  const int ntok = int(min(int64_t(kTPB), T - tok0));
  const int chunks = d >> 3;

  // The first 512-row block's weights, gains and inputs do not depend on the
  // norm: their loads go out before the mean square is formed, so that the two
  // passes over h do not wait for memory one after the other.
  const int rbeg = wave * (d >> 2), rend = rbeg + (d >> 2);
  float wv[8][8], gv[8], hv[kTPB][8];
  int jr[8];
#define NR_LOAD_BLOCK(J0)                                                                  \
  {                                                                                        \
    _Pragma("unroll") for (int r = 0; r < 8; ++r) {                                        \
      jr[r] = min((J0) + 64 * r + lane, rend - 1);                                         \
      load_wrow<BF16, E8>(wg, jr[r], E, wv[r]);                                            \
      gv[r] = load1<BF16>(g, jr[r]);                                                       \
    }                                                                                      \
    _Pragma("unroll") for (int t = 0; t < kTPB; ++t)                                       \
      _Pragma("unroll") for (int r = 0; r < 8; ++r)                                        \
        hv[t][r] = load1<BF16>(h, (tok0 + min(t, ntok - 1)) * d + jr[r]);                  \
  }
  NR_LOAD_BLOCK(rbeg)

  // mean square per token, in norm.hip's order
#pragma unroll
  for (int t = 0; t < kTPB; ++t) {
    if (t >= ntok) continue;
    float ss = 0.f;
    for (int c = threadIdx.x; c < chunks; c += 256) {
      float v[8];
      load8<BF16>(h, (tok0 + t) * d + int64_t(c) * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if (lane == 0) ssp[t][wave] = ss;
  }
  __syncthreads();
  float inv[kTPB];
#pragma unroll
  for (int t = 0; t < kTPB; ++t) {
    if (t >= ntok) {  // no token: its sums were never written
      inv[t] = 0.f;
      continue;
    }
    const float ms = (((ssp[t][0] + ssp[t][1]) + ssp[t][2]) + ssp[t][3]) / float(d);
    inv[t] = 1.0f / sqrtf(ms + eps);
  }

  float acc[kTPB][8];
#pragma unroll
  for (int t = 0; t < kTPB; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;

  for (int j0 = rbeg; j0 < rend; j0 += 512) {
    if (j0 != rbeg) NR_LOAD_BLOCK(j0)
#pragma unroll
    for (int t = 0; t < kTPB; ++t) {
      if (t >= ntok) continue;
      float xv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int64_t el = (tok0 + t) * d + jr[r];
        float v = (hv[t][r] * inv[t]) * gv[r];
        if constexpr (BF16) {  // x as stored: rounded once to bf16
          const uint32_t b = f32_to_bf16_bits(v);
          if (j0 + 64 * r + lane < rend) static_cast<uint16_t *>(x)[el] = uint16_t(b);
          v = bf16_bits_to_f32(b);
        } else {
          if (j0 + 64 * r + lane < rend) static_cast<float *>(x)[el] = v;
        }
        xv[r] = (j0 + 64 * r + lane < rend) ? v : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[t][e] = fmaf(xv[r], wv[r][e], acc[t][e]);
    }
  }
#undef NR_LOAD_BLOCK

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
  topk_out(total, t, tok0 + t, E, K, idx, w, logits);
}

// From this many tokens on, bf16 batches with 8 experts take route_wide_kernel
// (MI355X, d = 4096 and 6144, x resident in the last-level cache: equal at 2048
// tokens, 15.4 -> 11.2 us at 4096 and 49.6 -> 40.6 us at 16384 for d = 4096; below
// 2048 tokens its fewer workgroups lose, 8.3 against 6.5 us at 1024). Variants
// measured no better: the next 512-row block's loads issued before the current
// block's arithmetic, and 4 or 2 tokens per workgroup.
constexpr int64_t kWideMinT = 2048;

template <bool BF16, bool E8>
void launch(hipStream_t s, const void *x, const void *wg, int64_t T, int d, int E, int K,
            int32_t *idx, float *w, float *logits) {
  if (BF16 && E8 && T >= kWideMinT)
    hipLaunchKernelGGL(route_wide_kernel, dim3(unsigned((T + kWideTPB - 1) / kWideTPB)),
                       dim3(256), 0, s, static_cast<const uint16_t *>(x),
                       static_cast<const uint16_t *>(wg), T, d, K, idx, w, logits);
  else if (T <= 1024)
    hipLaunchKernelGGL((route_kernel<BF16, E8, 1>), dim3(unsigned(T)), dim3(256), 0, s, x, wg, T,
                       d, E, K, idx, w, logits);
  else
    hipLaunchKernelGGL((route_kernel<BF16, E8, 2>), dim3(unsigned((T + 1) / 2)), dim3(256), 0, s,
                       x, wg, T, d, E, K, idx, w, logits);
}

template <bool BF16, bool E8>
hipError_t launch_nr(hipStream_t s, const void *h, const void *g, float eps, const void *wg,
                     int64_t T, int d, int E, int K, void *x, int32_t *idx, float *w) {
  // tokens per workgroup as the router alone; where the router alone runs
  // route_wide_kernel, the norm and that router run as two launches (bitwise the
  // staged moe_rmsnorm + moe_route)
  if (BF16 && E8 && T >= kWideMinT) {
    const hipError_t e = launch_rmsnorm(true, h, g, eps, T, d, x, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_wide_kernel, dim3(unsigned((T + kWideTPB - 1) / kWideTPB)),
                       dim3(256), 0, s, static_cast<const uint16_t *>(x),
                       static_cast<const uint16_t *>(wg), T, d, K, idx, w, nullptr);
  } else if (T <= 1024) {
    hipLaunchKernelGGL((norm_route_kernel<BF16, E8, 1>), dim3(unsigned(T)), dim3(256), 0, s, h, g,
                       eps, wg, T, d, E, K, x, idx, w, nullptr);
  } else {
    hipLaunchKernelGGL((norm_route_kernel<BF16, E8, 2>), dim3(unsigned((T + 1) / 2)), dim3(256),
                       0, s, h, g, eps, wg, T, d, E, K, x, idx, w, nullptr);
  }
  return hipGetLastError();
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

hipError_t launch_norm_route(bool bf16, const void *h, const void *g, float eps, const void *wg,
                             int64_t T, int d, int E, int K, void *x, int32_t *idx, float *w,
                             hipStream_t s) {
  const bool e8 = (E == 8);
  if (bf16 && e8) return launch_nr<true, true>(s, h, g, eps, wg, T, d, E, K, x, idx, w);
  if (bf16) return launch_nr<true, false>(s, h, g, eps, wg, T, d, E, K, x, idx, w);
  if (e8) return launch_nr<false, true>(s, h, g, eps, wg, T, d, E, K, x, idx, w);
  return launch_nr<false, false>(s, h, g, eps, wg, T, d, E, K, x, idx, w);
}

}  // namespace moe
