// combine.hip -- weighted scatter back to token order.
//
// y[t] = sum_k w[t, k] * o_perm[slot_pos[t, k]] (crackai page, y = w_1 Expert_i1(x)
// + w_2 Expert_i2(x); notion page, output equation). Each token gathers its K
// expert rows, so no two threads write the same output and no atomics are
// needed; the K terms are added in k order with fused multiply-adds in float32
// and the sum is rounded once to the output type. When the down projection
// left `parts` partial sums per row (parts * S * d floats), a row is their sum
// in part order. With a residual (the block input of a pre-norm block), the
// weighted sum is added to it in float32 before the rounding.
#include "kernels.h"

namespace moe {
namespace {

template <bool OUT_BF16, int RES>  // RES: 0 none, 1 float32, 2 bf16 residual
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ o_perm, int parts,
                                                      const int32_t *__restrict__ slot_pos,
                                                      const float *__restrict__ w, int64_t T,
                                                      int64_t S, int K, int d, int chunks,
                                                      const void *__restrict__ residual,
                                                      void *__restrict__ y) {
  const int64_t t = int64_t(blockIdx.x) / chunks;
  const int col = (int(blockIdx.x % chunks) * 256 + threadIdx.x) * 4;
  if (t >= T || col >= d) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < K; ++k) {
    const int32_t p = slot_pos[t * K + k];
    if (p < 0 || p >= S) continue;
    const float wk = w[t * K + k];
    float4 o = *reinterpret_cast<const float4 *>(o_perm + int64_t(p) * d + col);
    for (int q = 1; q < parts; ++q) {
      const float4 oq =
          *reinterpret_cast<const float4 *>(o_perm + (q * S + int64_t(p)) * d + col);
      o.x += oq.x;
      o.y += oq.y;
      o.z += oq.z;
      o.w += oq.w;
    }
    acc.x = fmaf(wk, o.x, acc.x);
    acc.y = fmaf(wk, o.y, acc.y);
    acc.z = fmaf(wk, o.z, acc.z);
    acc.w = fmaf(wk, o.w, acc.w);
  }
  if constexpr (RES == 1) {
    const float4 r = *reinterpret_cast<const float4 *>(static_cast<const float *>(residual) + t * d + col);
    acc = make_float4(r.x + acc.x, r.y + acc.y, r.z + acc.z, r.w + acc.w);
  } else if constexpr (RES == 2) {
    const uint2 rb = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(residual) + t * d + col);
    acc = make_float4(bf16_bits_to_f32(rb.x & 0xFFFFu) + acc.x, bf16_bits_to_f32(rb.x >> 16) + acc.y,
                      bf16_bits_to_f32(rb.y & 0xFFFFu) + acc.z, bf16_bits_to_f32(rb.y >> 16) + acc.w);
  }
  if constexpr (OUT_BF16) {
    uint2 q;
    q.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
    q.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(y) + t * d + col) = q;
  } else {
    *reinterpret_cast<float4 *>(static_cast<float *>(y) + t * d + col) = acc;
  }
}

template <bool OUT_BF16, int RES>
void launch_c(dim3 grid, hipStream_t s, const float *o_perm, int parts, const int32_t *slot_pos,
              const float *w, int64_t T, int K, int d, int chunks, const void *residual, void *y) {
  hipLaunchKernelGGL((combine_kernel<OUT_BF16, RES>), grid, dim3(256), 0, s, o_perm, parts,
                     slot_pos, w, T, T * K, K, d, chunks, residual, y);
}

}  // namespace

hipError_t launch_combine(const float *o_perm, int parts, const int32_t *slot_pos, const float *w,
                          int64_t T, int K, int d, bool out_bf16, const void *residual,
                          bool in_bf16, void *y, hipStream_t s) {
  const int chunks = (d + 1023) / 1024;
  const dim3 grid(unsigned(T * chunks));
  const int res = residual == nullptr ? 0 : (in_bf16 ? 2 : 1);
#define C(OB, R) launch_c<OB, R>(grid, s, o_perm, parts, slot_pos, w, T, K, d, chunks, residual, y)
  if (out_bf16) {
    if (res == 0) C(true, 0);
    else if (res == 1) C(true, 1);
    else C(true, 2);
  } else {
    if (res == 0) C(false, 0);
    else if (res == 1) C(false, 1);
    else C(false, 2);
  }
#undef C
  return hipGetLastError();
}

}  // namespace moe
