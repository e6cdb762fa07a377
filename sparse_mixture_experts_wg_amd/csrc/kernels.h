// kernels.h -- internal launchers of the gfx950 kernels behind moe.h.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bf16 bits, round to nearest even (finite input).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> two bf16 in one 32-bit word (first in the low half), round to
// nearest even: the hardware conversion, the same bits as f32_to_bf16_bits for
// finite input.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// SiLU z * sigmoid(z) = z / (1 + e^-z), from the hardware base-2 exponential and
// reciprocal (each within about one ulp of float32): e^-z = 2^(-z log2 e). Large
// negative z give 2^+inf = inf and z * 0; large positive z give z * 1. The
// gate-up rounds silu(g) * u to bf16 afterwards (2^-8 relative), so the few ulps
// of float32 this differs from a correctly rounded quotient change about 6 of 10^6
// bf16 outputs, by one ulp (prefill_8x7b gate-up on MI355X). Against expf and an
// IEEE division the gate-up epilogue of the 256-token tiles shrinks from about 2100
// to 580 instructions per wavefront, and the launch from 1.58 to 1.53 ms.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504088896341f));
}

// ---- pre-norm ----------------------------------------------------------------
// x = RMSNorm(h) * g per row of d (a multiple of 128), rounded once to the type.
hipError_t launch_rmsnorm(bool bf16, const void *h, const void *g, float eps, int64_t T, int d,
                          void *x, hipStream_t s);

// ---- router -----------------------------------------------------------------
hipError_t launch_route(bool bf16, const void *x, const void *wg, int64_t T, int d, int E, int K,
                        int32_t *idx, float *w, float *logits, hipStream_t s);

// RMSNorm of the block input fused in front of the router: writes x (as
// launch_rmsnorm) and routes it (as launch_route, no logits); bitwise the same
// as the two launches.
hipError_t launch_norm_route(bool bf16, const void *h, const void *g, float eps, const void *wg,
                             int64_t T, int d, int E, int K, void *x, int32_t *idx, float *w,
                             hipStream_t s);

// ---- permute ----------------------------------------------------------------
// capacity > 0: each expert keeps its `capacity` earliest slots, later ones get
// slot_pos -1 and no row.
hipError_t launch_permute_index(const int32_t *idx, int64_t S, int K, int E, int capacity,
                                int32_t *offsets,
                                int32_t *perm_token, int32_t *slot_pos, hipStream_t s);
hipError_t launch_gather_rows(const void *x, const int32_t *perm_token, const int32_t *offsets,
                              int E, int64_t S, int64_t row_bytes, void *x_perm, hipStream_t s);

// ---- expert projections -------------------------------------------------------
// STREAM path (bf16 weight streaming; an expert's rows are taken in groups of 32
// or 64, each group streaming its weights). rows_hint: usual largest segment
// (T); rows_bound: no segment is longer (S); the grid's z extent is
// rows_bound / 32 or / 64, which the caller keeps below 2^16.
// rowmap (nullable): sorted row r of the gate-up input is row rowmap[r] of x_perm
// (the layer passes the unsorted input x and perm_token, skipping the gather).
hipError_t launch_stream_gate_up(const void *x_perm, const int32_t *rowmap,
                                 const int32_t *offsets, const void *w1, const void *w3,
                                 void *act, int E, int d, int h, int64_t rows_hint,
                                 int64_t rows_bound, hipStream_t s);
hipError_t launch_stream_down(const void *act, const int32_t *offsets, const void *w2,
                              float *o_perm, int E, int d, int h, int64_t rows_hint,
                              int64_t rows_bound, hipStream_t s);
// TILED path (bf16 matrix cores); bt: token tile, 64, 128 or 256; rowmap as
// for the streaming gate-up.
hipError_t launch_tiled_gate_up(const void *x_perm, const int32_t *rowmap, const int32_t *offsets,
                                const void *w1, const void *w3, void *act, int E, int64_t S,
                                int d, int h, int bt, hipStream_t s);
// parts (1, 2 or 4; needs h % (128 * parts) == 0): partial sums over h, part q
// at o_perm + q * S * d. Equal ranges of h, except that with 2 parts part 0 may take
// more of it (chosen on the device from the tile count, so that the last round of
// workgroups is full).
hipError_t launch_tiled_down(const void *act, const int32_t *offsets, const void *w2,
                             float *o_perm, int E, int64_t S, int d, int h, int bt, int parts,
                             hipStream_t s);
// float32 problems.
hipError_t launch_f32_gate_up(const float *x_perm, const int32_t *offsets, const float *w1,
                              const float *w3, float *act, int E, int64_t S, int d, int h,
                              hipStream_t s);
hipError_t launch_f32_down(const float *act, const int32_t *offsets, const float *w2,
                           float *o_perm, int E, int64_t S, int d, int h, hipStream_t s);

// ---- combine ----------------------------------------------------------------
// residual (nullable, [T, d] in the input type, bf16 if in_bf16): y = residual + the
// weighted sum, added in float32 before the single rounding.
hipError_t launch_combine(const float *o_perm, int parts, const int32_t *slot_pos, const float *w,
                          int64_t T, int K, int d, bool out_bf16, const void *residual,
                          bool in_bf16, void *y, hipStream_t s);

}  // namespace moe
