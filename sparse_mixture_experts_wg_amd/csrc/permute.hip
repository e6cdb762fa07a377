// permute.hip -- gather each expert's token-slots into one contiguous segment.
//
// Tokens spread unevenly over the experts and have to be gathered per expert
// before the expert matrices run and scattered back afterwards (ml-canon page,
// "Questions worth asking"; notion page, the expert-parallel paragraph: each
// expert's output is returned to the token's original place).
//
// permute_index: ONE workgroup of 1024 threads does a stable counting sort of
// the S = T*K slots by expert id. Thread i owns the contiguous slot range
// [i*c, (i+1)*c); it counts its slots per expert, a wavefront scan plus a scan
// over the 16 wavefront totals gives every thread its first row per expert,
// and a second pass over the same range assigns rows in slot order. The result
// is the stable order (ascending s = t*K + k within an expert) with no atomics.
// The slot index arrays are small (S int32), so one CU suffices. From 2048 up
// to 32768 slots the expert ids are first copied into LDS with coalesced 16-byte loads
// and the slot positions are collected there and written back coalesced (each
// thread's contiguous slot range would otherwise make every wavefront access
// touch 64 separate lines); up to 16384 slots the sorted-row -> token map is
// assembled in LDS too, above that a second kernel over the whole GPU scatters it
// from the slot positions (scatter_perm).
// With a capacity C (the capacity variant) a slot whose rank within its expert
// is C or more is dropped (slot_pos -1, no row) and the offsets count the kept
// rows min(n_e, C) only.
//
// permute_index_small: up to 64 slots (a decode batch) one wavefront does the
// same sort: lane s holds slot s, a ballot per expert gives the expert's count
// and the slot's rank among the lanes below it, so no barrier and no LDS are
// needed; the results are those of permute_index.
//
// gather_rows: one wavefront per sorted row copies x[perm_token[r]] with 16-byte
// loads/stores.
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesPerBlock = kThreads / 64;
constexpr int kStage = 32768;  // slots staged in LDS (128 KiB)
// Thread i owns the contiguous slots [i*c, (i+1)*c), so the lanes of a wavefront read
// slots c apart: LDS holds slot s at pad(s) = s + s / 32, which puts the slots of a
// wavefront's 64 lanes on distinct banks for any c <= 32 (one int of padding per 32).
__device__ __forceinline__ int64_t pad(int64_t s) { return s + (s >> 5); }
constexpr int kStagePadded = kStage + kStage / 32;
constexpr int kPermOff = kStage / 2 + kStage / 64;  // sorted-row map after the slots

__global__ __launch_bounds__(kThreads) void permute_index_kernel(
    const int32_t *__restrict__ idx, int64_t S, int K, int E, int capacity,
    int32_t *__restrict__ offsets,
    int32_t *__restrict__ perm_token, int32_t *__restrict__ slot_pos) {
  __shared__ int32_t wave_tot[kWavesPerBlock][8];
  __shared__ int32_t wave_pre[kWavesPerBlock][8];
  __shared__ int32_t expert_off[9];
  // expert ids, then slot positions (S <= kStage, at pad(s)); with S <= kStage / 2
  // the sorted-row -> token map follows at kPermOff
  __shared__ int32_t sidx[kStagePadded];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t chunk = (S + kThreads - 1) / kThreads;
  const int64_t s0 = min(S, int64_t(tid) * chunk);
  const int64_t s1 = min(S, s0 + chunk);
  // (small batches skip the staging: a few slots per thread gain nothing from it)
  const bool staged = S >= 2048 && S <= kStage;
  const bool staged_perm = staged && S <= kStage / 2;
  int32_t *sperm = sidx + kPermOff;
  if (staged) {
    for (int64_t i = tid; i < S; i += kThreads) sidx[pad(i)] = idx[i];
    __syncthreads();
  }

  int cnt[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cnt[e] = 0;
  for (int64_t s = s0; s < s1; ++s) {
    const int e = staged ? sidx[pad(s)] : idx[s];
#pragma unroll
    for (int q = 0; q < 8; ++q) cnt[q] += (q == e && q < E) ? 1 : 0;
  }

  // inclusive scan of cnt over the lanes of the wavefront
  int incl[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int v = cnt[e];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(v, off, 64);
      if (lane >= off) v += u;
    }
    incl[e] = v;
  }
  if (lane == 63) {
#pragma unroll
    for (int e = 0; e < 8; ++e) wave_tot[wave][e] = incl[e];
  }
  __syncthreads();
  if (tid < 8) {
    int run = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) {
      wave_pre[w][tid] = run;
      run += wave_tot[w][tid];
    }
    wave_tot[0][tid] = run;  // expert total (wave_tot[0] is no longer needed)
  }
  __syncthreads();
  const int cap = capacity > 0 ? capacity : 0x7FFFFFFF;
  if (tid == 0) {
    int run = 0;
    expert_off[0] = 0;
    for (int e = 0; e < 8; ++e) {
      run += (e < E) ? min(wave_tot[0][e], cap) : 0;
      expert_off[e + 1] = run;
    }
    for (int e = 0; e <= E; ++e) offsets[e] = expert_off[e];
  }
  __syncthreads();

  // rank of this thread's first slot of each expert among that expert's slots
  int rank[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) rank[e] = wave_pre[wave][e] + incl[e] - cnt[e];
  for (int64_t s = s0; s < s1; ++s) {
    const int e = staged ? sidx[pad(s)] : idx[s];
    int p = -1;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q == e && q < E) {
        if (rank[q] < cap) p = expert_off[q] + rank[q];
        rank[q] += 1;
      }
    }
    if (staged)
      sidx[pad(s)] = p;  // this thread's own slot: no other thread reads it
    else
      slot_pos[s] = p;
    // rows -> tokens: in LDS from 2048 to kStage / 2 slots, straight to memory below,
    // above left to scatter_perm_kernel, which spreads the scatter over the GPU
    if (p >= 0) {
      if (staged_perm)
        sperm[p] = int32_t(s / K);
      else if (S <= kStage / 2)
        perm_token[p] = int32_t(s / K);
    }
  }
  if (staged) {
    __syncthreads();
    for (int64_t i = tid; i < S; i += kThreads) slot_pos[i] = sidx[pad(i)];
    if (staged_perm) {
      // rows [0, offsets[E]) exist; the rest of perm_token is left as it was
      const int64_t R = expert_off[E];
      const int64_t R4 = R & ~int64_t(3);
      for (int64_t i = int64_t(tid) * 4; i < R4; i += 4 * kThreads)
        *reinterpret_cast<int4 *>(perm_token + i) = *reinterpret_cast<const int4 *>(sperm + i);
      for (int64_t i = R4 + tid; i < R; i += kThreads) perm_token[i] = sperm[i];
    }
  }
}

constexpr int kSmallSlots = 64;

__global__ __launch_bounds__(64) void permute_index_small_kernel(
    const int32_t *__restrict__ idx, int S, int K, int E, int capacity,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm_token,
    int32_t *__restrict__ slot_pos) {
  const int lane = threadIdx.x;
  const int e = lane < S ? idx[lane] : -1;
  const int cap = capacity > 0 ? capacity : 0x7FFFFFFF;
  const uint64_t below = (uint64_t(1) << lane) - 1;  // lanes 0 .. lane-1
  int run = 0, my_off = 0, my_rank = 0;
  for (int q = 0; q < E; ++q) {  // E <= 8, the same in every lane
    const uint64_t m = __ballot(e == q);
    if (lane == q) offsets[q] = run;
    if (e == q) {
      my_off = run;
      my_rank = __popcll(m & below);
    }
    run += min(int(__popcll(m)), cap);
  }
  if (lane == 0) offsets[E] = run;
  if (lane >= S) return;
  const int p = (e >= 0 && e < E && my_rank < cap) ? my_off + my_rank : -1;
  slot_pos[lane] = p;
  if (p >= 0) perm_token[p] = lane / K;
}

// perm_token[slot_pos[s]] = s / K over the whole grid, for batches whose
// sorted-row -> token map does not fit the sort's LDS (every row is written once).
__global__ __launch_bounds__(256) void scatter_perm_kernel(const int32_t *__restrict__ slot_pos,
                                                           int64_t S, int K,
                                                           int32_t *__restrict__ perm_token) {
  const int64_t s = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (s >= S) return;
  const int p = slot_pos[s];
  if (p >= 0) perm_token[p] = int32_t(s / K);
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4 *__restrict__ x,
                                                          const int32_t *__restrict__ perm_token,
                                                          const int32_t *__restrict__ offsets,
                                                          int E, int64_t S, int64_t row_vecs,
                                                          uint4 *__restrict__ x_perm) {
  const int64_t r = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= S || r >= offsets[E]) return;
  const int64_t t = perm_token[r];
  const uint4 *src = x + t * row_vecs;
  uint4 *dst = x_perm + r * row_vecs;
  for (int64_t i = lane; i < row_vecs; i += 64) dst[i] = src[i];
}

}  // namespace

hipError_t launch_permute_index(const int32_t *idx, int64_t S, int K, int E, int capacity,
                                int32_t *offsets, int32_t *perm_token, int32_t *slot_pos,
                                hipStream_t s) {
  if (S <= kSmallSlots)
    hipLaunchKernelGGL(permute_index_small_kernel, dim3(1), dim3(64), 0, s, idx, int(S), K, E,
                       capacity, offsets, perm_token, slot_pos);
  else {
    hipLaunchKernelGGL(permute_index_kernel, dim3(1), dim3(kThreads), 0, s, idx, S, K, E,
                       capacity, offsets, perm_token, slot_pos);
    if (S > kStage / 2)
      hipLaunchKernelGGL(scatter_perm_kernel, dim3(unsigned((S + 255) / 256)), dim3(256), 0, s,
                         slot_pos, S, K, perm_token);
  }
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void *x, const int32_t *perm_token, const int32_t *offsets,
                              int E, int64_t S, int64_t row_bytes, void *x_perm, hipStream_t s) {
  const dim3 grid(unsigned((S + 3) / 4));
  hipLaunchKernelGGL(gather_rows_kernel, grid, dim3(256), 0, s, static_cast<const uint4 *>(x),
                     perm_token, offsets, E, S, row_bytes / 16, static_cast<uint4 *>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
