// permute.hip -- gather each expert's token-slots into one contiguous segment.
//
// Tokens spread unevenly over the experts and have to be gathered per expert
// before the expert matrices run and scattered back afterwards (ml-canon page,
// "Questions worth asking"; notion page, the expert-parallel paragraph: each
// expert's output is returned to the token's original place).
//
// permute_index: ONE workgroup of 1024 threads does a stable counting sort of
// the S = T*K slots by expert id (used from 65 to kGridMinS - 1 slots). Thread i
// owns the contiguous slot range [i*c, (i+1)*c); it counts its slots per expert,
// a wavefront scan plus a scan over the 16 wavefront totals gives every thread its
// first row per expert, and a second pass over the same range assigns rows in slot
// order. The result is the stable order (ascending s = t*K + k within an expert)
// with no atomics. From 2048 slots on the expert ids are first copied into LDS and
// the slot positions and the sorted-row -> token map are collected there and
// written back coalesced (each thread's contiguous slot range would otherwise make
// every wavefront access touch 64 separate lines).
//
// permute_grid: from kGridMinS slots on, the same sort over a grid of workgroups
// (below).
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
    // rows -> tokens: in LDS from 2048 slots on, straight to memory below (the
    // kernel runs on fewer than kGridMinS <= kStage / 2 slots)
    if (p >= 0) {
      if (staged_perm)
        sperm[p] = int32_t(s / K);
      else
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

// Sum of v over the 64 lanes of the wavefront, in every lane, by DPP moves (no
// LDS): pairs and quads (quad_perm), the two quads of each half row and the two
// halves of each row (mirrors), row 0 into row 1 and row 2 into row 3
// (row_bcast15), rows 0-1 into rows 2-3 (row_bcast31); lane 63 then holds the
// total, which readlane hands to every lane.
__device__ __forceinline__ int wave_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast31
  return __builtin_amdgcn_readlane(v, 63);
}

// Large batches: the same stable sort spread over a grid of workgroups. Workgroup
// b owns the slots [b C, b C + C). Each workgroup first counts, per expert, all
// S slot ids (those before its range and the rest; S * 4 bytes from L2 per
// workgroup, with C chosen so that there are at most kGridMaxBlocks workgroups),
// which gives the expert offsets and the rank of its first slot of each expert
// among that expert's slots. Its own range then goes by in rounds of
// kGridThreads consecutive slots, one per thread: a ballot per expert gives a
// slot's rank among the lanes below it, the wavefront counts of the round are
// prefixed over the 8 wavefronts in LDS, and a running count per expert carries
// the ranks from one round to the next. Every slot is ranked once, without
// atomics, and the results are those of permute_index_kernel.
constexpr int kGridThreads = 512;
constexpr int kGridWaves = kGridThreads / 64;
constexpr int kGridMaxBlocks = 64;
// From this many slots on the grid kernel replaces the one-workgroup sort
// (MI355X, ids just written by another kernel: 11.0 against 9.7 us at 6001 slots,
// 22 against 10 at 16384, 37 against 13 at 32768; 9.0 against 9.7 at 4096).
// Below it the one-workgroup sort always assembles the row map itself.
constexpr int64_t kGridMinS = 5120;
static_assert(kGridMinS <= kStage / 2, "permute_index_kernel writes perm_token up to kStage / 2");

__global__ __launch_bounds__(kGridThreads) void permute_grid_kernel(
    const int32_t *__restrict__ idx, int64_t S, int64_t C, int K, int E, int capacity,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm_token,
    int32_t *__restrict__ slot_pos) {
  __shared__ int32_t red[kGridWaves][16];
  __shared__ int32_t run[8], off[9];
  __shared__ int32_t wcnt[2][kGridWaves][8];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t c0 = int64_t(blockIdx.x) * C;
  const int64_t c1 = min(S, c0 + C);

  // ---- per-expert counts of the slots before c0 and from c0 on. The ids were
  // just written by the router, so most reads go past L2: each lane keeps 8
  // 16-byte loads (4 ids each; idx is 16-byte aligned at the boundary) in flight
  // and counts in its own registers; the wavefront sums come from wave_sum at the
  // end. c0 is a multiple of 2048, so each group of 4 * kGridThreads slots lies
  // wholly before or from c0.
  int pre[8], post[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) pre[q] = post[q] = 0;
  constexpr int kPer = 4;
  for (int64_t i0 = 0; i0 < S; i0 += 8 * kPer * kGridThreads) {
    int e[8][kPer];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = i0 + (int64_t(u) * kGridThreads + tid) * kPer;
      if (i + kPer <= S) {
        const int4 v = *reinterpret_cast<const int4 *>(idx + i);
        e[u][0] = v.x;
        e[u][1] = v.y;
        e[u][2] = v.z;
        e[u][3] = v.w;
      } else {
#pragma unroll
        for (int c = 0; c < kPer; ++c) e[u][c] = i + c < S ? idx[i + c] : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (i0 + int64_t(u) * kPer * kGridThreads < c0) {
#pragma unroll
        for (int c = 0; c < kPer; ++c)
#pragma unroll
          for (int q = 0; q < 8; ++q) pre[q] += (e[u][c] == q) ? 1 : 0;
      } else {
#pragma unroll
        for (int c = 0; c < kPer; ++c)
#pragma unroll
          for (int q = 0; q < 8; ++q) post[q] += (e[u][c] == q) ? 1 : 0;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    pre[q] = wave_sum(pre[q]);
    post[q] = wave_sum(post[q]);
  }
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      red[wave][q] = pre[q];
      red[wave][8 + q] = post[q];
    }
  }
  __syncthreads();
  const int cap = capacity > 0 ? capacity : 0x7FFFFFFF;
  if (wave == 0) {
    // lane q < 8: slots of expert q before c0 (a) and from c0 on (lane q + 8's
    // sum); kept rows min(a + b, cap) scanned over the lanes into the offsets
    int v = 0;
    if (lane < 16)
      for (int w = 0; w < kGridWaves; ++w) v += red[w][lane];
    const int b = __shfl_down(v, 8, 64);
    int kept = (lane < E) ? min(v + b, cap) : 0;
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const int u = __shfl_up(kept, o, 64);
      if (lane >= o) kept += u;
    }
    if (lane < 8) {
      run[lane] = v;  // rank of this range's first slot of expert `lane`
      off[lane + 1] = kept;
    }
    if (lane == 0) off[0] = 0;
    if (blockIdx.x == 0) {
      if (lane == 0) offsets[0] = 0;
      if (lane < E) offsets[lane + 1] = kept;
    }
  }
  __syncthreads();

  // ---- rank the range in rounds of kGridThreads slots
  const uint64_t below = (uint64_t(1) << lane) - 1;
  int buf = 0;
  int e_next = c0 + tid < c1 ? idx[c0 + tid] : -1;
  for (int64_t base = c0; base < c1; base += kGridThreads, buf ^= 1) {
    const int64_t s = base + tid;
    const int e = e_next;  // this round's id, loaded during the previous round
    e_next = s + kGridThreads < c1 ? idx[s + kGridThreads] : -1;
    int my_rank = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint64_t m = __ballot(e == q);
      if (lane == q) wcnt[buf][wave][q] = int(__popcll(m));
      if (e == q) my_rank = int(__popcll(m & below));
    }
    __syncthreads();
    if (s < c1) {
      int p = -1;
      if (e >= 0 && e < E) {
        int r = run[e] + my_rank;
#pragma unroll
        for (int w = 0; w < kGridWaves; ++w) r += (w < wave) ? wcnt[buf][w][e] : 0;
        if (r < cap) p = off[e] + r;
      }
      slot_pos[s] = p;
      if (p >= 0) perm_token[p] = int32_t(s) / K;  // s < S < 2^31
    }
    __syncthreads();
    // the next round's ballots write the other wcnt buffer, so this update needs
    // no third barrier
    if (tid < 8) {
      int t = 0;
#pragma unroll
      for (int w = 0; w < kGridWaves; ++w) t += wcnt[buf][w][tid];
      run[tid] += t;
    }
  }
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
  if (S <= kSmallSlots) {
    hipLaunchKernelGGL(permute_index_small_kernel, dim3(1), dim3(64), 0, s, idx, int(S), K, E,
                       capacity, offsets, perm_token, slot_pos);
  } else if (S >= kGridMinS) {
    const int64_t per = (S + kGridMaxBlocks - 1) / kGridMaxBlocks;
    const int64_t C = max(int64_t(2048), (per + 2047) / 2048 * 2048);
    hipLaunchKernelGGL(permute_grid_kernel, dim3(unsigned((S + C - 1) / C)), dim3(kGridThreads),
                       0, s, idx, S, C, K, E, capacity, offsets, perm_token, slot_pos);
  } else {
    hipLaunchKernelGGL(permute_index_kernel, dim3(1), dim3(kThreads), 0, s, idx, S, K, E,
                       capacity, offsets, perm_token, slot_pos);
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
