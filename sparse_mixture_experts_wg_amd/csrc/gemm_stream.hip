// gemm_stream.hip -- expert projections for small batches: weight streaming.
//
// With few tokens per expert (decode), every routed expert's W1/W3/W2 must be
// read once from HBM while the arithmetic is negligible: the pages stress that
// all expert weights have to be resident although only 2 of 8 run per token
// (ml-canon page, "Questions worth asking"), and a 32-token batch reaches all 8
// experts. This kernel is built to keep HBM busy:
//
//  * A workgroup owns 16*NT output columns of one expert (for gate-up the W1
//    and the W3 rows of those columns); its 4 wavefronts split K into four
//    ranges of 64-wide k-stages (intra-workgroup split-K) and stream
//    independently; the 4 partial sums are added in LDS in the fixed order
//    0+1+2+3 (deterministic, no atomics).
//  * Weights go straight from HBM to LDS (global_load_lds_dwordx4, non-temporal:
//    each byte is used once). One instruction moves 8 weight rows x 128
//    contiguous bytes; HBM reaches about 7 TB/s with row segments of 128 bytes
//    or more, but only about 6 TB/s with the 64-byte segments that a direct
//    MFMA-operand load (16 rows x 64 bytes) would make.
//  * Each wavefront has a private ring of PD + 1 stage buffers in LDS and keeps
//    PD stages in flight; it waits with an explicit vmcnt, so no workgroup
//    barrier runs in the main loop. The 16-byte pieces of a row are XOR-swizzled
//    so that the MFMA operand reads (ds_read_b128) are free of bank conflicts.
//  * Weights are the MFMA A operand (16 weight rows x 32 k), the expert's tokens
//    the B operand (32 k x 16 tokens), v_mfma_f32_16x16x32_bf16. Token rows
//    (at most 16*KMT at a time, 2 or 4 tiles by batch size) are loaded into
//    registers with the stage they belong to; rows past the expert's end are
//    clamped duplicates whose results are never stored. An expert with no rows
//    exits before reading any weight; one with more rows than the accumulators
//    hold is split into groups of 16*KMT rows run by separate workgroups (each
//    group streams the expert's weights once more).
//  * Gate-up carries W1 and W3 rows of the same output columns, so the SwiGLU
//    epilogue silu(g) * u happens in registers before the single rounding to
//    bf16 (notion page, "Implementation").
#include "kernels.h"

namespace moe {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

constexpr int kSplitK = 4;  // wavefronts per workgroup, each a range of k-stages

// s_waitcnt immediate for vmcnt(n) alone (gfx9 encoding, n < 64).
constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// physical 16-byte piece = logical piece ^ swz16(row % 16): the 16 rows of an
// operand read land on distinct bank groups
__device__ __forceinline__ int swz16(int r) { return (r >> 1) & 7; }

// one 16-byte direct-to-LDS load per lane, non-temporal: lane L writes LDS bytes
// [16 L, 16 L + 16) after the wavefront-uniform base
__device__ __forceinline__ void dma16_nt(const uint16_t *g, lds_void *l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 2);
}

__device__ __forceinline__ bf16x8 ld16(const uint16_t *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// One group of at most 16*MT rows of expert e (rows row0 .. row0 + ne - 1).
// With a row map, sorted row r is row rowmap[r] of X (the layer reads the token
// rows straight from its input instead of a gathered copy).
template <int NMAT, int NT, int MT, int PD>
__device__ __forceinline__ void stream_rows(const uint16_t *__restrict__ X,
                                            const int32_t *__restrict__ rowmap,
                                            const uint16_t *__restrict__ Wa,
                                            const uint16_t *__restrict__ Wb,
                                            void *__restrict__ out, int N, int K, int e, int cb,
                                            int row0, int ne, lds_char *lds) {
  constexpr int NTILE = NMAT * NT;  // 16-row weight tiles: tile t = m * NT + nt
  constexpr int NR = NTILE * 16;    // weight rows per stage
  constexpr int NI = NR / 8;        // DMA instructions per stage
  constexpr int NS = PD + 1;        // ring slots
  constexpr int SB = NR * 128;      // bytes per slot: NR rows x 64 k
  constexpr int PS = NI + 2 * MT;   // vector memory instructions per stage
  static_assert(PD * PS < 64, "vmcnt range");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = cb * (16 * NT);
  const int nks = K >> 6;  // 64-wide k-stages (K is a multiple of 128)
  const int s0 = (wave * nks) / kSplitK, s1 = ((wave + 1) * nks) / kSplitK;
  lds_char *ring = lds + wave * (NS * SB);

  // DMA instruction i fills slot rows 8i .. 8i+7: lane p takes row 8i + p/8 and
  // writes physical piece p % 8, i.e. logical piece (p % 8) ^ swz16(row).
  const uint16_t *wsrc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int R = 8 * i + (lane >> 3);
    const int t = R >> 4, m = t / NT, nt = t % NT;
    const int piece = (lane & 7) ^ swz16(R & 15);
    wsrc[i] = (m == 0 ? Wa : Wb) + (size_t(e) * N + n0 + nt * 16 + (R & 15)) * size_t(K) + piece * 8;
  }
  // B operand: lane (r16, g) holds token row r16, k-piece g of a 32-wide k half
  const uint16_t *xsrc[MT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
    const int r = row0 + min(mi * 16 + r16, ne - 1);
    xsrc[mi] = X + size_t(rowmap ? rowmap[r] : r) * K + g * 8;
  }
  // A operand: lane (r16, g) reads weight row r16 of a tile, logical piece 4 hh + g
  uint32_t offA[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
    offA[hh] = uint32_t(r16 * 128 + (((4 * hh + g) ^ swz16(r16)) * 16));

  f32x4 acc[NTILE][MT];
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) acc[t][mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 tok[NS][MT][2];  // token operands of the stages in flight, by ring slot

  // Stage S into ring slot J: the weight DMA first, then the token loads. The
  // groups of a wavefront's stages stay in issue order, so "stage s is in" is
  // vmcnt(PS * stages issued after s).
#define ISSUE(J, S)                                                                        \
  {                                                                                        \
    const int kofs = (S) * 64;                                                             \
    _Pragma("unroll") for (int i = 0; i < NI; ++i)                                         \
      dma16_nt(wsrc[i] + kofs, (lds_void *)(ring + (J) * SB + i * 1024));                  \
    _Pragma("unroll") for (int mi = 0; mi < MT; ++mi)                                      \
      _Pragma("unroll") for (int hh = 0; hh < 2; ++hh)                                     \
        tok[J][mi][hh] = ld16(xsrc[mi] + kofs + hh * 32);                                  \
  }
#define COMPUTE(J)                                                                         \
  {                                                                                        \
    const lds_char *slot = ring + (J) * SB;                                                \
    bf16x8 a[NTILE][2];                                                                    \
    _Pragma("unroll") for (int t = 0; t < NTILE; ++t)                                      \
      _Pragma("unroll") for (int hh = 0; hh < 2; ++hh)                                     \
        a[t][hh] = *reinterpret_cast<lds_bf16x8 *>(slot + t * 2048 + offA[hh]);            \
    _Pragma("unroll") for (int hh = 0; hh < 2; ++hh)                                       \
      _Pragma("unroll") for (int t = 0; t < NTILE; ++t)                                    \
        _Pragma("unroll") for (int mi = 0; mi < MT; ++mi)                                  \
          acc[t][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t][hh], tok[J][mi][hh],   \
                                                               acc[t][mi], 0, 0, 0);       \
  }

  const int nst = s1 - s0;
  int base = s0;
  if (nst >= PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j) ISSUE(j, s0 + j)
    // steady state: every stage issues the one PD ahead, so each wait is exact
    // and the slot of stage s is (s - s0) % NS, known at compile time
    for (; base + NS + PD <= s1; base += NS) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        ISSUE((j + PD) % NS, base + j + PD)
        __builtin_amdgcn_s_waitcnt(vm_wait(PD * PS));
        COMPUTE(j)
      }
    }
    // tail: fewer than NS + PD stages left
#pragma unroll
    for (int j = 0; j < NS + PD - 1; ++j) {
      const int s = base + j;
      if (s >= s1) break;
      if (s + PD < s1) {
        ISSUE((j + PD) % NS, s + PD)
        __builtin_amdgcn_s_waitcnt(vm_wait(PD * PS));
      } else {
        const int later = s1 - 1 - s;  // stages issued after s, fewer than PD
        if (PD >= 3 && later == 2) __builtin_amdgcn_s_waitcnt(vm_wait(2 * PS));
        else if (PD >= 2 && later == 1) __builtin_amdgcn_s_waitcnt(vm_wait(PS));
        else __builtin_amdgcn_s_waitcnt(vm_wait(0));
      }
      COMPUTE(j % NS)
    }
  } else {
    // fewer stages than the prefetch depth (tiny K): one at a time
    for (int s = s0; s < s1; ++s) {
      ISSUE(0, s)
      __builtin_amdgcn_s_waitcnt(vm_wait(0));
      COMPUTE(0)
    }
  }
#undef ISSUE
#undef COMPUTE

  // Split-K reduction through LDS (the rings are free once every wavefront is
  // past the barrier): wavefronts 1..3 park their partial sums, wavefront 0
  // adds them in the order 1, 2, 3.
  __syncthreads();
  lds_f32x4 *red = reinterpret_cast<lds_f32x4 *>(lds);  // [kSplitK - 1][NTILE * MT][64]
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
        red[((wave - 1) * NTILE * MT + t * MT + mi) * 64 + lane] = acc[t][mi];
  }
  __syncthreads();
  if (wave != 0) return;  // the caller's barrier is reached by all wavefronts
#pragma unroll
  for (int w = 0; w < kSplitK - 1; ++w)
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) acc[t][mi] += red[(w * NTILE * MT + t * MT + mi) * 64 + lane];

  // D[i][j] of a 16x16 tile: lane holds token j = lane % 16 and weight rows
  // (output columns) i = 4 * (lane / 16) + 0..3.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const int tok_i = mi * 16 + r16;
      if (tok_i >= ne) continue;
      const int col = n0 + nt * 16 + 4 * g;
      const size_t o = size_t(row0 + tok_i) * N + col;
      if constexpr (NMAT == 2) {
        const f32x4 gv = acc[nt][mi], uv = acc[NT + nt][mi];
        uint2 q;
        q.x = pack_bf16x2(silu(gv[0]) * uv[0], silu(gv[1]) * uv[1]);
        q.y = pack_bf16x2(silu(gv[2]) * uv[2], silu(gv[3]) * uv[3]);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + o) = q;
      } else {
        const f32x4 v = acc[nt][mi];
        *reinterpret_cast<float4 *>(static_cast<float *>(out) + o) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
}

// Grid: (column blocks, E, row groups of 16*KMT rows). The row group is the
// slowest index: workgroups that read the same weight rows at the same time
// contend for the same lines (measured several times slower than one pass), so
// an expert's later row groups run after every first group and re-read its
// weights; workgroups of a row group an expert does not have exit at once.
template <int NMAT, int NT, int KMT, int PD>
__global__ __launch_bounds__(64 * kSplitK) void stream_kernel(const uint16_t *__restrict__ X,
                                                              const int32_t *__restrict__ rowmap,
                                                              const int32_t *__restrict__ offsets,
                                                              const uint16_t *__restrict__ Wa,
                                                              const uint16_t *__restrict__ Wb,
                                                              void *__restrict__ out, int N, int K) {
  constexpr int kSlot = NMAT * NT * 16 * 128;
  constexpr int kLds = kSplitK * (PD + 1) * kSlot;
  static_assert((kSplitK - 1) * NMAT * NT * KMT * 64 * 16 <= kLds, "reduction space");
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  const int e = blockIdx.y;
  const int cb = blockIdx.x;
  const int rg = blockIdx.z * (16 * KMT);
  const int seg0 = offsets[e];
  const int rows = min(offsets[e + 1] - seg0 - rg, 16 * KMT);
  if (rows <= 0) return;  // also every workgroup of an expert with no rows
  // the accumulator count follows the rows of the group, so that a 5-row expert
  // does not pay for 4 token tiles
  const int mt = (rows + 15) >> 4;
  lds_char *l = (lds_char *)lds;
  if (mt == 1)
    stream_rows<NMAT, NT, 1, PD>(X, rowmap, Wa, Wb, out, N, K, e, cb, seg0 + rg, rows, l);
  else if (KMT >= 2 && mt == 2)
    stream_rows<NMAT, NT, (KMT >= 2 ? 2 : 1), PD>(X, rowmap, Wa, Wb, out, N, K, e, cb, seg0 + rg, rows, l);
  else if (KMT >= 3 && mt == 3)
    stream_rows<NMAT, NT, (KMT >= 3 ? 3 : 1), PD>(X, rowmap, Wa, Wb, out, N, K, e, cb, seg0 + rg, rows, l);
  else
    stream_rows<NMAT, NT, KMT, PD>(X, rowmap, Wa, Wb, out, N, K, e, cb, seg0 + rg, rows, l);
}

// Measured on MI355X (decode, 8 experts of 14336 x 4096): gate-up with 2 x 32
// weight rows per workgroup and 2 stages in flight, down with 32 rows (64 rows
// once experts hold more than 32 tokens).
constexpr int kNTGateUp = 2, kPDGateUp = 2;
constexpr int kNTDownSmall = 2, kNTDownLarge = 4, kPDDown = 2;

}  // namespace

// rows_hint: the rows an expert usually has at most (T for a routed batch, whose
// experts get one row per token at most); it selects how many token tiles the
// accumulators hold. rows_bound: a bound no segment can exceed (S = offsets[E]
// at most); it sets how many row groups the grid provides. rowmap (nullable):
// sorted row r of the gate-up input is row rowmap[r] of x_perm.
hipError_t launch_stream_gate_up(const void *x_perm, const int32_t *rowmap,
                                 const int32_t *offsets, const void *w1, const void *w3,
                                 void *act, int E, int d, int h, int64_t rows_hint,
                                 int64_t rows_bound, hipStream_t s) {
  auto X = static_cast<const uint16_t *>(x_perm);
  auto A = static_cast<const uint16_t *>(w1);
  auto B = static_cast<const uint16_t *>(w3);
  const int ncb = h / (16 * kNTGateUp);
  if (rows_hint <= 32) {
    const int nz = int((rows_bound + 31) / 32);
    hipLaunchKernelGGL((stream_kernel<2, kNTGateUp, 2, kPDGateUp>),
                       dim3(unsigned(ncb), unsigned(E), unsigned(nz)), dim3(64 * kSplitK), 0, s, X,
                       rowmap, offsets, A, B, act, h, d);
  } else {
    const int nz = int((rows_bound + 63) / 64);
    hipLaunchKernelGGL((stream_kernel<2, kNTGateUp, 4, kPDGateUp>),
                       dim3(unsigned(ncb), unsigned(E), unsigned(nz)), dim3(64 * kSplitK), 0, s, X,
                       rowmap, offsets, A, B, act, h, d);
  }
  return hipGetLastError();
}

hipError_t launch_stream_down(const void *act, const int32_t *offsets, const void *w2,
                              float *o_perm, int E, int d, int h, int64_t rows_hint,
                              int64_t rows_bound, hipStream_t s) {
  auto X = static_cast<const uint16_t *>(act);
  auto A = static_cast<const uint16_t *>(w2);
  auto B = static_cast<const uint16_t *>(nullptr);
  auto O = static_cast<void *>(o_perm);
  if (rows_hint <= 32) {
    const int nz = int((rows_bound + 31) / 32);
    const int ncb = d / (16 * kNTDownSmall);
    hipLaunchKernelGGL((stream_kernel<1, kNTDownSmall, 2, kPDDown>),
                       dim3(unsigned(ncb), unsigned(E), unsigned(nz)), dim3(64 * kSplitK), 0, s, X,
                       static_cast<const int32_t *>(nullptr), offsets, A, B, O, d, h);
  } else {
    const int nz = int((rows_bound + 63) / 64);
    const int ncb = d / (16 * kNTDownLarge);
    hipLaunchKernelGGL((stream_kernel<1, kNTDownLarge, 4, kPDDown>),
                       dim3(unsigned(ncb), unsigned(E), unsigned(nz)), dim3(64 * kSplitK), 0, s, X,
                       static_cast<const int32_t *>(nullptr), offsets, A, B, O, d, h);
  }
  return hipGetLastError();
}

}  // namespace moe
