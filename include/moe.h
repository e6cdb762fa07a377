/*
 * moe.h -- C ABI of an MI355X (gfx950) implementation of the Mixtral sparse
 * mixture-of-experts feed-forward layer.
 *
 * The layer (Mixtral of Experts pages: crackai "Top-2 Routing in Detail";
 * notion "Architectural details", sparse-gating and output equations):
 *   l      = x . W_g                         router logits, [T, E]
 *   G(x)   = Softmax(TopK(l))                every non-top-K logit -> -inf
 *   y_t    = sum_k w_{t,k} * SwiGLU_{i_{t,k}}(x_t)
 *   SwiGLU_e(x) = W2_e (silu(W1_e x) * (W3_e x)),  silu(z) = z / (1 + e^-z)
 * split into the steps a GPU runs: route, permute (gather each expert's tokens
 * into one contiguous segment), the two expert projections, and a weighted
 * combine back to token order.
 *
 * Conventions for every entry point
 *  - Every data pointer is a DEVICE pointer owned by the caller and must be
 *    16-byte aligned. The library never allocates, frees or synchronises; all
 *    work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    runs asynchronously. Inputs must stay valid until the work completes.
 *  - Arrays are dense and row-major. dtype applies to x, W_g, W1, W3, W2 and the
 *    hidden activations; router outputs, o_perm and the softmax are float32.
 *    bf16 is stored as its 16 upper float32 bits (round-to-nearest-even).
 *  - Inputs must be finite. Output for non-finite input is unspecified.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is enqueued and a moe_status other than MOE_OK is returned,
 *    with a message from moe_last_error() (per thread). A device fault surfaces
 *    at the caller's next synchronisation.
 *  - Supported problems: 1 <= E <= 8, K in {1, 2}, K <= E, T >= 1,
 *    T <= 2^26 and T * ceil(d / 1024) < 2^24, d and h positive multiples of
 *    128 up to 2^20, h*d < 2^31; the tiled path also bounds its grid (column
 *    blocks x token blocks), MOE_ERR_UNSUPPORTED past it.
 *  - Results are deterministic: no atomics take part in any value, and every
 *    sum has a fixed order.
 *  - Device memory of the library's own, in the code objects' static data and
 *    present on a GPU once the library is loaded there: one read-only 128 KiB
 *    row of zeros (the padding rows of the tiled kernels read it) and the
 *    MOE_NOALLOC_SCRATCH_BYTES scratch array of moe_forward_noalloc. No other
 *    call keeps any state.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                        */
  MOE_ERR_SHAPE = 2,       /* T, d, h, E or K < 1, or K > E                      */
  MOE_ERR_UNSUPPORTED = 3, /* outside the supported problems listed above        */
  MOE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                   */
  MOE_ERR_WORKSPACE = 5,   /* workspace smaller than the size query returns      */
  MOE_ERR_HIP = 6          /* the HIP runtime reported an error while enqueuing  */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Expert-projection variant. STREAM: weight streaming for small batches (an
 * expert's rows are taken 32 or 64 at a time, each group streaming the expert's
 * weights; at most 2^21 routed rows); TILED: LDS-tiled matrix-core GEMM for
 * large batches. AUTO picks STREAM when T <= MOE_STREAM_MAX_T (d <= 4096) or
 * T <= MOE_STREAM_MAX_T_WIDE (larger d), else TILED.
 * float32 problems always use one plain tiled kernel. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_STREAM = 1, MOE_PATH_TILED = 2 } moe_path;

/* Largest T for which MOE_PATH_AUTO picks MOE_PATH_STREAM: MOE_STREAM_MAX_T
 * for d <= 4096, MOE_STREAM_MAX_T_WIDE for larger d (batch-size sweeps on
 * MI355X at the Mixtral 8x7B shape, d = 4096, h = 14336, and the 8x22B shape,
 * d = 6144, h = 16384). */
#define MOE_STREAM_MAX_T 96
#define MOE_STREAM_MAX_T_WIDE 32

/* moe_problem.capacity (the capacity variant; the pages name the capacity
 * factor, a cap on the tokens per expert, as general MoE practice: ml-canon
 * page "52 Mixtral", Questions worth asking). With capacity C > 0 each expert
 * keeps its C earliest token-slots in (token, k) order; a later slot is dropped:
 * moe_permute gives it slot_pos -1 and no row, and it adds nothing to its
 * token's output (the kept weights are not renormalised). A capacity factor cf
 * corresponds to C = ceil(cf * T * K / E). 0 keeps every slot (Mixtral). */

/* Rows per expert of a capacity factor cf = cf_num / cf_den:
 * C = ceil(cf * T * K / E), in exact integer arithmetic (a float product would
 * round up one row too many whenever it lands just above an integer, e.g. 1.1 x
 * 400 / 8). Returns C (a value >= T keeps every slot), or -status when T, K or E
 * is < 1, K > E, cf_num < 0 or cf_den < 1 (MOE_ERR_SHAPE), or C does not fit an
 * int32 (MOE_ERR_UNSUPPORTED). Host only. */
int64_t moe_capacity_rows(int64_t T, int32_t K, int32_t E, int64_t cf_num, int64_t cf_den);

/* moe_problem.flags bits.
 * MOE_FLAG_DOWN_PARTIALS: the caller lets moe_expert_down / moe_expert_swiglu
 *   split the sum over h into moe_down_parts(p) float32 partial sums, stored one
 *   after another in o_perm ([parts, S, d]), and moe_combine (given the same
 *   flags) adds them in part order before weighting. With few row tiles per
 *   expert this keeps every compute unit busy in the down projection. The parts
 *   cover consecutive ranges of h, not necessarily of equal length (the library
 *   sizes them from the routing); only their sum is defined. */
#define MOE_FLAG_DOWN_PARTIALS 1

typedef struct {
  int64_t T;         /* tokens                                   */
  int64_t d;         /* model dimension                          */
  int64_t h;         /* expert hidden dimension (14336 in 8x7B)  */
  int32_t E;         /* experts (8)                              */
  int32_t K;         /* experts per token (2)                    */
  int32_t dtype;     /* moe_dtype of x, W_g, W1, W3, W2, act     */
  int32_t out_dtype; /* moe_dtype of y                           */
  int32_t path;      /* moe_path                                 */
  int32_t flags;     /* MOE_FLAG_* bits, 0 for none              */
  int32_t capacity;  /* rows per expert at most, 0 for no cap    */
  int32_t reserved;  /* must be 0                                */
} moe_problem;

/* Human-readable name of a status code. */
const char *moe_status_string(int status);

/* Detail of the last error returned on this thread ("" if none). */
const char *moe_last_error(void);

/* Number of float32 partial sums per row that moe_expert_down and
 * moe_expert_swiglu write into o_perm for `p` (1, or 2 or 4 when p->flags has
 * MOE_FLAG_DOWN_PARTIALS and the down projection is split), or -status if `p`
 * is invalid. o_perm then holds parts * S * d floats. */
int moe_down_parts(const moe_problem *p);

/* Which expert-projection variant `p` runs on (MOE_PATH_STREAM or
 * MOE_PATH_TILED), or a negative moe_status if `p` is invalid. Host only. */
int moe_resolve_path(const moe_problem *p);

/*
 * Router: logits l = x . W_g accumulated in float32 (never rounded to bf16),
 * the top-K experts by (logit descending, lower index first on an exact tie),
 * and their gate weights, the softmax of the kept logits (crackai page,
 * "Top-2 Routing in Detail"; notion page, sparse-gating equation). For K = 2:
 * w_0 = 1 / (1 + exp(l_1 - l_0)), w_1 = exp(l_1 - l_0) * w_0.
 *   x        [T, d]  dtype
 *   w_g      [d, E]  dtype
 *   topk_idx [T, K]  int32 out; slot 0 holds the larger logit
 *   topk_w   [T, K]  float32 out
 *   logits   [T, E]  float32 out, or NULL
 */
moe_status moe_route(const moe_problem *p, const void *x, const void *w_g,
                     int32_t *topk_idx, float *topk_w, float *logits, void *stream);

/*
 * Permute: stable counting sort of the S = T*K token-slots by expert, then a
 * row gather, so that each expert's tokens form one contiguous segment (the
 * gather/scatter of tokens spread unevenly over experts, ml-canon page,
 * "Questions worth asking"). Within one expert rows follow ascending slot
 * index s = t*K + k. Expert ids outside [0, E) are dropped: their slot_pos is
 * -1, they take no row, and offsets[E] counts only kept slots.
 *   x          [T, d]   dtype
 *   topk_idx   [T, K]   int32
 *   offsets    [E + 1]  int32 out: segment e is rows offsets[e] .. offsets[e+1]-1
 *   perm_token [S]      int32 out: token of each sorted row (rows >= offsets[E] untouched)
 *   slot_pos   [T, K]   int32 out: sorted row of slot (t, k)
 *   x_perm     [S, d]   dtype out: x_perm[r] = x[perm_token[r]]; or NULL: the
 *                       index arrays only (x is then not read and may be NULL),
 *                       for moe_expert_gate_up_rows, which reads the rows
 *                       through perm_token itself
 */
moe_status moe_permute(const moe_problem *p, const void *x, const int32_t *topk_idx,
                       int32_t *offsets, int32_t *perm_token, int32_t *slot_pos,
                       void *x_perm, void *stream);

/*
 * Expert gate-up projection with the SwiGLU epilogue, for every expert's
 * segment of rows: act[r] = silu(W1_e x_r) * (W3_e x_r), accumulated in float32
 * and rounded once to dtype (notion page, "Implementation": SwiGLU experts).
 *   x_perm  [S, d]     dtype (rows offsets[0] .. offsets[E]-1 are read)
 *   offsets [E + 1]    int32, non-decreasing, offsets[0] = 0, offsets[E] <= S
 *   w1, w3  [E, h, d]  dtype
 *   act     [S, h]     dtype out (rows >= offsets[E] untouched)
 */
moe_status moe_expert_gate_up(const moe_problem *p, const void *x_perm, const int32_t *offsets,
                              const void *w1, const void *w3, void *act, void *stream);

/*
 * moe_expert_gate_up with the permute's row gather folded into the
 * projection's loads: sorted row r is read from x[perm_token[r]] (the
 * gather/scatter of tokens over experts, ml-canon page, "Questions worth
 * asking"), so no x_perm copy is made. act is bitwise that of moe_permute's
 * x_perm through moe_expert_gate_up.
 *   x          [T, d]   dtype (bf16 only: MOE_ERR_UNSUPPORTED for float32)
 *   perm_token [S]      int32, as moe_permute writes it; the entries of rows
 *                       < offsets[E] must lie in [0, T) (not checked on the
 *                       device: an id out of range reads outside x)
 *   offsets, w1, w3, act as for moe_expert_gate_up
 */
moe_status moe_expert_gate_up_rows(const moe_problem *p, const void *x, const int32_t *perm_token,
                                   const int32_t *offsets, const void *w1, const void *w3,
                                   void *act, void *stream);

/*
 * Expert down projection: o_perm[r] = W2_e act[r] for every expert's segment,
 * accumulated and stored in float32 -- the outer matrix of the SwiGLU expert
 * (notion page, "Implementation": SwiGLU experts; SwiGLU_e(x) =
 * W2_e (silu(W1_e x) * W3_e x)), applied to the activations moe_expert_gate_up
 * wrote.
 *   act     [S, h]     dtype
 *   offsets [E + 1]    int32 (as above)
 *   w2      [E, d, h]  dtype
 *   o_perm  [S, d]     float32 out (rows >= offsets[E] untouched); with
 *                      MOE_FLAG_DOWN_PARTIALS [parts, S, d] partial sums,
 *                      parts = moe_down_parts(p)
 */
moe_status moe_expert_down(const moe_problem *p, const void *act, const int32_t *offsets,
                           const void *w2, float *o_perm, void *stream);

/* Bytes of workspace moe_expert_swiglu needs (0 if `p` is invalid). */
size_t moe_expert_workspace_bytes(const moe_problem *p);

/*
 * Both expert projections: o_perm[r] = SwiGLU_e(x_perm[r]) for every segment,
 * the expert function E_i of the output equation (notion page, "Architectural
 * details", y = sum_i G(x)_i E_i(x), with the SwiGLU experts of "Implementation"),
 * with the hidden activations in `ws` (at least moe_expert_workspace_bytes);
 * o_perm as for moe_expert_down.
 */
moe_status moe_expert_swiglu(const moe_problem *p, const void *x_perm, const int32_t *offsets,
                             const void *w1, const void *w3, const void *w2, float *o_perm,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * Combine: y[t] = sum_{k=0}^{K-1} topk_w[t, k] * o_perm[slot_pos[t, k]], in
 * float32 in k order, rounded once to out_dtype (crackai page,
 * y = w_1 Expert_i1(x) + w_2 Expert_i2(x); notion page, output equation).
 * Slots with slot_pos outside [0, T*K) (-1 marks a dropped slot) contribute
 * nothing. With MOE_FLAG_DOWN_PARTIALS, o_perm[r] is the sum of the
 * moe_down_parts(p) partials of row r, added in part order.
 *   o_perm   [S, d]  float32 ([parts, S, d] with MOE_FLAG_DOWN_PARTIALS)
 *   slot_pos [T, K]  int32
 *   topk_w   [T, K]  float32
 *   y        [T, d]  out_dtype out
 */
moe_status moe_combine(const moe_problem *p, const float *o_perm, const int32_t *slot_pos,
                       const float *topk_w, void *y, void *stream);

/*
 * Combine plus a residual: y[t] = residual[t] + sum_k topk_w[t, k] * o_perm[...],
 * the weighted sum formed as in moe_combine and added to the residual in
 * float32 before the single rounding to out_dtype.
 *   residual [T, d]  dtype (the input of a pre-norm block)
 */
moe_status moe_combine_residual(const moe_problem *p, const float *o_perm,
                                const int32_t *slot_pos, const float *topk_w,
                                const void *residual, void *y, void *stream);

/*
 * RMSNorm of the block input, the normalisation in front of the MoE layer in
 * Mixtral's LLaMA-like blocks (ml-canon page "52 Mixtral", Connections; the
 * pages name RMSNorm but give no formula or epsilon, so this is its standard
 * form with a caller-given eps):
 *   x[t, j] = h[t, j] / sqrt(mean_j' h[t, j']^2 + eps) * norm_w[j]
 * The mean square and the scaling are float32; x is rounded once to dtype.
 *   h [T, d] dtype, norm_w [d] dtype, x [T, d] dtype out; eps finite, > 0
 *   (MOE_ERR_UNSUPPORTED otherwise).
 */
moe_status moe_rmsnorm(const moe_problem *p, const void *h, const void *norm_w, float eps,
                       void *x, void *stream);

/* Bytes of workspace moe_block_forward needs (0 if `p` is invalid). */
size_t moe_block_workspace_bytes(const moe_problem *p);

/*
 * The pre-norm block around the layer: y = h + MoE(RMSNorm(h) * norm_w), i.e.
 * moe_rmsnorm, then the layer of moe_forward on the normalised x (kept in `ws`),
 * with the residual added in the combine step. Arguments as for moe_rmsnorm and
 * moe_forward; ws: at least moe_block_workspace_bytes(p), 256-byte aligned.
 */
moe_status moe_block_forward(const moe_problem *p, const void *h, const void *norm_w, float eps,
                             const void *w_g, const void *w1, const void *w3, const void *w2,
                             void *y, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                             void *stream);

/* Bytes of workspace moe_forward needs (0 if `p` is invalid). */
size_t moe_forward_workspace_bytes(const moe_problem *p);

/*
 * The whole layer: route -> permute -> gate-up -> down -> combine on `stream`,
 * i.e. y = sum_i G(x)_i SwiGLU_i(x) with G(x) = Softmax(Top2(x . W_g)) (notion
 * page, "Architectural details": sparse-gating and output equations; crackai
 * page, "Top-2 Routing in Detail": y = w_1 Expert_i1(x) + w_2 Expert_i2(x)).
 *   x [T, d], w_g [d, E], w1/w3 [E, h, d], w2 [E, d, h] in dtype
 *   y [T, d] out_dtype out
 *   topk_idx [T, K] int32 and topk_w [T, K] float32: optional outputs (NULL to
 *   keep them in the workspace)
 *   ws: at least moe_forward_workspace_bytes(p) bytes, 256-byte aligned
 */
moe_status moe_forward(const moe_problem *p, const void *x, const void *w_g, const void *w1,
                       const void *w3, const void *w2, void *y, int32_t *topk_idx,
                       float *topk_w, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_forward and moe_block_forward for profiling callers: the same layer,
 * bitwise the same results, plus two HIP events (hipEvent_t, created by the
 * caller, NULL for none) recorded on `stream` right before and right after the
 * launch of the expert gate-up (the layer's dominant kernel), so that its time
 * inside a stream of whole-layer calls can be read with hipEventElapsedTime.
 */
moe_status moe_forward_profiled(const moe_problem *p, const void *x, const void *w_g,
                                const void *w1, const void *w3, const void *w2, void *y,
                                int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                                void *stream, void *gate_up_begin, void *gate_up_end);
moe_status moe_block_forward_profiled(const moe_problem *p, const void *h, const void *norm_w,
                                      float eps, const void *w_g, const void *w1, const void *w3,
                                      const void *w2, void *y, int32_t *topk_idx, float *topk_w,
                                      void *ws, size_t ws_bytes, void *stream,
                                      void *gate_up_begin, void *gate_up_end);

/* Size of the static scratch array moe_forward_noalloc uses as its workspace. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * moe_forward for callers that cannot allocate device memory (code under
 * stream capture, serving loops, harnesses that forbid hipMalloc): the same
 * layer, bitwise the same results, with the workspace taken from a static
 * device array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU holds from
 * the library's load until the process ends. No call allocates or frees
 * anything. Problems whose moe_forward_workspace_bytes exceeds that size are
 * rejected with MOE_ERR_WORKSPACE (at d = 4096, h = 14336, E = 8, K = 2 this
 * admits a few hundred tokens, decode batches included). Every call on one GPU
 * uses that GPU's one array: calls that overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller. The array's
 * device address is looked up on the first call on each device (with that
 * device current). Arguments as for moe_forward, without ws and ws_bytes.
 */
moe_status moe_forward_noalloc(const moe_problem *p, const void *x, const void *w_g,
                               const void *w1, const void *w3, const void *w2, void *y,
                               int32_t *topk_idx, float *topk_w, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
