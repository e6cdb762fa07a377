/*
 * moe_oracle.c -- plain, slow, float64 CPU reference of the Mixtral sparse
 * mixture-of-experts feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY. It is loaded by the test-suite, by the smoke check
 * and by the benchmark's CPU-baseline leg, never by the product path. It shares
 * no code, header or table with the GPU implementation.
 *
 * What it computes, following the Mixtral of Experts pages:
 *   router logits   l = x . W_g, shape [tokens, 8]
 *                   (crackai "Mixtral of Experts", "Top-2 Routing in Detail")
 *   gate            G(x) = Softmax(TopK(x . W_g)); every logit outside the top K
 *                   is replaced by -inf so its weight is 0
 *                   (notion "Mixtral of Experts", "Sparse gating" equation)
 *   layer output    y = sum_i G(x)_i * SwiGLU_i(x)
 *                   (notion page, output equation with K = 2)
 *   expert          SwiGLU_i(x) = W2_i (silu(W1_i x) * (W3_i x)),
 *                   silu(z) = z / (1 + exp(-z)), no biases
 *                   (the pages name the SwiGLU expert; the explicit form is the
 *                   standard gated-linear-unit FFN with the SiLU gate)
 * The permute step (gather each expert's tokens into one contiguous segment,
 * ml-canon page, "Questions worth asking") is written as a stable counting sort.
 *
 * Around the layer (the pre-norm block): the pages build Mixtral on a
 * LLaMA-like architecture with RMSNorm (ml-canon "52 Mixtral", Connections),
 * which normalises the block input before the feed-forward layer; the block
 * output adds the layer's output to that input (the residual path):
 *   x = h / sqrt(mean_j h_j^2 + eps) * g,   out = h + y(x)
 * The pages give no formula or epsilon for RMSNorm; this is its standard form
 * with a caller-given eps. x is rounded once to the layer's input type (it is
 * the layer's input x), here directly from the double value.
 *
 * Capacity variant: the pages name the capacity factor, a cap on the tokens an
 * expert takes (ml-canon page, "Questions worth asking"), as general MoE
 * practice. With a cap of C rows per expert, an expert keeps its C earliest
 * slots in (token, k) order and drops the rest; a dropped slot contributes
 * nothing to its token's output and the kept weights are not renormalised (the
 * pages say nothing about either, this is the plain reading).
 *
 * Every value is widened exactly to double (bf16 bits << 16, or float); every
 * dot product is summed in ascending index order. A product of two bf16 or two
 * fp32 values is exact in double, so contraction into fused multiply-add cannot
 * change a router logit or a first-layer product.
 *
 * Top-K order: by logit descending, lower expert index first on an exact tie.
 *
 * Compile-time ORACLE_MUTANT=n plants one deliberate mistake; the test-suite
 * builds those variants to show that its pins catch each of them. The default
 * build (ORACLE_MUTANT undefined) has none.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

static inline double ld(const void *p, int dt, size_t i) {
  if (dt == ORACLE_BF16) {
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float *)p)[i];
}

static inline size_t esize(int dt) { return dt == ORACLE_BF16 ? 2u : 4u; }

static inline double silu(double z) {
#if ORACLE_MUTANT == 2
  return z / (1.0 + exp(z));
#else
  return z / (1.0 + exp(-z));
#endif
}

int oracle_version(void) { return 1; }
int oracle_mutant(void) { return ORACLE_MUTANT; }

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* l[t, e] = sum_j x[t, j] * W_g[j, e]; x [T, d], W_g [d, E] row-major. */
void oracle_logits(int64_t T, int64_t d, int32_t E, int32_t dt, const void *x,
                   const void *wg, double *logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      double s = 0.0;
      for (int64_t j = 0; j < d; ++j) {
#if ORACLE_MUTANT == 5
        s += ld(x, dt, (size_t)(t * d + j)) * ld(wg, dt, (size_t)e * d + j);
#else
        s += ld(x, dt, (size_t)(t * d + j)) * ld(wg, dt, (size_t)j * E + e);
#endif
      }
      logits[t * E + e] = s;
    }
  }
}

/* Index of the largest logit among experts not yet taken; the lower index
 * wins an exact tie. Returns -1 when every expert is taken. */
static int best_remaining(const double *l, int32_t E, const unsigned char *taken) {
  int best = -1;
  for (int e = 0; e < E; ++e) {
    if (taken[e]) continue;
#if ORACLE_MUTANT == 3
    if (best < 0 || l[e] < l[best]) best = e;
#else
    if (best < 0 || l[e] > l[best]) best = e;
#endif
  }
  return best;
}

/*
 * Top-K selection and the gate weights G(x) = Softmax(TopK(l)).
 *   idx[t, k]  k-th selected expert (k = 0 has the largest logit)
 *   w[t, k]    softmax of the logits with every non-selected entry at -inf,
 *              i.e. exp(l_k - m) / sum_k' exp(l_k' - m), m = the largest kept
 *   margin[t]  last kept logit minus the largest dropped one (+inf if K == E);
 *              for K = 2 this is the 2nd-to-3rd logit margin
 */
void oracle_topk(int64_t T, int32_t E, int32_t K, const double *logits,
                 int32_t *idx, double *w, double *margin) {
  for (int64_t t = 0; t < T; ++t) {
    const double *l = logits + t * E;
    unsigned char taken[64];
    memset(taken, 0, sizeof taken);
    for (int32_t k = 0; k < K; ++k) {
      int b = best_remaining(l, E, taken);
      idx[t * K + k] = b;
      taken[b] = 1;
    }
    if (margin) {
      int r = best_remaining(l, E, taken);
#if ORACLE_MUTANT == 9
      margin[t] = (K >= 2) ? l[idx[t * K]] - l[idx[t * K + 1]] : INFINITY;
      (void)r;
#else
      margin[t] = (r < 0) ? INFINITY : l[idx[t * K + K - 1]] - l[r];
#endif
    }
    double m = l[idx[t * K]];
    double z = 0.0;
#if ORACLE_MUTANT == 4
    /* softmax over all experts, no renormalisation over the kept ones */
    for (int32_t e = 0; e < E; ++e) z += exp(l[e] - m);
#else
    for (int32_t k = 0; k < K; ++k) z += exp(l[idx[t * K + k]] - m);
#endif
    for (int32_t k = 0; k < K; ++k) w[t * K + k] = exp(l[idx[t * K + k]] - m) / z;
  }
}

/*
 * Gate weights for a given expert set per token: the softmax of the logits
 * with every expert outside the set at -inf (the sparse-gating equation applied
 * to a set chosen elsewhere, e.g. by a tie-sensitive selection).
 */
void oracle_set_weights(int64_t T, int32_t E, int32_t K, const double *logits,
                        const int32_t *idx, double *w) {
  for (int64_t t = 0; t < T; ++t) {
    const double *l = logits + t * E;
    double m = l[idx[t * K]];
    for (int32_t k = 1; k < K; ++k)
      if (l[idx[t * K + k]] > m) m = l[idx[t * K + k]];
    double z = 0.0;
    for (int32_t k = 0; k < K; ++k) z += exp(l[idx[t * K + k]] - m);
    for (int32_t k = 0; k < K; ++k) w[t * K + k] = exp(l[idx[t * K + k]] - m) / z;
  }
}

/*
 * Stable counting sort of the T*K token-slots by expert.
 *   offsets[E+1]      exclusive prefix sum of the per-expert counts
 *   perm_token[S]     token of each row of the expert-sorted order
 *   slot_pos[T, K]    row of slot (t, k) in the expert-sorted order
 * Within one expert, rows follow ascending slot index s = t*K + k.
 */
void oracle_permute(int64_t T, int32_t E, int32_t K, const int32_t *idx,
                    int32_t *offsets, int32_t *perm_token, int32_t *slot_pos) {
  int64_t S = T * K;
  int64_t next[64];
  for (int32_t e = 0; e <= E; ++e) offsets[e] = 0;
  for (int64_t s = 0; s < S; ++s) offsets[idx[s] + 1] += 1;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
  for (int32_t e = 0; e < E; ++e) next[e] = offsets[e];
#if ORACLE_MUTANT == 8
  for (int64_t s = S - 1; s >= 0; --s) {
#else
  for (int64_t s = 0; s < S; ++s) {
#endif
    int64_t p = next[idx[s]]++;
    perm_token[p] = (int32_t)(s / K);
    slot_pos[s] = (int32_t)p;
  }
}

/*
 * The same stable sort with a cap of C rows per expert (C <= 0: no cap): in
 * ascending slot order an expert keeps a slot while it holds fewer than C, later
 * slots get slot_pos -1 and no row. offsets count kept rows only.
 */
void oracle_permute_capped(int64_t T, int32_t E, int32_t K, const int32_t *idx, int64_t C,
                           int32_t *offsets, int32_t *perm_token, int32_t *slot_pos) {
  int64_t S = T * K;
  int64_t seen[64], next[64];
  for (int32_t e = 0; e < E; ++e) seen[e] = 0;
  /* slot s is kept when fewer than C earlier slots went to its expert */
  for (int32_t e = 0; e <= E; ++e) offsets[e] = 0;
  for (int64_t s = 0; s < S; ++s) {
    int32_t e = idx[s];
#if ORACLE_MUTANT == 14
    int keep = (C <= 0) || (seen[e] >= 0);  /* ignores the cap */
#else
    int keep = (C <= 0) || (seen[e] < C);
#endif
    seen[e]++;
    if (keep) offsets[e + 1] += 1;
  }
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
  for (int32_t e = 0; e < E; ++e) {
    next[e] = offsets[e];
    seen[e] = 0;
  }
  for (int64_t s = 0; s < S; ++s) {
    int32_t e = idx[s];
#if ORACLE_MUTANT == 14
    int keep = (C <= 0) || (seen[e] >= 0);
#else
    int keep = (C <= 0) || (seen[e] < C);
#endif
    seen[e]++;
    if (keep) {
      int64_t p = next[e]++;
      perm_token[p] = (int32_t)(s / K);
      slot_pos[s] = (int32_t)p;
    } else {
      slot_pos[s] = -1;
    }
  }
}

#define BLK 16

/*
 * One expert on a block of nb <= BLK rows: act[r, j] = silu(g) * u with
 * g = (W1 x_r)_j, u = (W3 x_r)_j. The rows come interleaved, xt[i * BLK + r] =
 * x_r[i] (entries of rows r >= nb are zero), so that the BLK dot products that
 * share one weight row advance side by side; each of them is still its own sum
 * over i in ascending order. wrow is a d-long scratch row.
 */
static void gate_up_block(int nb, int64_t d, int64_t h, int dt, const double *xt,
                          const void *w1e, const void *w3e, double *act, double *wrow) {
  for (int64_t j = 0; j < h; ++j) {
    double g[BLK], u[BLK];
    for (int64_t i = 0; i < d; ++i) wrow[i] = ld(w1e, dt, (size_t)j * d + i);
    for (int r = 0; r < BLK; ++r) g[r] = 0.0;
    for (int64_t i = 0; i < d; ++i) {
      const double wv = wrow[i];
      const double *xi = xt + i * BLK;
      for (int r = 0; r < BLK; ++r) g[r] += xi[r] * wv;
    }
    for (int64_t i = 0; i < d; ++i) wrow[i] = ld(w3e, dt, (size_t)j * d + i);
    for (int r = 0; r < BLK; ++r) u[r] = 0.0;
    for (int64_t i = 0; i < d; ++i) {
      const double wv = wrow[i];
      const double *xi = xt + i * BLK;
      for (int r = 0; r < BLK; ++r) u[r] += xi[r] * wv;
    }
    for (int r = 0; r < nb; ++r) {
#if ORACLE_MUTANT == 1
      act[r * h + j] = silu(g[r]);
      (void)u;
#else
      act[r * h + j] = silu(g[r]) * u[r];
#endif
    }
  }
}

/*
 * out[r, i] = sum_j W2[i, j] * act[r, j] for nb <= BLK rows, each sum over j in
 * ascending order. at is h * BLK scratch for the rows interleaved as in
 * gate_up_block; wrow is h-long scratch.
 */
static void down_block(int nb, int64_t d, int64_t h, int dt, const double *act,
                       const void *w2e, double *out, double *wrow, double *at) {
  for (int64_t j = 0; j < h; ++j)
    for (int r = 0; r < BLK; ++r) at[j * BLK + r] = r < nb ? act[r * h + j] : 0.0;
  for (int64_t i = 0; i < d; ++i) {
    for (int64_t j = 0; j < h; ++j) {
#if ORACLE_MUTANT == 6
      wrow[j] = ld(w2e, dt, (size_t)j * d + i);
#else
      wrow[j] = ld(w2e, dt, (size_t)i * h + j);
#endif
    }
    double s[BLK];
    for (int r = 0; r < BLK; ++r) s[r] = 0.0;
    for (int64_t j = 0; j < h; ++j) {
      const double wv = wrow[j];
      const double *aj = at + j * BLK;
      for (int r = 0; r < BLK; ++r) s[r] += wv * aj[r];
    }
    for (int r = 0; r < nb; ++r) out[r * d + i] = s[r];
  }
}

/* xt[i * BLK + r] = x_r[i] for the nb rows given by their row pointers' element
 * offsets into x (dt), zero for r >= nb. */
static void interleave_rows(int nb, int64_t d, int dt, const void *x, const size_t *row0,
                            double *xt) {
  for (int64_t i = 0; i < d; ++i)
    for (int r = 0; r < BLK; ++r) xt[i * BLK + r] = r < nb ? ld(x, dt, row0[r] + (size_t)i) : 0.0;
}

/* act[n, h] (double) = silu(W1 x) * (W3 x) for n rows of one expert. */
void oracle_gate_up(int64_t n, int64_t d, int64_t h, int32_t dt, const void *xrows,
                    const void *w1e, const void *w3e, double *act) {
  int64_t nblk = (n + BLK - 1) / BLK;
#pragma omp parallel
  {
    double *xt = (double *)malloc(sizeof(double) * BLK * d);
    double *wrow = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b) {
      int nb = (int)((n - b * BLK) < BLK ? (n - b * BLK) : BLK);
      size_t row0[BLK];
      for (int r = 0; r < nb; ++r) row0[r] = (size_t)(b * BLK + r) * d;
      interleave_rows(nb, d, dt, xrows, row0, xt);
      gate_up_block(nb, d, h, dt, xt, w1e, w3e, act + b * BLK * h, wrow);
    }
    free(xt);
    free(wrow);
  }
}

/* out[n, d] (double) = act W2^T for n rows; act stored in act_dt, W2 in dt. */
void oracle_down(int64_t n, int64_t d, int64_t h, int32_t act_dt, const void *act,
                 int32_t dt, const void *w2e, double *out) {
  int64_t nblk = (n + BLK - 1) / BLK;
#pragma omp parallel
  {
    double *a = (double *)malloc(sizeof(double) * BLK * h);
    double *at = (double *)malloc(sizeof(double) * BLK * h);
    double *wrow = (double *)malloc(sizeof(double) * h);
#pragma omp for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b) {
      int nb = (int)((n - b * BLK) < BLK ? (n - b * BLK) : BLK);
      for (int r = 0; r < nb; ++r)
        for (int64_t j = 0; j < h; ++j) a[r * h + j] = ld(act, act_dt, (size_t)(b * BLK + r) * h + j);
      down_block(nb, d, h, dt, a, w2e, out + b * BLK * d, wrow, at);
    }
    free(a);
    free(at);
    free(wrow);
  }
}

/*
 * Layer output for a list of tokens: y[i, :] = sum_{k=0}^{K-1} w[t, k] *
 * SwiGLU_{idx[t, k]}(x_t), t = tokens[i], summed in k order starting from 0.
 * idx/w are [T, K] (from oracle_topk, or a forced expert set and its weights).
 * Work is grouped by expert in blocks of up to 16 (token, slot) pairs that share
 * one pass over the weight rows; that is cache blocking only, every sum keeps its
 * ascending order.
 */
void oracle_forward_tokens(int64_t n, const int64_t *tokens, int64_t d, int64_t h,
                           int32_t E, int32_t K, int32_t dt, const void *x,
                           const void *w1, const void *w3, const void *w2,
                           const int32_t *idx, const double *w, double *y) {
  int64_t npairs = n * K;
  /* pairs grouped by expert, ascending (i, k) within an expert */
  int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (npairs ? npairs : 1));
  int64_t cnt[65];
  memset(cnt, 0, sizeof cnt);
  for (int64_t p = 0; p < npairs; ++p) cnt[idx[tokens[p / K] * K + p % K] + 1]++;
  for (int32_t e = 0; e < E; ++e) cnt[e + 1] += cnt[e];
  int64_t fill[64];
  for (int32_t e = 0; e < E; ++e) fill[e] = cnt[e];
  for (int64_t p = 0; p < npairs; ++p) order[fill[idx[tokens[p / K] * K + p % K]]++] = p;
  /* block list: (expert, start, count) */
  int64_t nblk = 0;
  for (int32_t e = 0; e < E; ++e) nblk += (cnt[e + 1] - cnt[e] + BLK - 1) / BLK;
  int64_t *bstart = (int64_t *)malloc(sizeof(int64_t) * (nblk ? nblk : 1));
  int32_t *bexp = (int32_t *)malloc(sizeof(int32_t) * (nblk ? nblk : 1));
  int64_t nb_i = 0;
  for (int32_t e = 0; e < E; ++e)
    for (int64_t s = cnt[e]; s < cnt[e + 1]; s += BLK) {
      bstart[nb_i] = s;
      bexp[nb_i] = e;
      ++nb_i;
    }
  double *obuf = (double *)malloc(sizeof(double) * (size_t)(npairs ? npairs : 1) * d);
  size_t wsz = (size_t)h * d * esize(dt);
#pragma omp parallel
  {
    double *xt = (double *)malloc(sizeof(double) * BLK * d);
    double *act = (double *)malloc(sizeof(double) * BLK * h);
    double *at = (double *)malloc(sizeof(double) * BLK * h);
    double *ob = (double *)malloc(sizeof(double) * BLK * d);
    double *wrow = (double *)malloc(sizeof(double) * (d > h ? d : h));
#pragma omp for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b) {
      int32_t e = bexp[b];
      int64_t s0 = bstart[b];
      int nb = (int)((cnt[e + 1] - s0) < BLK ? (cnt[e + 1] - s0) : BLK);
      size_t row0[BLK];
      for (int r = 0; r < nb; ++r) row0[r] = (size_t)tokens[order[s0 + r] / K] * d;
      interleave_rows(nb, d, dt, x, row0, xt);
      const char *w1e = (const char *)w1 + (size_t)e * wsz;
      const char *w3e = (const char *)w3 + (size_t)e * wsz;
      const char *w2e = (const char *)w2 + (size_t)e * wsz;
      gate_up_block(nb, d, h, dt, xt, w1e, w3e, act, wrow);
      down_block(nb, d, h, dt, act, w2e, ob, wrow, at);
      for (int r = 0; r < nb; ++r)
        memcpy(obuf + (size_t)order[s0 + r] * d, ob + (size_t)r * d, sizeof(double) * d);
    }
    free(xt);
    free(act);
    free(at);
    free(ob);
    free(wrow);
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t t = tokens[i];
    for (int64_t c = 0; c < d; ++c) {
      double s = 0.0;
      for (int32_t k = 0; k < K; ++k) {
#if ORACLE_MUTANT == 7
        int32_t kw = K - 1 - k;
#else
        int32_t kw = k;
#endif
        s += w[t * K + kw] * obuf[(size_t)(i * K + k) * d + c];
      }
      y[i * d + c] = s;
    }
  }
  free(obuf);
  free(bstart);
  free(bexp);
  free(order);
}

/*
 * Round a double once to the nearest bfloat16 (8 significant bits), ties to
 * even; returns the bit pattern. Finite inputs in the normal range of bf16.
 */
uint16_t oracle_round_bf16(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
  int e;
  double f = frexp(fabs(v), &e); /* |v| = f * 2^e, f in [0.5, 1) */
  double m = ldexp(f, 8);        /* [128, 256): 8 significant bits kept */
  double r = nearbyint(m);       /* default rounding mode: to nearest, ties to even */
#if ORACLE_MUTANT == 13
  r = floor(m + 0.5); /* ties away from zero */
#endif
  double q = ldexp(r, e - 8);
  float qf = (float)q; /* exact: q has at most 9 significant bits */
  if (v < 0) qf = -qf;
  uint32_t u;
  memcpy(&u, &qf, sizeof u);
  return (uint16_t)(u >> 16);
}

/*
 * RMSNorm of T rows of d values (see the header):
 *   x_exact[t, j] = h[t, j] / sqrt(mean_j' h[t, j']^2 + eps) * g[j]  (double)
 *   x_out[t, j]   = x_exact rounded once to dt (bf16 bits or float)
 * Sums in ascending index order.
 */
void oracle_rmsnorm(int64_t T, int64_t d, int32_t dt, const void *h, const void *g, double eps,
                    double *x_exact, void *x_out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      double v = ld(h, dt, (size_t)(t * d + j));
      ss += v * v;
    }
#if ORACLE_MUTANT == 10
    double inv = 1.0 / sqrt(ss / (double)d);
    (void)eps;
#elif ORACLE_MUTANT == 11
    double inv = 1.0 / sqrt(ss + eps);
#else
    double inv = 1.0 / sqrt(ss / (double)d + eps);
#endif
    for (int64_t j = 0; j < d; ++j) {
#if ORACLE_MUTANT == 12
      double xv = ld(h, dt, (size_t)(t * d + j)) * inv;
      (void)g;
#else
      double xv = ld(h, dt, (size_t)(t * d + j)) * inv * ld(g, dt, (size_t)j);
#endif
      x_exact[t * d + j] = xv;
      if (dt == ORACLE_BF16)
        ((uint16_t *)x_out)[t * d + j] = oracle_round_bf16(xv);
      else
        ((float *)x_out)[t * d + j] = (float)xv;
    }
  }
}

/*
 * Gate weights after the capacity cap: a dropped slot (slot_pos < 0) weighs 0,
 * kept slots keep their weight (no renormalisation over the kept ones).
 */
void oracle_capped_weights(int64_t T, int32_t K, const int32_t *slot_pos, const double *w,
                           double *w_out) {
  for (int64_t t = 0; t < T; ++t) {
    double kept = 0.0;
    for (int32_t k = 0; k < K; ++k)
      if (slot_pos[t * K + k] >= 0) kept += w[t * K + k];
    for (int32_t k = 0; k < K; ++k) {
      double v = slot_pos[t * K + k] >= 0 ? w[t * K + k] : 0.0;
#if ORACLE_MUTANT == 15
      if (kept > 0.0) v /= kept;
#endif
      w_out[t * K + k] = v;
    }
    (void)kept;
  }
}
