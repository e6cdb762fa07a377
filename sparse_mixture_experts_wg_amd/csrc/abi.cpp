// abi.cpp -- the C ABI declared in include/moe.h: host-side validation, the
// workspace layout and the launch sequence. No allocation, no synchronisation.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <exception>

#include "abi_internal.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

moe_status ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

}  // namespace

// Error reporting for the library's other host sources (abi_internal.h).
moe_status moe::set_error(moe_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int64_t kMaxIndex = (int64_t(1) << 31) - 1;

size_t esize(int dt) { return dt == MOE_BF16 ? 2 : 4; }
size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int resolve(const moe_problem *p);

int gate_up_tile(const moe_problem *p);
int down_tile(const moe_problem *p);

moe_status check_problem(const moe_problem *p) {
  if (!p) return fail(MOE_ERR_NULL, "problem descriptor is NULL");
  if (p->T < 1 || p->d < 1 || p->h < 1 || p->E < 1 || p->K < 1)
    return fail(MOE_ERR_SHAPE, "T=%lld d=%lld h=%lld E=%d K=%d: every size must be >= 1",
                (long long)p->T, (long long)p->d, (long long)p->h, p->E, p->K);
  if (p->K > p->E) return fail(MOE_ERR_SHAPE, "K=%d exceeds E=%d", p->K, p->E);
  if (p->E > 8) return fail(MOE_ERR_UNSUPPORTED, "E=%d: at most 8 experts", p->E);
  if (p->K > 2) return fail(MOE_ERR_UNSUPPORTED, "K=%d: K must be 1 or 2", p->K);
  if (p->d % 128 || p->h % 128)
    return fail(MOE_ERR_UNSUPPORTED, "d=%lld h=%lld: both must be multiples of 128",
                (long long)p->d, (long long)p->h);
  if (p->d > kMaxDim || p->h > kMaxDim)
    return fail(MOE_ERR_UNSUPPORTED, "d=%lld h=%lld: at most 2^20", (long long)p->d,
                (long long)p->h);
  if (p->h * p->d > kMaxIndex)
    return fail(MOE_ERR_UNSUPPORTED, "h*d=%lld: one expert matrix must stay below 2^31 elements",
                (long long)(p->h * p->d));
  if (p->T > kMaxIndex / p->K || p->T > kMaxIndex / ((p->d + 1023) / 1024) ||
      p->T > (int64_t(1) << 26))
    return fail(MOE_ERR_UNSUPPORTED, "T=%lld too large for 32-bit slot indices", (long long)p->T);
  if ((p->dtype != MOE_F32 && p->dtype != MOE_BF16) ||
      (p->out_dtype != MOE_F32 && p->out_dtype != MOE_BF16))
    return fail(MOE_ERR_UNSUPPORTED, "dtype=%d out_dtype=%d: use MOE_F32 or MOE_BF16", p->dtype,
                p->out_dtype);
  if (p->path < MOE_PATH_AUTO || p->path > MOE_PATH_TILED)
    return fail(MOE_ERR_UNSUPPORTED, "path=%d unknown", p->path);
  if (p->dtype == MOE_F32 && p->path == MOE_PATH_STREAM)
    return fail(MOE_ERR_UNSUPPORTED, "the STREAM path is bf16 only");
  if (p->capacity < 0) return fail(MOE_ERR_SHAPE, "capacity=%d must be >= 0", p->capacity);
  if (p->reserved != 0) return fail(MOE_ERR_UNSUPPORTED, "reserved field must be 0");
  if (p->flags & ~MOE_FLAG_DOWN_PARTIALS)
    return fail(MOE_ERR_UNSUPPORTED, "flags=0x%x: unknown bits", unsigned(p->flags));
  // HIP counts the work-items of a grid dimension in 32 bits. The largest 1-D
  // grids are the combine's (T * ceil(d / 1024) workgroups of 256; the router,
  // the norm and the gather launch fewer) and the tiled GEMMs' (column blocks x
  // (token blocks + E), x at most 4 partial sums for the down projection,
  // workgroups of 512).
  const int64_t kMaxItems = (int64_t(1) << 32) - 1;
  const int64_t S = p->T * p->K;
  if (p->T * ((p->d + 1023) / 1024) * 256 > kMaxItems)
    return fail(MOE_ERR_UNSUPPORTED,
                "T=%lld d=%lld: T * ceil(d / 1024) must stay below 2^24 (grid size)",
                (long long)p->T, (long long)p->d);
  // workgroups of the tiled launches (as the kernels' grid: 8 XCDs; for 256-token
  // tiles every XCD may get ceil(column blocks / 8) blocks of every token block)
  auto tiled_wgs = [&](int64_t ct, int64_t bt, int64_t parts) {
    const int64_t mt = (S + bt - 1) / bt + p->E;
    const int64_t per_xcd = bt == 256 ? (ct + 7) / 8 * mt : (ct * mt + 7) / 8;
    return per_xcd * 8 * parts;
  };
  const int64_t wgs_gu = tiled_wgs((p->h + 127) / 128, gate_up_tile(p), 1);
  const int64_t wgs_dn = tiled_wgs((p->d + 255) / 256, down_tile(p), 4);
  if (std::max(wgs_gu, wgs_dn) * 512 > kMaxItems)
    return fail(MOE_ERR_UNSUPPORTED, "problem too large for one launch (tiled grid size)");
  // stream grid: S / 32 row groups in the z dimension
  if (p->dtype == MOE_BF16 && resolve(p) == MOE_PATH_STREAM && (S + 31) / 32 >= (int64_t(1) << 16))
    return fail(MOE_ERR_UNSUPPORTED, "T=%lld too large for the STREAM path (use TILED)",
                (long long)p->T);
  return MOE_OK;
}

int resolve(const moe_problem *p) {
  if (p->dtype == MOE_F32) return MOE_PATH_TILED;
  if (p->path != MOE_PATH_AUTO) return p->path;
  const int64_t max_t = p->d <= 4096 ? MOE_STREAM_MAX_T : MOE_STREAM_MAX_T_WIDE;
  return p->T <= max_t ? MOE_PATH_STREAM : MOE_PATH_TILED;
}

moe_status check_ptr(const void *ptr, const char *name, bool required = true) {
  if (!ptr) return required ? fail(MOE_ERR_NULL, "%s is NULL", name) : MOE_OK;
  if (reinterpret_cast<uintptr_t>(ptr) % 16)
    return fail(MOE_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

#define CHECK(expr)                   \
  do {                                \
    moe_status st_ = (expr);          \
    if (st_ != MOE_OK) return st_;    \
  } while (0)

moe_status hip_result(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

// Token tile of the tiled bf16 kernels, from the rows an expert holds on
// average (n): 64 tokens up to n = 48, 128 while an expert's expected largest
// share, n + sqrt(n) rows, still fits one tile (n <= 118), 256 above. With
// small tiles each weight tile is read once and little matrix work is padding;
// once most experts spill into a second 128-token tile, 256 is faster. Measured
// on MI355X at d = 4096, h = 14336 under balanced and Zipf-skewed routing
// (T = 448: 128-token tiles 27% faster than 256; T = 496, experts of 110-141
// rows: 5% slower).
constexpr int64_t kCUs = 256;

int64_t rows_per_expert(const moe_problem *p) { return (p->T * p->K + p->E - 1) / p->E; }

int64_t isqrt(int64_t n) {
  int64_t r = 0;
  while ((r + 1) * (r + 1) <= n) ++r;
  return r;
}

int token_tile(const moe_problem *p) {
  const int64_t n = rows_per_expert(p);
  return n <= 48 ? 64 : n + isqrt(n) <= 128 ? 128 : 256;
}
int gate_up_tile(const moe_problem *p) { return token_tile(p); }
int down_tile(const moe_problem *p) { return token_tile(p); }

// Partial sums of the down projection (see MOE_FLAG_DOWN_PARTIALS): the tiled
// kernel can cut the sum over h into 2 or 4 parts, each a workgroup of its own,
// so that few tiles still fill the GPU. Workgroups run one per compute unit at
// a time (two for 64-token tiles). The tiles are estimated from an even split
// of the rows plus one standard deviation of a random split (n + sqrt(n) rows
// per expert): 4 parts when all of them fit one round, 1 part from 8 rounds
// on, else 2 -- the choices that measured fastest on MI355X from T = 64 to
// 16384 (d = 4096, h = 14336) and at d = 6144, h = 16384. Each part needs an
// even count of 64-wide k-blocks.
int down_parts(const moe_problem *p) {
  if (!(p->flags & MOE_FLAG_DOWN_PARTIALS) || p->dtype != MOE_BF16) return 1;
  if (resolve(p) != MOE_PATH_TILED) return 1;
  const int64_t bt = down_tile(p);
  const int64_t slots = bt == 64 ? 2 * kCUs : kCUs;
  const int64_t n = rows_per_expert(p);
  const int64_t sd = isqrt(n);
  const int64_t tiles = ((p->d + 255) / 256) * p->E * ((n + sd + bt - 1) / bt);
  const int64_t nk = p->h / 64;
  int parts = tiles * 4 <= slots ? 4 : (tiles + slots - 1) / slots >= 8 ? 1 : 2;
  while (parts > 1 && nk % (2 * parts)) parts /= 2;
  return parts;
}

struct ForwardLayout {
  size_t idx, w, offsets, perm, slot, x_perm, act, o_perm, total;
  int parts;
};

ForwardLayout forward_layout(const moe_problem *p) {
  const size_t S = size_t(p->T) * p->K;
  ForwardLayout L{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at += align256(bytes);
    return here;
  };
  L.idx = take(S * 4);
  L.w = take(S * 4);
  L.offsets = take(size_t(p->E + 1) * 4);
  L.perm = take(S * 4);
  L.slot = take(S * 4);
  // float32 problems gather the token rows into x_perm; the bf16 gate-up reads
  // them through perm_token and needs no copy
  L.x_perm = p->dtype == MOE_F32 ? take(S * p->d * esize(p->dtype)) : 0;
  L.act = take(S * p->h * esize(p->dtype));
  moe_problem q = *p;
  q.flags |= MOE_FLAG_DOWN_PARTIALS;  // the layer's own o_perm may hold partials
  L.parts = down_parts(&q);
  L.o_perm = take(size_t(L.parts) * S * p->d * 4);
  L.total = at;
  return L;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

// ---- the steps, after validation ----------------------------------------------

moe_status check_eps(float eps) {
  if (!(eps > 0.0f) || !(eps < 1e30f))
    return fail(MOE_ERR_UNSUPPORTED, "eps=%g: must be finite and > 0", double(eps));
  return MOE_OK;
}

moe_status do_rmsnorm(const moe_problem *p, const void *h, const void *g, float eps, void *x,
                      hipStream_t s) {
  return hip_result(moe::launch_rmsnorm(p->dtype == MOE_BF16, h, g, eps, p->T, int(p->d), x, s),
                    "rmsnorm launch");
}

moe_status do_route(const moe_problem *p, const void *x, const void *w_g, int32_t *idx, float *w,
                    float *logits, hipStream_t s) {
  return hip_result(moe::launch_route(p->dtype == MOE_BF16, x, w_g, p->T, int(p->d), p->E, p->K,
                                      idx, w, logits, s),
                    "route launch");
}

// x_perm == nullptr: the index arrays only (the caller reads x through perm).
moe_status do_permute(const moe_problem *p, const void *x, const int32_t *idx, int32_t *offsets,
                      int32_t *perm, int32_t *slot, void *x_perm, hipStream_t s) {
  const int64_t S = p->T * p->K;
  CHECK(hip_result(moe::launch_permute_index(idx, S, p->K, p->E, p->capacity, offsets, perm, slot, s),
                   "permute launch"));
  if (!x_perm) return MOE_OK;
  return hip_result(moe::launch_gather_rows(x, perm, offsets, p->E, S, p->d * esize(p->dtype),
                                            x_perm, s),
                    "gather launch");
}

// rowmap (nullable, bf16 only): sorted row r is row rowmap[r] of x_perm.
moe_status do_gate_up(const moe_problem *p, const void *x_perm, const int32_t *offsets,
                      const void *w1, const void *w3, void *act, hipStream_t s,
                      const int32_t *rowmap = nullptr) {
  const int64_t S = p->T * p->K;
  hipError_t e;
  if (p->dtype == MOE_F32)
    e = moe::launch_f32_gate_up(static_cast<const float *>(x_perm), offsets,
                                static_cast<const float *>(w1), static_cast<const float *>(w3),
                                static_cast<float *>(act), p->E, S, int(p->d), int(p->h), s);
  else if (resolve(p) == MOE_PATH_STREAM)
    e = moe::launch_stream_gate_up(x_perm, rowmap, offsets, w1, w3, act, p->E, int(p->d),
                                   int(p->h), p->T, S, s);
  else
    e = moe::launch_tiled_gate_up(x_perm, rowmap, offsets, w1, w3, act, p->E, S, int(p->d),
                                  int(p->h), gate_up_tile(p), s);
  return hip_result(e, "gate-up launch");
}

moe_status do_down(const moe_problem *p, const void *act, const int32_t *offsets, const void *w2,
                   float *o_perm, int parts, hipStream_t s) {
  const int64_t S = p->T * p->K;
  hipError_t e;
  if (p->dtype == MOE_F32)
    e = moe::launch_f32_down(static_cast<const float *>(act), offsets,
                             static_cast<const float *>(w2), o_perm, p->E, S, int(p->d), int(p->h),
                             s);
  else if (resolve(p) == MOE_PATH_STREAM)
    e = moe::launch_stream_down(act, offsets, w2, o_perm, p->E, int(p->d), int(p->h), p->T, S,
                                s);
  else
    e = moe::launch_tiled_down(act, offsets, w2, o_perm, p->E, S, int(p->d), int(p->h),
                               down_tile(p), parts, s);
  return hip_result(e, "down launch");
}

moe_status do_combine(const moe_problem *p, const float *o_perm, int parts, const int32_t *slot,
                      const float *w, const void *residual, void *y, hipStream_t s) {
  return hip_result(moe::launch_combine(o_perm, parts, slot, w, p->T, p->K, int(p->d),
                                        p->out_dtype == MOE_BF16, residual,
                                        p->dtype == MOE_BF16, y, s),
                    "combine launch");
}

template <class F>
moe_status guarded(F &&f) {
  try {
    return f();
  } catch (const std::exception &ex) {
    return fail(MOE_ERR_HIP, "internal error: %s", ex.what());
  } catch (...) {
    return fail(MOE_ERR_HIP, "internal error");
  }
}

// Arguments of the whole layer besides x; nothing is enqueued before they pass.
moe_status check_layer_args(const void *w_g, const void *w1, const void *w3, const void *w2,
                            const void *y, const int32_t *topk_idx, const float *topk_w,
                            const void *ws) {
  CHECK(check_ptr(w_g, "w_g"));
  CHECK(check_ptr(w1, "w1"));
  CHECK(check_ptr(w3, "w3"));
  CHECK(check_ptr(w2, "w2"));
  CHECK(check_ptr(y, "y"));
  CHECK(check_ptr(topk_idx, "topk_idx", false));
  CHECK(check_ptr(topk_w, "topk_w", false));
  CHECK(check_ptr(ws, "ws"));
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(MOE_ERR_ALIGN, "ws is not 256-byte aligned");
  return MOE_OK;
}

// The pre-norm block's input: x = RMSNorm(h) * g is written to `x` by the
// router's own kernel.
struct NormIn {
  const void *h, *g;
  float eps;
};

// The whole layer on checked arguments; `residual` (nullable) is added to y;
// with `norm`, x is first computed from norm->h (fused into the route step).
// ev_gu0 / ev_gu1 (nullable): HIP events recorded on the stream right before and
// right after the gate-up launch (the profiled entry points).
moe_status run_layer(const moe_problem *p, const void *x, const void *w_g, const void *w1,
                     const void *w3, const void *w2, const void *residual, void *y,
                     int32_t *topk_idx, float *topk_w, void *ws, void *stream,
                     const NormIn *norm = nullptr, hipEvent_t ev_gu0 = nullptr,
                     hipEvent_t ev_gu1 = nullptr) {
  const ForwardLayout L = forward_layout(p);
  char *base = static_cast<char *>(ws);
  int32_t *idx = topk_idx ? topk_idx : reinterpret_cast<int32_t *>(base + L.idx);
  float *w = topk_w ? topk_w : reinterpret_cast<float *>(base + L.w);
  int32_t *offsets = reinterpret_cast<int32_t *>(base + L.offsets);
  int32_t *perm = reinterpret_cast<int32_t *>(base + L.perm);
  int32_t *slot = reinterpret_cast<int32_t *>(base + L.slot);
  void *x_perm = p->dtype == MOE_F32 ? base + L.x_perm : nullptr;
  void *act = base + L.act;
  float *o_perm = reinterpret_cast<float *>(base + L.o_perm);
  const hipStream_t s = as_stream(stream);
  if (norm)
    CHECK(hip_result(moe::launch_norm_route(p->dtype == MOE_BF16, norm->h, norm->g, norm->eps, w_g,
                                            p->T, int(p->d), p->E, p->K, const_cast<void *>(x),
                                            idx, w, s),
                     "rmsnorm+route launch"));
  else
    CHECK(do_route(p, x, w_g, idx, w, nullptr, s));
  if (p->dtype == MOE_BF16) {
    // the bf16 gate-up kernels read each token row of x through perm_token, so
    // the layer needs no gathered copy of x
    CHECK(do_permute(p, x, idx, offsets, perm, slot, nullptr, s));
    if (ev_gu0) CHECK(hip_result(hipEventRecord(ev_gu0, s), "event record"));
    CHECK(do_gate_up(p, x, offsets, w1, w3, act, s, perm));
    if (ev_gu1) CHECK(hip_result(hipEventRecord(ev_gu1, s), "event record"));
  } else {
    CHECK(do_permute(p, x, idx, offsets, perm, slot, x_perm, s));
    if (ev_gu0) CHECK(hip_result(hipEventRecord(ev_gu0, s), "event record"));
    CHECK(do_gate_up(p, x_perm, offsets, w1, w3, act, s));
    if (ev_gu1) CHECK(hip_result(hipEventRecord(ev_gu1, s), "event record"));
  }
  CHECK(do_down(p, act, offsets, w2, o_perm, L.parts, s));
  CHECK(do_combine(p, o_perm, L.parts, slot, w, residual, y, s));
  return ok();
}

}  // namespace

extern "C" {

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char *moe_last_error(void) { return g_err; }

int64_t moe_capacity_rows(int64_t T, int32_t K, int32_t E, int64_t cf_num, int64_t cf_den) {
  if (T < 1 || K < 1 || E < 1 || K > E) {
    fail(MOE_ERR_SHAPE, "T=%lld K=%d E=%d: every size must be >= 1 and K <= E", (long long)T, K, E);
    return -int64_t(MOE_ERR_SHAPE);
  }
  if (cf_num < 0 || cf_den < 1) {
    fail(MOE_ERR_SHAPE, "capacity factor %lld/%lld: need num >= 0 and den >= 1",
         (long long)cf_num, (long long)cf_den);
    return -int64_t(MOE_ERR_SHAPE);
  }
  // ceil(num * T * K / (den * E)) in exact integer arithmetic
  const unsigned __int128 n = (unsigned __int128)cf_num * uint64_t(T) * uint64_t(K);
  const unsigned __int128 q = (unsigned __int128)cf_den * uint64_t(E);
  const unsigned __int128 c = (n + q - 1) / q;
  if (c > (unsigned __int128)INT32_MAX) {
    fail(MOE_ERR_UNSUPPORTED, "capacity %s rows does not fit moe_problem.capacity", "> 2^31 - 1");
    return -int64_t(MOE_ERR_UNSUPPORTED);
  }
  ok();
  return int64_t(c);
}

int moe_down_parts(const moe_problem *p) {
  const moe_status st = check_problem(p);
  if (st != MOE_OK) return -int(st);
  return down_parts(p);
}

int moe_resolve_path(const moe_problem *p) {
  const moe_status st = check_problem(p);
  if (st != MOE_OK) return -int(st);
  return resolve(p);
}

moe_status moe_route(const moe_problem *p, const void *x, const void *w_g, int32_t *topk_idx,
                     float *topk_w, float *logits, void *stream) {
  return guarded([&] {
    CHECK(check_problem(p));
    CHECK(check_ptr(x, "x"));
    CHECK(check_ptr(w_g, "w_g"));
    CHECK(check_ptr(topk_idx, "topk_idx"));
    CHECK(check_ptr(topk_w, "topk_w"));
    CHECK(check_ptr(logits, "logits", false));
    CHECK(do_route(p, x, w_g, topk_idx, topk_w, logits, as_stream(stream)));
    return ok();
  });
}

moe_status moe_permute(const moe_problem *p, const void *x, const int32_t *topk_idx,
                       int32_t *offsets, int32_t *perm_token, int32_t *slot_pos, void *x_perm,
                       void *stream) {
  return guarded([&] {
    CHECK(check_problem(p));
    CHECK(check_ptr(topk_idx, "topk_idx"));
    CHECK(check_ptr(offsets, "offsets"));
    CHECK(check_ptr(perm_token, "perm_token"));
    CHECK(check_ptr(slot_pos, "slot_pos"));
    CHECK(check_ptr(x_perm, "x_perm", false));
    if (x_perm) CHECK(check_ptr(x, "x"));  // NULL x_perm: index arrays only
    CHECK(do_permute(p, x, topk_idx, offsets, perm_token, slot_pos, x_perm, as_stream(stream)));
    return ok();
  });
}

moe_status moe_expert_gate_up(const moe_problem *p, const void *x_perm, const int32_t *offsets,
                              const void *w1, const void *w3, void *act, void *stream) {
  return guarded([&] {
    CHECK(check_problem(p));
    CHECK(check_ptr(x_perm, "x_perm"));
    CHECK(check_ptr(offsets, "offsets"));
    CHECK(check_ptr(w1, "w1"));
    CHECK(check_ptr(w3, "w3"));
    CHECK(check_ptr(act, "act"));
    CHECK(do_gate_up(p, x_perm, offsets, w1, w3, act, as_stream(stream)));
    return ok();
  });
}

moe_status moe_expert_gate_up_rows(const moe_problem *p, const void *x, const int32_t *perm_token,
                                   const int32_t *offsets, const void *w1, const void *w3,
                                   void *act, void *stream) {
  return guarded([&] {
    CHECK(check_problem(p));
    if (p->dtype != MOE_BF16)
      return fail(MOE_ERR_UNSUPPORTED,
                  "gate-up through perm_token is bf16 only; float32 reads moe_permute's x_perm");
    CHECK(check_ptr(x, "x"));
    CHECK(check_ptr(perm_token, "perm_token"));
    CHECK(check_ptr(offsets, "offsets"));
    CHECK(check_ptr(w1, "w1"));
    CHECK(check_ptr(w3, "w3"));
    CHECK(check_ptr(act, "act"));
    CHECK(do_gate_up(p, x, offsets, w1, w3, act, as_stream(stream), perm_token));
    return ok();
  });
}

moe_status moe_expert_down(const moe_problem *p, const void *act, const int32_t *offsets,
                           const void *w2, float *o_perm, void *stream) {
  return guarded([&] {
    CHECK(check_problem(p));
    CHECK(check_ptr(act, "act"));
    CHECK(check_ptr(offsets, "offsets"));
    CHECK(check_ptr(w2, "w2"));
    CHECK(check_ptr(o_perm, "o_perm"));
    CHECK(do_down(p, act, offsets, w2, o_perm, down_parts(p), as_stream(stream)));
    return ok();
  });
}

size_t moe_expert_workspace_bytes(const moe_problem *p) {
  if (check_problem(p) != MOE_OK) return 0;
  return align256(size_t(p->T) * p->K * p->h * esize(p->dtype));
}

moe_status moe_expert_swiglu(const moe_problem *p, const void *x_perm, const int32_t *offsets,
                             const void *w1, const void *w3, const void *w2, float *o_perm,
                             void *ws, size_t ws_bytes, void *stream) {
  return guarded([&] {
    CHECK(check_problem(p));
    CHECK(check_ptr(x_perm, "x_perm"));
    CHECK(check_ptr(offsets, "offsets"));
    CHECK(check_ptr(w1, "w1"));
    CHECK(check_ptr(w3, "w3"));
    CHECK(check_ptr(w2, "w2"));
    CHECK(check_ptr(o_perm, "o_perm"));
    CHECK(check_ptr(ws, "ws"));
    const size_t need = moe_expert_workspace_bytes(p);
    if (ws_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
    const hipStream_t s = as_stream(stream);
    CHECK(do_gate_up(p, x_perm, offsets, w1, w3, ws, s));
    CHECK(do_down(p, ws, offsets, w2, o_perm, down_parts(p), s));
    return ok();
  });
}

moe_status moe_combine(const moe_problem *p, const float *o_perm, const int32_t *slot_pos,
                       const float *topk_w, void *y, void *stream) {
  return guarded([&] {
    CHECK(check_problem(p));
    CHECK(check_ptr(o_perm, "o_perm"));
    CHECK(check_ptr(slot_pos, "slot_pos"));
    CHECK(check_ptr(topk_w, "topk_w"));
    CHECK(check_ptr(y, "y"));
    CHECK(do_combine(p, o_perm, down_parts(p), slot_pos, topk_w, nullptr, y, as_stream(stream)));
    return ok();
  });
}

size_t moe_forward_workspace_bytes(const moe_problem *p) {
  if (check_problem(p) != MOE_OK) return 0;
  return forward_layout(p).total;
}

moe_status moe_forward_profiled(const moe_problem *p, const void *x, const void *w_g,
                                const void *w1, const void *w3, const void *w2, void *y,
                                int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                                void *stream, void *gate_up_begin, void *gate_up_end) {
  return guarded([&] {
    CHECK(check_problem(p));
    CHECK(check_ptr(x, "x"));
    CHECK(check_layer_args(w_g, w1, w3, w2, y, topk_idx, topk_w, ws));
    if (ws_bytes < forward_layout(p).total)
      return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes,
                  forward_layout(p).total);
    return run_layer(p, x, w_g, w1, w3, w2, nullptr, y, topk_idx, topk_w, ws, stream, nullptr,
                     static_cast<hipEvent_t>(gate_up_begin), static_cast<hipEvent_t>(gate_up_end));
  });
}

moe_status moe_forward(const moe_problem *p, const void *x, const void *w_g, const void *w1,
                       const void *w3, const void *w2, void *y, int32_t *topk_idx, float *topk_w,
                       void *ws, size_t ws_bytes, void *stream) {
  return moe_forward_profiled(p, x, w_g, w1, w3, w2, y, topk_idx, topk_w, ws, ws_bytes, stream,
                              nullptr, nullptr);
}

moe_status moe_rmsnorm(const moe_problem *p, const void *h, const void *norm_w, float eps,
                       void *x, void *stream) {
  return guarded([&] {
    CHECK(check_problem(p));
    CHECK(check_eps(eps));
    CHECK(check_ptr(h, "h"));
    CHECK(check_ptr(norm_w, "norm_w"));
    CHECK(check_ptr(x, "x"));
    CHECK(do_rmsnorm(p, h, norm_w, eps, x, as_stream(stream)));
    return ok();
  });
}

moe_status moe_combine_residual(const moe_problem *p, const float *o_perm,
                                const int32_t *slot_pos, const float *topk_w,
                                const void *residual, void *y, void *stream) {
  return guarded([&] {
    CHECK(check_problem(p));
    CHECK(check_ptr(o_perm, "o_perm"));
    CHECK(check_ptr(slot_pos, "slot_pos"));
    CHECK(check_ptr(topk_w, "topk_w"));
    CHECK(check_ptr(residual, "residual"));
    CHECK(check_ptr(y, "y"));
    CHECK(do_combine(p, o_perm, down_parts(p), slot_pos, topk_w, residual, y,
                     as_stream(stream)));
    return ok();
  });
}

size_t moe_block_workspace_bytes(const moe_problem *p) {
  if (check_problem(p) != MOE_OK) return 0;
  return forward_layout(p).total + align256(size_t(p->T) * p->d * esize(p->dtype));
}

moe_status moe_block_forward(const moe_problem *p, const void *h, const void *norm_w, float eps,
                             const void *w_g, const void *w1, const void *w3, const void *w2,
                             void *y, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                             void *stream) {
  return moe_block_forward_profiled(p, h, norm_w, eps, w_g, w1, w3, w2, y, topk_idx, topk_w, ws,
                                    ws_bytes, stream, nullptr, nullptr);
}

moe_status moe_block_forward_profiled(const moe_problem *p, const void *h, const void *norm_w,
                                      float eps, const void *w_g, const void *w1, const void *w3,
                                      const void *w2, void *y, int32_t *topk_idx, float *topk_w,
                                      void *ws, size_t ws_bytes, void *stream,
                                      void *gate_up_begin, void *gate_up_end) {
  return guarded([&] {
    CHECK(check_problem(p));
    CHECK(check_eps(eps));
    CHECK(check_ptr(h, "h"));
    CHECK(check_ptr(norm_w, "norm_w"));
    CHECK(check_layer_args(w_g, w1, w3, w2, y, topk_idx, topk_w, ws));
    const size_t need = moe_block_workspace_bytes(p);
    if (ws_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
    // the normalised input x lives after the layer's own workspace
    void *x = static_cast<char *>(ws) + forward_layout(p).total;
    const NormIn norm{h, norm_w, eps};
    return run_layer(p, x, w_g, w1, w3, w2, h, y, topk_idx, topk_w, ws, stream, &norm,
                     static_cast<hipEvent_t>(gate_up_begin), static_cast<hipEvent_t>(gate_up_end));
  });
}

}  // extern "C"
