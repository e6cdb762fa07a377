"""GPU parity: every step of the HIP path against the CPU oracle on the same
seeded inputs, through the C ABI (via the thin binding).

Small shapes are compared in full, and so are the five full-size workloads: the
routing and the layer output of every token (the maximum error over all T x d
entries, against the RMS of all of them), as is the 2^18-token stress case of the
permute.
"""
import numpy as np
import pytest

import moe_inputs as mi
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mixture_experts_wg_amd as m

    return m


def _say(msg):
    print(msg, flush=True)


def _layer_ref(oracle, inp, cfg, tokens, idx_gpu, w_gpu, **routing_tol):
    l, idx, w, margin = oracle.route(inp["x"], inp["w_g"], cfg.K, cfg.dtype)
    idx_eval, diff = parity.check_routing(idx_gpu, w_gpu, l, idx, margin, cfg.K, oracle,
                                          **routing_tol)
    toks = np.union1d(tokens, diff).astype(np.int64)
    w_eval = oracle.set_weights(l, idx_eval)
    y_ref = oracle.forward_tokens(toks, inp["x"], inp["w1"], inp["w3"], inp["w2"], idx_eval,
                                  w_eval, cfg.dtype)
    return toks, y_ref, diff, margin


def _run_forward(moe, cfg, inp, path="auto", out_dtype="f32"):
    p = moe.problem(cfg.T, cfg.d, cfg.h, cfg.E, cfg.K, cfg.dtype, out_dtype, path)
    dev = parity.upload_inputs(inp, cfg.dtype)
    idx = torch.empty((cfg.T, cfg.K), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.K), dtype=torch.float32, device="cuda")
    y = moe.forward(p, dev["x"], dev["w_g"], dev["w1"], dev["w3"], dev["w2"], topk_idx=idx,
                    topk_w=w)
    torch.cuda.synchronize()
    yh = parity.host_array(y)
    if out_dtype == "bf16":
        yh = mi.bf16_bits_to_f32(yh)
    return yh.astype(np.float64), parity.host_array(idx), parity.host_array(w), dev, p


def _run_staged_as_bench(moe, cfg, dev):
    """The staged entry points in bench.py's launch configuration: partial sums
    allowed in the down projection and, for bf16, the token rows read through
    perm_token instead of a gathered copy."""
    p = moe.problem(cfg.T, cfg.d, cfg.h, cfg.E, cfg.K, cfg.dtype, "f32", "auto",
                    moe.FLAG_DOWN_PARTIALS)
    idx, w, _ = moe.route(p, dev["x"], dev["w_g"])
    if cfg.dtype == "bf16":
        off, perm, slot, _ = moe.permute(p, dev["x"], idx, gather=False)
        act = moe.expert_gate_up_rows(p, dev["x"], perm, off, dev["w1"], dev["w3"])
    else:
        off, perm, slot, xp = moe.permute(p, dev["x"], idx)
        act = moe.expert_gate_up(p, xp, off, dev["w1"], dev["w3"])
    o = moe.expert_down(p, act, off, dev["w2"])
    y = moe.combine(p, o, slot, w)
    torch.cuda.synchronize()
    return parity.host_array(y).astype(np.float64)


# ---- whole layer, small shapes (every token compared) ------------------------------

SMALL = [
    # name, config, path
    ("tiny_f32", mi.CONFIGS["tiny_f32"], "auto"),
    ("bf16_tiled_ragged", mi.Config("s1", T=1000, d=256, h=640, wg_std="fan_in_d"), "tiled"),
    # about 1024 rows per expert, every token compared
    ("bf16_tiled_T4096", mi.Config("s1b", T=4096, d=256, h=512, wg_std="fan_in_d"), "auto"),
    ("bf16_tiled_T65", mi.Config("s2", T=65, d=384, h=256, wg_std="fan_in_d"), "tiled"),
    ("bf16_auto_T97_tiled", mi.Config("s2b", T=97, d=384, h=256, wg_std="fan_in_d"), "auto"),
    ("bf16_auto_T96_stream", mi.Config("s2c", T=96, d=256, h=384, wg_std="fan_in_d"), "auto"),
    ("bf16_tiled_T193", mi.Config("s2d", T=193, d=384, h=256, wg_std="fan_in_d"), "tiled"),
    # about 113 rows per expert: still 128-token tiles (n + sqrt(n) <= 128)
    ("bf16_tiled128_T450", mi.Config("s2e", T=450, d=256, h=512, wg_std="fan_in_d"), "auto"),
    ("bf16_stream_T64", mi.Config("s3", T=64, d=512, h=1024, wg_std="fan_in_d"), "auto"),
    ("bf16_stream_T7", mi.Config("s4", T=7, d=256, h=384, wg_std="fan_in_d"), "stream"),
    ("bf16_stream_T100_multigroup", mi.Config("s5", T=100, d=256, h=256, wg_std="fan_in_d"),
     "stream"),
    ("bf16_tiled_T1", mi.Config("s6", T=1, d=128, h=128, wg_std="fan_in_d"), "tiled"),
    ("bf16_E4_K1", mi.Config("s7", T=300, d=256, h=384, E=4, K=1, wg_std="fan_in_d"), "auto"),
    ("bf16_E3_K2_stream", mi.Config("s8", T=40, d=128, h=256, E=3, K=2, wg_std="fan_in_d"),
     "stream"),
    # one expert: the layer is a dense SwiGLU FFN (w = 1); two experts with K = 2: a full
    # softmax over both
    ("bf16_E1_K1_tiled", mi.Config("s10", T=500, d=256, h=384, E=1, K=1, wg_std="fan_in_d"),
     "auto"),
    ("bf16_E2_K2_stream", mi.Config("s11", T=20, d=256, h=256, E=2, K=2, wg_std="fan_in_d"),
     "auto"),
    # 256-token tiles with fewer column blocks than XCDs (d = 384: 2 down blocks; h = 640:
    # 5 gate-up blocks) and 6 experts of about 667 rows (3 even tiles each); K = 1 with
    # about 375 rows per expert (2 tiles of 12 fragments)
    ("bf16_E6_T2000_tiled", mi.Config("s14", T=2000, d=384, h=640, E=6, K=2,
                                      wg_std="fan_in_d"), "auto"),
    ("bf16_K1_T3000_tiled", mi.Config("s15", T=3000, d=256, h=384, E=8, K=1,
                                      wg_std="fan_in_d"), "auto"),
    ("f32_ragged", mi.Config("s9", T=333, d=128, h=384, dtype="f32", w13_std="fan_in_d",
                             w2_std="fan_in_h"), "auto"),
    # extreme widths: h above the 65536-element zero row (the down projection's padding
    # rows fall back to duplicates), and a wide d for the router and the gate-up
    ("bf16_wide_h", mi.Config("s12", T=300, d=128, h=65664, wg_std="fan_in_d"), "auto"),
    ("bf16_wide_d", mi.Config("s13", T=200, d=16384, h=128, wg_std="fan_in_d"), "auto"),
    # the same widths on the streaming path (h = 128: two k-stages over four wavefronts,
    # so two of them have none)
    ("bf16_stream_wide_h", mi.Config("s14", T=20, d=128, h=65664, wg_std="fan_in_d"),
     "stream"),
    ("bf16_stream_wide_d", mi.Config("s15", T=20, d=16384, h=128, wg_std="fan_in_d"),
     "stream"),
]


@pytest.mark.parametrize("name,cfg,path", SMALL, ids=[s[0] for s in SMALL])
def test_forward_small(moe, oracle, name, cfg, path):
    _say(f"forward {name} T={cfg.T} d={cfg.d} h={cfg.h} E={cfg.E} K={cfg.K} {cfg.dtype} {path}")
    inp = mi.make_inputs(cfg, seed=0)
    y, idx, w, _, _ = _run_forward(moe, cfg, inp, path)
    toks, y_ref, diff, _ = _layer_ref(oracle, inp, cfg, np.arange(cfg.T), idx, w)
    rel = parity.check_output(y[toks], y_ref, cfg.dtype)
    _say(f"  max|err|/RMS = {rel:.3e}, near-tie set changes: {len(diff)}")


def test_forward_bf16_output(moe, oracle):
    cfg = mi.Config("o", T=130, d=256, h=384, wg_std="fan_in_d")
    inp = mi.make_inputs(cfg, seed=1)
    y, idx, w, _, _ = _run_forward(moe, cfg, inp, "auto", out_dtype="bf16")
    toks, y_ref, _, _ = _layer_ref(oracle, inp, cfg, np.arange(cfg.T), idx, w)
    # the bf16 output adds one rounding of at most half an ulp (2^-9 relative)
    y_ref_b = mi.bf16_bits_to_f32(mi.f32_to_bf16_bits(y_ref.astype(np.float32)))
    parity.check_output(y[toks], y_ref_b, "bf16")
    assert np.max(np.abs(y[toks] - y_ref)) <= 2e-2 * np.sqrt(np.mean(y_ref ** 2)) + \
        np.max(np.abs(y_ref)) * 2.0 ** -8


def test_forward_deterministic_and_paths_agree(moe):
    cfg = mi.Config("det", T=48, d=256, h=512, wg_std="fan_in_d")
    inp = mi.make_inputs(cfg, seed=2)
    y1 = _run_forward(moe, cfg, inp, "stream")[0]
    y2 = _run_forward(moe, cfg, inp, "stream")[0]
    assert np.array_equal(y1, y2), "stream path not bitwise repeatable"
    y3 = _run_forward(moe, cfg, inp, "tiled")[0]
    y4 = _run_forward(moe, cfg, inp, "tiled")[0]
    assert np.array_equal(y3, y4), "tiled path not bitwise repeatable"
    rms = np.sqrt(np.mean(y1 ** 2))
    assert np.max(np.abs(y1 - y3)) <= 1e-3 * rms


def test_batch_invariance(moe):
    """Routing and output are per token (crackai page: routing is independent per
    token): permuting the batch permutes the outputs, bit for bit."""
    cfg = mi.Config("perm", T=700, d=256, h=384, wg_std="fan_in_d")
    inp = mi.make_inputs(cfg, seed=3)
    y = _run_forward(moe, cfg, inp, "tiled")[0]
    perm = np.random.default_rng(0).permutation(cfg.T)
    inp2 = dict(inp, x=np.ascontiguousarray(inp["x"][perm]))
    y2 = _run_forward(moe, cfg, inp2, "tiled")[0]
    assert np.array_equal(y2, y[perm])


def test_identical_experts_equal_one_ffn(moe, oracle):
    cfg = mi.Config("same", T=200, d=256, h=384, wg_std="fan_in_d")
    inp = mi.make_inputs(cfg, seed=4)
    for k in ("w1", "w3", "w2"):
        inp[k] = np.ascontiguousarray(np.broadcast_to(inp[k][:1], inp[k].shape))
    y = _run_forward(moe, cfg, inp, "tiled")[0]
    one = cfg.with_(E=1, K=1)
    inp1 = dict(inp, w_g=np.ascontiguousarray(inp["w_g"][:, :1]),
                w1=inp["w1"][:1], w3=inp["w3"][:1], w2=inp["w2"][:1])
    ref = oracle.forward(inp1, 1, "bf16")["y"]
    parity.check_output(y, ref, "bf16")
    y1 = _run_forward(moe, one, inp1, "tiled")[0]
    parity.check_output(y1, ref, "bf16")


def test_skewed_routing_empty_experts(moe, oracle):
    """A router that sends every token to experts 5 and 2 leaves six experts empty."""
    cfg = mi.Config("skew", T=300, d=256, h=384, wg_std="fan_in_d")
    inp = mi.make_inputs(cfg, seed=5)
    x = mi.to_float64(inp["x"], "bf16")
    x[:, 0] = 1.0
    inp["x"] = mi.f32_to_bf16_bits(x.astype(np.float32))
    wg = mi.to_float64(inp["w_g"], "bf16")
    wg[0, :] = -8.0
    wg[0, 5] = 8.0
    wg[0, 2] = 6.0
    inp["w_g"] = mi.f32_to_bf16_bits(wg.astype(np.float32))
    for path in ("tiled", "stream"):
        y, idx, w, _, _ = _run_forward(moe, cfg, inp, path)
        assert set(np.unique(idx).tolist()) == {2, 5}
        toks, y_ref, _, _ = _layer_ref(oracle, inp, cfg, np.arange(cfg.T), idx, w)
        parity.check_output(y[toks], y_ref, "bf16", path)


# ---- the five workloads ----------------------------------------------------------

WORKLOADS = ["tiny_f32", "decode_8x7b", "prefill_8x7b", "skew_8x7b", "prefill_8x22b"]


@pytest.mark.parametrize("name", WORKLOADS)
def test_forward_workload(moe, oracle, name):
    cfg = mi.CONFIGS[name]
    _say(f"workload {name}: generating T={cfg.T} d={cfg.d} h={cfg.h}")
    inp = mi.make_inputs(cfg, seed=0)
    _say("  running GPU forward")
    y, idx, w, dev, p = _run_forward(moe, cfg, inp, "auto")
    _say("  running the staged steps as bench.py times them")
    y_st = _run_staged_as_bench(moe, cfg, dev)
    del dev
    assert np.array_equal(y_st, y), "staged steps differ from moe_forward"
    toks = np.arange(cfg.T)
    _say(f"  oracle on {len(toks)} of {cfg.T} tokens")
    toks, y_ref, diff, margin = _layer_ref(oracle, inp, cfg, toks, idx, w)
    rel = parity.check_output(y[toks], y_ref, cfg.dtype, name)
    counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
    _say(f"  {name}: max|err|/RMS = {rel:.3e} on {len(toks)} tokens; tokens with margin <= 1e-3:"
         f" {int(np.sum(margin <= 1e-3))}, set changes: {len(diff)}; rows per expert {counts.tolist()}")
    if name == "skew_8x7b":
        share = counts / counts.sum()
        assert abs(share[0] - mi.zipf_shares()[0]) < 5e-3


def test_forward_large_batch(moe, oracle):
    """2^18 tokens (524,288 slots: the permute far past its LDS staging, a tiled
    grid of about 2^16 workgroups): the permutation exactly, the routing and the
    output of every token against the oracle."""
    cfg = mi.Config("big", T=1 << 18, d=128, h=256, wg_std="fan_in_d")
    _say(f"large batch: T={cfg.T} d={cfg.d} h={cfg.h}")
    inp = mi.make_inputs(cfg, seed=5)
    y, idx, w, dev, p = _run_forward(moe, cfg, inp, "auto")
    off, perm, slot, none = moe.permute(p, None, parity.device_array(idx, "i32"), gather=False)
    torch.cuda.synchronize()
    assert none is None
    off_r, perm_r, slot_r = oracle.permute(idx, cfg.E)
    assert np.array_equal(parity.host_array(off), off_r)
    assert np.array_equal(parity.host_array(perm), perm_r)
    assert np.array_equal(parity.host_array(slot), slot_r)
    toks, y_ref, diff, _ = _layer_ref(oracle, inp, cfg, np.arange(cfg.T), idx, w)
    rel = parity.check_output(y[toks], y_ref, cfg.dtype, "large batch")
    _say(f"  max|err|/RMS = {rel:.3e} on {len(toks)} tokens, near-tie set changes: {len(diff)}")


# ---- single steps ------------------------------------------------------------------

@pytest.mark.parametrize("name", WORKLOADS + ["small_E3", "odd_T1501_d384", "odd_T2053_d384",
                                               "bf16_E6_T1100", "f32_E5_d640"])
def test_route_step(moe, oracle, name):
    if name == "small_E3":
        cfg = mi.Config("r", T=517, d=256, h=128, E=3, K=2, wg_std="fan_in_d")
    elif name == "odd_T2053_d384":  # 8 tokens per workgroup (5 in the last), 96-row quarters
        cfg = mi.Config("r", T=2053, d=384, h=128, wg_std="fan_in_d")
    elif name == "odd_T1501_d384":  # 2 tokens per workgroup, a ragged 512-row block
        cfg = mi.Config("r", T=1501, d=384, h=128, wg_std="fan_in_d")
    elif name == "bf16_E6_T1100":  # 2 tokens per workgroup (fewer than 8 experts)
        cfg = mi.Config("r", T=1101, d=384, h=128, E=6, K=2, wg_std="fan_in_d")
    elif name == "f32_E5_d640":
        cfg = mi.Config("r", T=2049, d=640, h=128, E=5, K=2, dtype="f32", wg_std="fan_in_d")
    else:
        cfg = mi.CONFIGS[name]
    inp = mi.make_inputs(cfg, seed=0, experts=False)
    p = moe.problem(cfg.T, cfg.d, cfg.h, cfg.E, cfg.K, cfg.dtype)
    dev = parity.upload_inputs(inp, cfg.dtype)
    idx, w, logits = moe.route(p, dev["x"], dev["w_g"], want_logits=True)
    torch.cuda.synchronize()
    l, idx_ref, w_ref, margin = oracle.route(inp["x"], inp["w_g"], cfg.K, cfg.dtype)
    lg = parity.host_array(logits).astype(np.float64)
    scale = np.max(np.abs(l))
    assert np.max(np.abs(lg - l)) <= 1e-5 * scale + 1e-6, "float32 logits off"
    ih = parity.host_array(idx)
    parity.check_routing(ih, parity.host_array(w), l, idx_ref, margin, cfg.K, oracle)
    # slot 0 is the larger logit (ties aside)
    la = np.take_along_axis(lg, ih[:, :1].astype(np.int64), 1)
    assert np.all(la >= np.max(lg, axis=1, keepdims=True))


PERMUTE_CASES = [
    ("random", 5000, 8, 2),
    ("one_token", 1, 8, 2),
    ("one_expert", 100, 1, 1),
    ("k1", 777, 8, 1),
    ("big", 40000, 8, 2),
    # up to 64 slots one wavefront sorts them (a decode batch: T = 32, K = 2), up
    # to 5119 one workgroup (staging slots and row map in LDS from 2048 on), from
    # 5120 a grid of workgroups of 2048-slot ranges (a ragged last range, and one
    # workgroup per 1/64 of the slots past 131072): both sides of each boundary
    ("slots_64", 32, 8, 2),
    ("slots_63", 63, 8, 1),
    ("slots_65", 65, 8, 1),
    ("slots_42_E3", 21, 3, 2),
    ("slots_2047", 2047, 8, 1),
    ("slots_2048", 1024, 8, 2),
    ("slots_5119", 5119, 8, 1),
    ("slots_5120", 2560, 8, 2),
    ("slots_6001_E5", 6001, 5, 1),
    ("slots_16384", 8192, 8, 2),
    ("slots_16385", 16385, 5, 1),
    ("slots_20000", 10000, 8, 2),
    ("slots_32768", 16384, 8, 2),
    ("slots_32769", 32769, 3, 1),
]


@pytest.mark.parametrize("case,T,E,K", PERMUTE_CASES, ids=[c[0] for c in PERMUTE_CASES])
def test_permute_step_exact(moe, oracle, case, T, E, K):
    d = 128
    idx = mi.make_routing(T, E, K, seed=T)
    x = mi.make_x(mi.Config("p", T=T, d=d, h=128, E=E, K=K), seed=1)
    p = moe.problem(T, d, 128, E, K, "bf16")
    off, perm, slot, xp = moe.permute(p, parity.device_array(x, "bf16"),
                                      parity.device_array(idx, "i32"))
    torch.cuda.synchronize()
    off_r, perm_r, slot_r = oracle.permute(idx, E)
    assert np.array_equal(parity.host_array(off), off_r)
    assert np.array_equal(parity.host_array(perm), perm_r)
    assert np.array_equal(parity.host_array(slot), slot_r)
    assert np.array_equal(parity.host_array(xp), x[perm_r])


@pytest.mark.parametrize("T", [300, 32], ids=["T300", "T32_one_wavefront"])
def test_permute_all_to_one_and_dropped_ids(moe, oracle, T):
    E, K, d = 8, 2, 256
    idx = np.zeros((T, K), dtype=np.int32)
    idx[:, 1] = 3
    idx[7, 0] = -1   # dropped
    idx[9, 1] = 8    # dropped (>= E)
    x = mi.make_x(mi.Config("p", T=T, d=d, h=128), seed=2)
    p = moe.problem(T, d, 128, E, K, "bf16")
    off, perm, slot, xp = moe.permute(p, parity.device_array(x, "bf16"),
                                      parity.device_array(idx, "i32"))
    torch.cuda.synchronize()
    keep = (idx >= 0) & (idx < E)
    flat = idx.reshape(-1)
    order = np.argsort(np.where(keep.reshape(-1), flat, E), kind="stable")[: int(keep.sum())]
    counts = np.bincount(flat[keep.reshape(-1)], minlength=E)
    assert np.array_equal(parity.host_array(off), np.concatenate([[0], np.cumsum(counts)]))
    n = int(keep.sum())
    assert np.array_equal(parity.host_array(perm)[:n], order // K)
    sh = parity.host_array(slot).reshape(-1)
    assert np.all(sh[~keep.reshape(-1)] == -1)
    assert np.array_equal(sh[order], np.arange(n))
    assert np.array_equal(parity.host_array(xp)[:n], x[order // K])


# ---- capacity variant ---------------------------------------------------------------

@pytest.mark.parametrize("T,E,K,cap", [(700, 8, 2, 1), (700, 8, 2, 50), (700, 8, 2, 175),
                                       (700, 8, 2, 100000), (333, 3, 1, 40), (64, 8, 2, 3),
                                       (32, 8, 2, 3), (40, 5, 1, 2),
                                       (5000, 8, 2, 1200), (10000, 8, 2, 2400),
                                       (20000, 8, 2, 4900)])
def test_permute_capacity_exact(moe, oracle, T, E, K, cap):
    idx = mi.make_routing(T, E, K, seed=T + cap)
    idx[: T // 2, 0] = 0  # crowd expert 0 so that the cap bites
    if K > 1:
        idx[: T // 2, 1] = np.where(idx[: T // 2, 1] == 0, 1, idx[: T // 2, 1])
    d = 128
    x = mi.make_x(mi.Config("pc", T=T, d=d, h=128, E=E, K=K), seed=3)
    p = moe.problem(T, d, 128, E, K, "bf16", capacity=cap)
    off, perm, slot, xp = moe.permute(p, parity.device_array(x, "bf16"),
                                      parity.device_array(idx, "i32"))
    torch.cuda.synchronize()
    off_r, perm_r, slot_r = oracle.permute_capped(idx, E, cap)
    n = int(off_r[-1])
    assert np.array_equal(parity.host_array(off), off_r)
    assert np.array_equal(parity.host_array(slot), slot_r)
    assert np.array_equal(parity.host_array(perm)[:n], perm_r[:n])
    assert np.array_equal(parity.host_array(xp)[:n], x[perm_r[:n]])


def _capacity_ref(oracle, inp, cfg, cap, idx_gpu, w_gpu, tokens):
    """Oracle layer under the cap, with rule R: near-tie tokens keep the GPU's valid set,
    and the cap is applied to that routing (a different set for an early token changes
    which later slots an expert still has room for)."""
    l, idx, w, margin = oracle.route(inp["x"], inp["w_g"], cfg.K, cfg.dtype)
    idx_eval, diff = parity.check_routing(idx_gpu, w_gpu, l, idx, margin, cfg.K, oracle)
    _, _, slot_ref = oracle.permute_capped(idx_eval, cfg.E, cap)
    w_cap = oracle.capped_weights(slot_ref, oracle.set_weights(l, idx_eval))
    y_ref = oracle.forward_tokens(tokens, inp["x"], inp["w1"], inp["w3"], inp["w2"], idx_eval,
                                  w_cap, cfg.dtype)
    return y_ref, slot_ref


@pytest.mark.parametrize("name,cfg,cf,path", [
    ("tiled_cf1", mi.Config("c1", T=600, d=256, h=384, wg_std="fan_in_d", zipf_bias=True), 1.0,
     "auto"),
    ("stream_cf1", mi.Config("c2", T=96, d=256, h=256, wg_std="fan_in_d", zipf_bias=True), 1.0,
     "auto"),
    ("tiled_cf0.5", mi.Config("c3", T=400, d=128, h=256, wg_std="fan_in_d"), 0.5, "tiled"),
], ids=["tiled_cf1", "stream_cf1", "tiled_cf0.5"])
def test_forward_capacity(moe, oracle, name, cfg, cf, path):
    """The capacity variant: every expert keeps its earliest C = ceil(cf T K / E) slots;
    the output matches the oracle's capped layer and the dropped slots are the same."""
    inp = mi.make_inputs(cfg, seed=15)
    cap = moe.capacity_rows(cfg.T, cfg.K, cfg.E, cf)
    p = moe.problem(cfg.T, cfg.d, cfg.h, cfg.E, cfg.K, cfg.dtype, "f32", path,
                    moe.FLAG_DOWN_PARTIALS, capacity=cap)  # partial sums as moe_forward uses
    dev = parity.upload_inputs(inp, cfg.dtype)
    idx, w, _ = moe.route(p, dev["x"], dev["w_g"])
    offsets, perm, slot, x_perm = moe.permute(p, dev["x"], idx)
    y_staged = moe.combine(p, moe.expert_swiglu(p, x_perm, offsets, dev["w1"], dev["w3"],
                                                dev["w2"]), slot, w)
    y = moe.forward(p, dev["x"], dev["w_g"], dev["w1"], dev["w3"], dev["w2"])
    torch.cuda.synchronize()
    yh = parity.host_array(y).astype(np.float64)
    assert np.array_equal(parity.host_array(y_staged).astype(np.float64), yh)
    ih, wh, sh = parity.host_array(idx), parity.host_array(w), parity.host_array(slot)
    y_ref, slot_ref = _capacity_ref(oracle, inp, cfg, cap, ih, wh, np.arange(cfg.T))
    assert np.array_equal(sh < 0, slot_ref < 0), "dropped slots differ"
    assert np.sum(sh < 0) > 0, "the cap dropped nothing: the test would test nothing"
    parity.check_output(yh, y_ref, cfg.dtype, f"capacity {name}")


def test_capacity_at_least_T_changes_nothing(moe):
    cfg = mi.Config("c4", T=300, d=256, h=384, wg_std="fan_in_d")
    inp = mi.make_inputs(cfg, seed=16)
    y0 = _run_forward(moe, cfg, inp, "tiled")[0]
    p = moe.problem(cfg.T, cfg.d, cfg.h, cfg.E, cfg.K, "bf16", "f32", "tiled", capacity=cfg.T)
    dev = parity.upload_inputs(inp, "bf16")
    y = moe.forward(p, dev["x"], dev["w_g"], dev["w1"], dev["w3"], dev["w2"])
    torch.cuda.synchronize()
    assert np.array_equal(parity.host_array(y).astype(np.float64), y0)


def _segments(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


EXPERT_CASES = [
    # name, path, T, d, h, counts per expert, flags, partial sums expected
    ("stream_mixed", "stream", 64, 512, 640, [0, 5, 64, 1, 0, 33, 17, 2], 0, 1),
    ("stream_small", "stream", 32, 256, 384, [3, 0, 0, 16, 32, 1, 0, 4], 0, 1),
    ("stream_over64", "stream", 150, 256, 256, [150, 0, 70, 0, 0, 0, 0, 1], 0, 1),
    # segments longer than T are allowed by the offsets contract (up to S = T*K)
    ("stream_segment_over_T", "stream", 40, 256, 256, [70, 0, 0, 0, 0, 0, 0, 10], 0, 1),
    ("stream_T16_segment_30", "stream", 16, 256, 256, [30, 0, 2, 0, 0, 0, 0, 0], 0, 1),
    ("tiled_mixed", "tiled", 1500, 256, 640, [0, 300, 1, 256, 513, 0, 77, 1000], 0, 1),
    ("tiled_one", "tiled", 40, 128, 128, [0, 0, 0, 0, 0, 0, 0, 1], 0, 1),
    ("tiled_d384", "tiled", 600, 384, 256, [200, 57, 0, 0, 300, 0, 1, 9], 0, 1),
    # down projection split into partial sums over h
    ("tiled_partials", "tiled", 600, 384, 512, [200, 57, 0, 0, 300, 0, 1, 9], 1, 4),
    ("tiled_partials_h1024", "tiled", 300, 256, 1024, [0, 256, 1, 0, 300, 0, 0, 40], 1, 4),
    # a few dozen rows per expert on average: 64- and 128-token tiles
    ("tiled64", "tiled", 100, 256, 512, [0, 70, 1, 64, 65, 0, 0, 0], 1, 4),
    ("tiled128", "tiled", 350, 256, 512, [129, 0, 128, 127, 1, 0, 200, 115], 1, 4),
    # many rows per expert: several 256-token tiles per segment (segments of 1, 255,
    # 256, 257 and > 1024 rows), 1, 2 and 4 partial sums
    ("tiled_many_rows", "tiled", 1200, 384, 256, [500, 0, 257, 255, 1, 0, 700, 256], 0, 1),
    ("tiled_long_segments", "tiled", 4096, 256, 384, [0, 1500, 1, 384, 769, 0, 2000, 3000], 0, 1),
    ("tiled_partials2", "tiled", 4096, 2048, 512, [0, 1500, 1, 256, 769, 0, 2000, 3000], 1, 2),
    ("tiled_partials4_long", "tiled", 4096, 256, 1024, [3000, 1, 0, 257, 0, 1500, 2000, 769], 1, 4),
    # 256-token tiles holding 16..113 rows: segments end on both sides of the 16-, 48-,
    # 64- and 112-row marks (edges of 16-token fragments and of a wavefront column's
    # 64 tokens)
    ("tiled_tail_fragments", "tiled", 600, 256, 512, [65, 112, 113, 64, 16, 17, 48, 49], 0, 1),
    ("tiled_tail_fragments_p4", "tiled", 600, 256, 512, [65, 112, 113, 64, 16, 17, 48, 49], 1,
     4),
    # an expert's 256-token tiles split its rows evenly: 5 tiles of 212-213 rows (14
    # fragments), 208-209 (13), single tiles of 224 and 225 rows (14 and 15 fragments)
    ("tiled_even_split", "tiled", 2000, 256, 512, [1062, 1043, 1026, 208, 209, 224, 225, 0],
     0, 1),
    ("tiled_even_split_p4", "tiled", 2000, 256, 512, [1062, 1043, 1026, 208, 209, 224, 225, 0],
     1, 4),
    # tiles of 1, 2, 9, 12, 13 and 16 fragments, two of 9 (262 rows) and three of 11
    # (513 rows) in one launch: every wavefront loop of the 256-token tile, with all,
    # half or none of a wavefront's token copies
    ("tiled_fragment_counts", "tiled", 2000, 256, 512, [1, 17, 129, 180, 200, 250, 262, 513],
     0, 1),
    ("tiled_fragment_counts_p4", "tiled", 2000, 256, 512,
     [1, 17, 129, 180, 200, 250, 262, 513], 1, 4),
]


@pytest.mark.parametrize("name,path,T,d,h,counts,flags,parts_expected", EXPERT_CASES,
                         ids=[c[0] for c in EXPERT_CASES])
def test_expert_steps(moe, oracle, name, path, T, d, h, counts, flags, parts_expected):
    E, K = len(counts), 2
    S = T * K
    off = _segments(counts)
    assert off[-1] <= S
    _say(f"expert steps {name}: T={T} d={d} h={h} counts={counts}")
    cfg = mi.Config("ex", T=S, d=d, h=h, E=E, K=K, x_kind="rmsnorm")
    inp = mi.make_inputs(cfg, seed=7)
    xp = inp["x"]  # [S, d] rows already "permuted"
    act_in = mi.make_act(S, h, "bf16", seed=8)
    p = moe.problem(T, d, h, E, K, "bf16", "f32", path, flags)
    parts = moe.down_parts(p)
    assert parts == parts_expected
    dev_x = parity.device_array(xp, "bf16")
    dev_off = parity.device_array(off, "i32")
    w1 = parity.device_array(inp["w1"], "bf16")
    w3 = parity.device_array(inp["w3"], "bf16")
    w2 = parity.device_array(inp["w2"], "bf16")
    act = moe.expert_gate_up(p, dev_x, dev_off, w1, w3)
    o = moe.expert_down(p, parity.device_array(act_in, "bf16"), dev_off, w2)
    o_full = moe.expert_swiglu(p, dev_x, dev_off, w1, w3, w2)
    torch.cuda.synchronize()
    # rows at and past offsets[E] are never written: read only the rows below it
    n = int(off[-1])
    act_h = mi.bf16_bits_to_f32(parity.host_array(act)[:n]).astype(np.float64)
    o_h = parity.host_array(o).astype(np.float64)
    of_h = parity.host_array(o_full).astype(np.float64)
    if parts > 1:  # [parts, S, d] partial sums over h; the row is their sum
        o_h = o_h.reshape(parts, S, d)[:, :n].sum(axis=0)
        of_h = of_h.reshape(parts, S, d)[:, :n].sum(axis=0)
    else:
        o_h, of_h = o_h[:n], of_h[:n]
    for e in range(E):
        a, b = off[e], off[e + 1]
        if a == b:
            continue
        ref = oracle.gate_up(xp[a:b], inp["w1"][e], inp["w3"][e], "bf16")
        rms = np.sqrt(np.mean(ref ** 2))
        err = np.abs(act_h[a:b] - ref) / (2.0 ** -8 * np.abs(ref) + 1e-3 * rms)
        assert np.max(err) <= 1.0, f"gate-up expert {e}: {np.max(err):.3f}"
        ref_o = oracle.down(act_in[a:b], "bf16", inp["w2"][e], "bf16")
        rms_o = np.sqrt(np.mean(ref_o ** 2))
        assert np.max(np.abs(o_h[a:b] - ref_o)) <= 2e-4 * rms_o, f"down expert {e}"
        ref_f = oracle.down(mi.f32_to_bf16_bits(ref.astype(np.float32)), "bf16", inp["w2"][e],
                            "bf16")
        parity.check_output(of_h[a:b], ref_f, "bf16", f"swiglu expert {e}")


@pytest.mark.parametrize("path,T,d,h,cap", [
    ("stream", 1, 256, 384, 0), ("stream", 40, 256, 384, 0), ("stream", 112, 384, 256, 9),
    ("tiled", 100, 256, 512, 0), ("tiled", 350, 256, 512, 0), ("tiled", 1200, 384, 256, 0),
    ("tiled", 600, 256, 256, 100),
], ids=["stream_T1", "stream_T40", "stream_T112_cap9", "tiled64_T100", "tiled128_T350",
        "tiled256_T1200", "tiled_cap100"])
def test_gate_up_rows_equals_gathered(moe, path, T, d, h, cap):
    """moe_expert_gate_up_rows (rows read through perm_token) gives bitwise the
    act of moe_permute's x_perm through moe_expert_gate_up; the index-only
    permute writes the same index arrays as the gathering one."""
    cfg = mi.Config("gr", T=T, d=d, h=h, wg_std="fan_in_d")
    inp = mi.make_inputs(cfg, seed=21)
    dev = parity.upload_inputs(inp, "bf16")
    p = moe.problem(T, d, h, 8, 2, "bf16", "f32", path, capacity=cap)
    _say(f"gate_up_rows {path} T={T} d={d} h={h} cap={cap}")
    idx, _, _ = moe.route(p, dev["x"], dev["w_g"])
    off, perm, slot, xp = moe.permute(p, dev["x"], idx)
    off2, perm2, slot2, none = moe.permute(p, None, idx, gather=False)
    assert none is None
    act = moe.expert_gate_up(p, xp, off, dev["w1"], dev["w3"])
    act2 = moe.expert_gate_up_rows(p, dev["x"], perm2, off2, dev["w1"], dev["w3"])
    torch.cuda.synchronize()
    o = parity.host_array(off)
    assert np.array_equal(o, parity.host_array(off2))
    n = int(o[-1])
    assert np.array_equal(parity.host_array(perm)[:n], parity.host_array(perm2)[:n])
    assert np.array_equal(parity.host_array(slot), parity.host_array(slot2))
    assert np.array_equal(parity.host_array(act)[:n], parity.host_array(act2)[:n])


def test_combine_step(moe):
    T, K, d = 257, 2, 384
    rng = np.random.default_rng(9)
    S = T * K
    o_perm = rng.standard_normal((S, d)).astype(np.float32)
    slot = rng.permutation(S).reshape(T, K).astype(np.int32)
    slot[5, 1] = -1
    w = rng.random((T, K)).astype(np.float32)
    p = moe.problem(T, d, 128, 8, K, "bf16", "f32")
    y = moe.combine(p, parity.device_array(o_perm, "f32"), parity.device_array(slot, "i32"),
                    parity.device_array(w, "f32"))
    torch.cuda.synchronize()
    y = parity.host_array(y).astype(np.float64)
    ref = np.zeros((T, d))
    for k in range(K):
        ok = slot[:, k] >= 0
        ref[ok] += w[ok, k:k + 1].astype(np.float64) * o_perm[slot[ok, k]].astype(np.float64)
    assert np.max(np.abs(y - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_combine_adds_partials(moe):
    """With MOE_FLAG_DOWN_PARTIALS the combine reads parts x [S, d] partial sums."""
    T, K, d, h = 300, 2, 256, 512
    p = moe.problem(T, d, h, 8, K, "bf16", "f32", "tiled", moe.FLAG_DOWN_PARTIALS)
    parts = moe.down_parts(p)
    assert parts == 4
    S = T * K
    rng = np.random.default_rng(10)
    o = rng.standard_normal((parts, S, d)).astype(np.float32)
    slot = rng.permutation(S).reshape(T, K).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    y = moe.combine(p, parity.device_array(o, "f32"), parity.device_array(slot, "i32"),
                    parity.device_array(w, "f32"))
    torch.cuda.synchronize()
    y = parity.host_array(y).astype(np.float64)
    row = o[0].copy()
    for q in range(1, parts):  # float32 sum of the parts in order, then weighted
        row += o[q]
    row = row.astype(np.float64)
    ref = sum(w[:, k:k + 1].astype(np.float64) * row[slot[:, k]] for k in range(K))
    assert np.max(np.abs(y - ref)) <= 1e-6 * np.max(np.abs(ref))


@pytest.mark.parametrize("T,cap", [(40, 0), (100, 0), (60, 9), (1, 0), (16, 0), (32, 0),
                                   (32, 5), (20, 3)])
def test_stream_forward_equals_staged(moe, T, cap):
    """On the streaming path moe_forward reads the token rows of x through perm_token
    instead of a gathered copy; the staged entry points gather with moe_permute.
    Same kernels otherwise: bit-identical outputs (also under a capacity cap), from
    one token to well past the one-wavefront sort's 64 slots."""
    cfg = mi.Config("sf", T=T, d=256, h=384, wg_std="fan_in_d")
    inp = mi.make_inputs(cfg, seed=12)
    p = moe.problem(T, cfg.d, cfg.h, cfg.E, cfg.K, "bf16", "f32", "stream", 0, cap)
    dev = parity.upload_inputs(inp, "bf16")
    y_fwd = moe.forward(p, dev["x"], dev["w_g"], dev["w1"], dev["w3"], dev["w2"])
    idx, w, _ = moe.route(p, dev["x"], dev["w_g"])
    offsets, perm, slot, x_perm = moe.permute(p, dev["x"], idx)
    act = moe.expert_gate_up(p, x_perm, offsets, dev["w1"], dev["w3"])
    o = moe.expert_down(p, act, offsets, dev["w2"])
    y = moe.combine(p, o, slot, w)
    torch.cuda.synchronize()
    assert np.array_equal(parity.host_array(y), parity.host_array(y_fwd))


@pytest.mark.parametrize("T,path", [(32, "stream"), (300, "tiled")])
def test_forward_profiled_equals_forward(moe, T, path):
    """moe_forward_profiled / moe_block_forward_profiled: bitwise the results of
    moe_forward / moe_block_forward, and the two events they record around the
    gate-up launch bracket a positive time."""
    cfg = mi.Config("fp", T=T, d=256, h=384, wg_std="fan_in_d")
    inp = mi.make_inputs(cfg, seed=21)
    blk = mi.make_block(cfg, seed=22)
    p = moe.problem(T, cfg.d, cfg.h, cfg.E, cfg.K, "bf16", "f32", path, moe.FLAG_DOWN_PARTIALS)
    dev = parity.upload_inputs(inp, "bf16")
    h_in = parity.device_array(blk["h"], "bf16")
    g = parity.device_array(blk["norm_w"], "bf16")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    y0 = moe.forward(p, dev["x"], dev["w_g"], dev["w1"], dev["w3"], dev["w2"])
    y1 = moe.forward(p, dev["x"], dev["w_g"], dev["w1"], dev["w3"], dev["w2"], events=ev[:2])
    b0 = moe.block_forward(p, h_in, g, 1e-5, dev["w_g"], dev["w1"], dev["w3"], dev["w2"])
    b1 = moe.block_forward(p, h_in, g, 1e-5, dev["w_g"], dev["w1"], dev["w3"], dev["w2"],
                           events=ev[2:])
    torch.cuda.synchronize()
    assert np.array_equal(parity.host_array(y0), parity.host_array(y1))
    assert np.array_equal(parity.host_array(b0), parity.host_array(b1))
    assert ev[0].elapsed_time(ev[1]) > 0 and ev[2].elapsed_time(ev[3]) > 0
    with pytest.raises(ValueError):
        moe.forward(p, dev["x"], dev["w_g"], dev["w1"], dev["w3"], dev["w2"],
                    events=[torch.cuda.Event(enable_timing=True)] * 2)


def test_staged_with_partials_equals_forward(moe, oracle):
    """The staged entry points with MOE_FLAG_DOWN_PARTIALS run the same kernels as
    moe_forward (which always allows partial sums): bit-identical outputs."""
    cfg = mi.Config("staged", T=500, d=256, h=512, wg_std="fan_in_d")
    inp = mi.make_inputs(cfg, seed=11)
    y_fwd = _run_forward(moe, cfg, inp, "tiled")[0]
    p = moe.problem(cfg.T, cfg.d, cfg.h, cfg.E, cfg.K, "bf16", "f32", "tiled",
                    moe.FLAG_DOWN_PARTIALS)
    parts = moe.down_parts(p)
    assert parts == 4
    dev = parity.upload_inputs(inp, "bf16")
    idx, w, _ = moe.route(p, dev["x"], dev["w_g"])
    offsets, perm, slot, x_perm = moe.permute(p, dev["x"], idx)
    act = moe.expert_gate_up(p, x_perm, offsets, dev["w1"], dev["w3"])
    o = moe.expert_down(p, act, offsets, dev["w2"])
    y = moe.combine(p, o, slot, w)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (parts, cfg.T * cfg.K, cfg.d)
    assert np.array_equal(parity.host_array(y).astype(np.float64), y_fwd)
    toks, y_ref, _, _ = _layer_ref(oracle, inp, cfg, np.arange(cfg.T), parity.host_array(idx),
                                   parity.host_array(w))
    parity.check_output(y_fwd[toks], y_ref, "bf16", "staged partials")


# ---- pre-norm block: RMSNorm before the layer, residual after ----------------------

BLOCK_EPS = 1e-5
# The GPU normalises in float32 and the oracle in float64, and each rounds x once
# to bf16, so a few elements of x differ by one bf16 unit (test_rmsnorm_step bounds
# how many). One such element moves a router logit by 2^-7 |x_j| |W_g[j, e]| at
# most, so against the oracle's own normalisation the routing of the block is
# compared with a near-tie margin of 1e-2 and a gate-weight tolerance of 2e-3
# instead of 1e-3 and 1e-5; the layer's output tolerance is unchanged. The routing
# itself is also held to the layer's rule (1e-3, 1e-5) on the x the block routed:
# moe_rmsnorm's output, bitwise the block's own (test_block_staged_equals_one_call),
# routed by the oracle (_block_routing_strict).
BLOCK_ROUTING = dict(tie_margin=1e-2, w_tol=2e-3)


@pytest.mark.parametrize("dtype,T,d", [("bf16", 33, 4096), ("bf16", 5, 128), ("f32", 17, 384)])
def test_rmsnorm_step(moe, oracle, dtype, T, d):
    cfg = mi.Config("rn", T=T, d=d, h=128, dtype=dtype)
    blk = mi.make_block(cfg, seed=12)
    p = moe.problem(T, d, 128, 8, 2, dtype, "f32")
    x = moe.rmsnorm(p, parity.device_array(blk["h"], dtype),
                    parity.device_array(blk["norm_w"], dtype), BLOCK_EPS)
    torch.cuda.synchronize()
    xg = parity.host_array(x)
    x_ref, exact = oracle.rmsnorm(blk["h"], blk["norm_w"], BLOCK_EPS, dtype)
    if dtype == "bf16":
        # float32 scaling then one rounding vs the exact value rounded once: equal
        # except where the exact value sits within float32 error of a rounding tie
        a = xg.view(np.int16).astype(np.int32)
        b = x_ref.view(np.int16).astype(np.int32)
        assert np.max(np.abs(a - b)) <= 1
        assert np.mean(a != b) < 5e-3
    else:
        err = np.abs(xg.astype(np.float64) - exact) / (np.abs(exact) + 1e-30)
        assert np.max(err) <= 2e-6


def _run_block(moe, cfg, inp, blk, path="auto", out_dtype="f32"):
    p = moe.problem(cfg.T, cfg.d, cfg.h, cfg.E, cfg.K, cfg.dtype, out_dtype, path)
    dev = parity.upload_inputs(inp, cfg.dtype)
    idx = torch.empty((cfg.T, cfg.K), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.K), dtype=torch.float32, device="cuda")
    y = moe.block_forward(p, parity.device_array(blk["h"], cfg.dtype),
                          parity.device_array(blk["norm_w"], cfg.dtype), BLOCK_EPS, dev["w_g"],
                          dev["w1"], dev["w3"], dev["w2"], topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    yh = parity.host_array(y)
    if out_dtype == "bf16":
        yh = mi.bf16_bits_to_f32(yh)
    return yh.astype(np.float64), parity.host_array(idx), parity.host_array(w), p, dev


def _block_routing_strict(moe, oracle, inp, blk, cfg, p, idx_gpu, w_gpu):
    """The block's routing against the oracle's router applied to the GPU's
    normalised x, with the layer's near-tie margin and weight tolerance."""
    x = moe.rmsnorm(p, parity.device_array(blk["h"], cfg.dtype),
                    parity.device_array(blk["norm_w"], cfg.dtype), BLOCK_EPS)
    torch.cuda.synchronize()
    xg = parity.host_array(x)
    l, idx, _, margin = oracle.route(xg, inp["w_g"], cfg.K, cfg.dtype)
    parity.check_routing(idx_gpu, w_gpu, l, idx, margin, cfg.K, oracle)


def _block_ref(oracle, inp, blk, cfg, tokens, idx_gpu, w_gpu):
    x, _ = oracle.rmsnorm(blk["h"], blk["norm_w"], BLOCK_EPS, cfg.dtype)
    toks, y_ref, diff, _ = _layer_ref(oracle, dict(inp, x=x), cfg, tokens, idx_gpu, w_gpu,
                                      **(BLOCK_ROUTING if cfg.dtype == "bf16" else {}))
    h64 = mi.to_float64(blk["h"], cfg.dtype)[toks]
    return toks, y_ref, h64, diff


@pytest.mark.parametrize("name,cfg,path", [
    ("stream_T40", mi.Config("b1", T=40, d=256, h=384, wg_std="fan_in_d"), "auto"),
    ("tiled_T300", mi.Config("b2", T=300, d=256, h=512, wg_std="fan_in_d"), "auto"),
    ("f32_T64", mi.Config("b3", T=64, d=128, h=256, dtype="f32", w13_std="fan_in_d",
                          w2_std="fan_in_h"), "auto"),
], ids=["stream_T40", "tiled_T300", "f32_T64"])
def test_block_forward(moe, oracle, name, cfg, path):
    """y = h + MoE(RMSNorm(h) g): the MoE part within the layer's tolerance of the
    oracle (the residual itself is added exactly in float32)."""
    inp = mi.make_inputs(cfg, seed=13)
    blk = mi.make_block(cfg, seed=13)
    y, idx, w, p, _ = _run_block(moe, cfg, inp, blk, path)
    _block_routing_strict(moe, oracle, inp, blk, cfg, p, idx, w)
    toks, y_ref, h64, diff = _block_ref(oracle, inp, blk, cfg, np.arange(cfg.T), idx, w)
    parity.check_output(y[toks] - h64, y_ref, cfg.dtype, f"block {name} (MoE part)")
    # the output itself: residual + MoE part, float32 rounding of the sum only
    assert np.max(np.abs(y[toks] - (h64 + y_ref))) <= \
        parity.Y_TOL[cfg.dtype] * np.sqrt(np.mean(y_ref ** 2)) + 2.0 ** -23 * np.max(np.abs(h64))


@pytest.mark.parametrize("T,d,dtype,E", [
    (250, 256, "bf16", 8), (700, 256, "bf16", 8), (1501, 256, "bf16", 8),
    (300, 128, "f32", 8), (90, 256, "bf16", 6), (1100, 128, "f32", 4), (1100, 256, "bf16", 6),
    (2053, 256, "bf16", 8),
], ids=["bf16_T250", "bf16_T700", "bf16_T1501", "f32_T300", "bf16_E6", "f32_T1100_E4",
        "bf16_T1100_E6", "bf16_T2053"])
def test_block_staged_equals_one_call(moe, T, d, dtype, E):
    """moe_rmsnorm + the staged layer + moe_combine_residual reproduce
    moe_block_forward bit for bit (routing, weights and y; bf16 output too).
    Below 2048 tokens (and for other than 8 bf16 experts) the one call normalises
    inside the router's kernel, from there on it runs the norm and the 8-token
    router as the staged calls do; T spans 1, 2 and 8 tokens per workgroup and an
    odd count in the last workgroup."""
    std = {} if dtype == "bf16" else dict(w13_std="fan_in_d", w2_std="fan_in_h")
    cfg = mi.Config("bs", T=T, d=d, h=512, E=E, dtype=dtype, wg_std="fan_in_d", **std)
    inp = mi.make_inputs(cfg, seed=14)
    blk = mi.make_block(cfg, seed=14)
    flags = moe.FLAG_DOWN_PARTIALS if dtype == "bf16" else 0
    for out_dtype in (("f32", "bf16") if dtype == "bf16" else ("f32",)):
        y1, idx1, w1, _, dev = _run_block(moe, cfg, inp, blk, "tiled", out_dtype)
        p = moe.problem(cfg.T, cfg.d, cfg.h, cfg.E, cfg.K, dtype, out_dtype, "tiled", flags)
        hdev = parity.device_array(blk["h"], dtype)
        x = moe.rmsnorm(p, hdev, parity.device_array(blk["norm_w"], dtype), BLOCK_EPS)
        idx, w, _ = moe.route(p, x, dev["w_g"])
        offsets, perm, slot, x_perm = moe.permute(p, x, idx)
        act = moe.expert_gate_up(p, x_perm, offsets, dev["w1"], dev["w3"])
        o = moe.expert_down(p, act, offsets, dev["w2"])
        y = moe.combine_residual(p, o, slot, w, hdev)
        torch.cuda.synchronize()
        assert np.array_equal(parity.host_array(idx), idx1), out_dtype
        assert np.array_equal(parity.host_array(w).view(np.uint32), w1.view(np.uint32)), out_dtype
        y2 = parity.host_array(y)
        if out_dtype == "bf16":
            y2 = mi.bf16_bits_to_f32(y2)
        assert np.array_equal(y2.astype(np.float64), y1), out_dtype


def test_block_decode_workload(moe, oracle):
    """The pre-norm block at the Mixtral 8x7B decode shape, every token checked."""
    cfg = mi.CONFIGS["decode_8x7b"]
    inp = mi.make_inputs(cfg, seed=0)
    blk = mi.make_block(cfg, seed=0)
    y, idx, w, p, dev = _run_block(moe, cfg, inp, blk, "auto")
    del dev
    _block_routing_strict(moe, oracle, inp, blk, cfg, p, idx, w)
    toks, y_ref, h64, _ = _block_ref(oracle, inp, blk, cfg, np.arange(cfg.T), idx, w)
    parity.check_output(y[toks] - h64, y_ref, cfg.dtype, "block decode_8x7b (MoE part)")


def test_errors_raise(moe):
    p = moe.problem(10, 256, 384, 8, 2, "bf16")
    x = torch.zeros((10, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        moe.route(p, x, torch.zeros((256, 7), dtype=torch.bfloat16, device="cuda"))
    bad = moe.problem(10, 200, 384, 8, 2, "bf16")
    with pytest.raises(moe.MoeError):
        moe.route(bad, torch.zeros((10, 200), dtype=torch.bfloat16, device="cuda"),
                  torch.zeros((200, 8), dtype=torch.bfloat16, device="cuda"))
