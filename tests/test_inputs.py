"""The seeded input generator (CPU only)."""
import json

import numpy as np
import pytest

import moe_inputs as mi


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e38],
                 dtype=np.float32)
    b = mi.f32_to_bf16_bits(f)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 -> 1+2^-6 (even)
    assert b.tolist()[:5] == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020]
    back = mi.bf16_bits_to_f32(b)
    assert np.all(np.abs(back - f) <= np.abs(f) * 2**-8)


def test_same_seed_same_bytes_other_seed_differs():
    cfg = mi.CONFIGS["tiny_f32"]
    a = mi.fingerprint(mi.make_inputs(cfg, 0))
    b = mi.fingerprint(mi.make_inputs(cfg, 0))
    c = mi.fingerprint(mi.make_inputs(cfg, 1))
    assert a == b
    assert all(a[k] != c[k] for k in a)


def test_streams_are_independent_of_expert_count_order():
    # x and W_g come from the first two child streams whatever else is drawn
    cfg = mi.CONFIGS["tiny_f32"]
    full = mi.make_inputs(cfg, 3)
    part = mi.make_inputs(cfg, 3, experts=False)
    assert np.array_equal(full["x"], part["x"]) and np.array_equal(full["w_g"], part["w_g"])
    assert np.array_equal(mi.make_x(cfg, 3), full["x"])


@pytest.mark.parametrize("name", list(mi.CONFIGS))
def test_shapes_dtypes_and_distributions(name):
    cfg = mi.CONFIGS[name]
    small = cfg.with_(T=min(cfg.T, 256))
    inp = mi.make_inputs(small, 0, experts=False)
    st = np.uint16 if cfg.dtype == "bf16" else np.float32
    assert inp["x"].shape == (small.T, cfg.d) and inp["x"].dtype == st
    assert inp["w_g"].shape == (cfg.d, cfg.E) and inp["w_g"].dtype == st
    x = mi.to_float64(inp["x"], cfg.dtype)
    if cfg.x_kind == "rmsnorm":
        rms = np.sqrt(np.mean(x * x, axis=1))
        assert np.all(np.abs(rms - 1.0) < 5e-3)
    else:
        assert abs(x.std() - 1.0) < 0.05
    wg = mi.to_float64(inp["w_g"], cfg.dtype)
    body = wg[1:] if cfg.zipf_bias else wg
    assert abs(body.std() / cfg.std("wg") - 1.0) < 0.1
    if cfg.zipf_bias:
        assert np.all(x[:, 0] == 1.0)
        assert np.array_equal(wg[0], mi.load_zipf_bias().astype(np.float64))


def test_expert_weights_shapes_and_std():
    cfg = mi.CONFIGS["tiny_f32"].with_(h=128)
    inp = mi.make_inputs(cfg, 0)
    assert inp["w1"].shape == (8, 128, 128) and inp["w2"].shape == (8, 128, 128)
    assert abs(inp["w1"].std() / cfg.std("w13") - 1) < 0.05
    assert abs(inp["w2"].std() / cfg.std("w2") - 1) < 0.05
    # distinct streams per expert and per matrix
    assert not np.array_equal(inp["w1"][0], inp["w1"][1])
    assert not np.array_equal(inp["w1"][0], inp["w3"][0])


def test_zipf_shares_target():
    p = mi.zipf_shares()
    assert abs(p.sum() - 1) < 1e-15 and 0.40 < p[0] < 0.45 and np.all(np.diff(p) < 0)


@pytest.mark.slow
def test_zipf_bias_reaches_target_shares(oracle):
    rec = json.load(open(mi.ZIPF_BIAS_FILE))
    assert rec["max_share_error"] < 1e-3
    cfg = mi.CONFIGS["skew_8x7b"]
    inp = mi.make_inputs(cfg, 0, experts=False)
    _, idx, _, _ = oracle.route(inp["x"], inp["w_g"], cfg.K, cfg.dtype)
    shares = np.bincount(idx.reshape(-1), minlength=cfg.E) / idx.size
    assert np.allclose(shares, rec["achieved_shares"], atol=1e-12)
    assert np.max(np.abs(shares - mi.zipf_shares())) < 1e-3


def test_make_routing_distinct_experts():
    idx = mi.make_routing(100, 8, 2, 0)
    assert idx.shape == (100, 2) and idx.dtype == np.int32
    assert np.all(idx[:, 0] != idx[:, 1]) and idx.min() >= 0 and idx.max() < 8
