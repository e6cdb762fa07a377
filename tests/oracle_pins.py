"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with: a library routine, a closed form, an invariant the pages fix, a
hand-derived example, or brute force on tiny inputs. ``PINS`` lists them; the
test-suite runs them on the real oracle (all must pass) and on deliberately
broken builds of it (each must be caught by at least one pin).
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy.special import expit, softmax

from moe_inputs import bf16_bits_to_f32, f32_to_bf16_bits, to_float64
from oracle import ref_numpy

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_bf16(rng, shape, std=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def _rand_f32(rng, shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)


def _dense_gate(idx, w, E):
    G = np.zeros((idx.shape[0], E))
    np.put_along_axis(G, idx.astype(np.int64), w, axis=1)
    return G


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) / scale if a.size else 0.0
    assert err <= rtol, f"{what}: max|diff|/max|ref| = {err:.3e} > {rtol:.1e}"


# --- router ------------------------------------------------------------------

def pin_logits_match_library_gemv(o):
    """Router logits x . W_g (crackai page, Top-2 Routing in Detail; notion page,
    sparse-gating equation) equal numpy's float64 matrix product on exactly
    widened inputs, for bf16 and fp32 storage and a non-square W_g."""
    rng = _rng(1)
    for dt in ("bf16", "f32"):
        for (T, d, E) in ((37, 96, 8), (5, 64, 3)):
            if dt == "bf16":
                x, wg = _rand_bf16(rng, (T, d)), _rand_bf16(rng, (d, E))
            else:
                x, wg = _rand_f32(rng, (T, d)), _rand_f32(rng, (d, E))
            ref = to_float64(x, dt) @ to_float64(wg, dt)
            _close(o.logits(x, wg, dt), ref, 1e-13, f"logits {dt} {T}x{d}x{E}")


def pin_bf16_widening_exact(o):
    """bf16 storage is widened exactly: known bit patterns give known logits."""
    bits = np.array([[0x3F80, 0xC020, 0x3F00, 0x4100]], dtype=np.uint16)  # 1, -2.5, 0.5, 8
    wg = f32_to_bf16_bits(np.eye(4, dtype=np.float32))
    l = o.logits(bits, wg, "bf16")
    assert np.array_equal(l, np.array([[1.0, -2.5, 0.5, 8.0]])), l
    assert np.array_equal(bf16_bits_to_f32(bits).astype(np.float64), l)


def pin_topk_is_masked_softmax(o):
    """G(x) = Softmax(TopK(l)) with every non-top-K logit at -inf (notion page,
    sparse-gating equation): dense gate equals scipy's softmax of the masked
    logits, for K = 1, 2, 3."""
    rng = _rng(2)
    l = rng.standard_normal((300, 8)) * 2.0
    for K in (1, 2, 3):
        idx, w, _ = o.topk(l, K)
        ref_sets = ref_numpy.topk_sets(l, K)
        assert np.array_equal(np.sort(idx, 1), np.sort(ref_sets, 1)), f"top-{K} sets"
        G = _dense_gate(idx, w, 8)
        G_ref = ref_numpy.masked_softmax_gate(l, K)
        assert np.max(np.abs(G - G_ref)) <= 1e-15, f"masked softmax K={K}"


def pin_topk_matches_softmax_then_renormalise(o):
    """The ml-canon page's snippet (softmax over all 8, keep 2, divide by their
    sum) gives the same sets, order and weights as the oracle."""
    rng = _rng(3)
    l = rng.standard_normal((400, 8)) * 1.5
    idx, w, _ = o.topk(l, 2)
    idx2, w2 = ref_numpy.softmax_topk_renorm_gate(l, 2)
    assert np.array_equal(idx, idx2), "slot order / sets"
    assert np.max(np.abs(w - w2)) <= 1e-15, np.max(np.abs(w - w2))


def pin_two_way_closed_form(o):
    """With two kept logits l_a >= l_b: w_a = sigma(l_a - l_b), w_b = 1 - w_a,
    and the slot-0 expert has the larger logit (crackai page, y = w_1 E_i1 + w_2 E_i2)."""
    rng = _rng(4)
    l = rng.standard_normal((500, 8)) * 3.0
    idx, w, _ = o.topk(l, 2)
    la = np.take_along_axis(l, idx[:, :1].astype(np.int64), 1)[:, 0]
    lb = np.take_along_axis(l, idx[:, 1:].astype(np.int64), 1)[:, 0]
    assert np.all(la >= lb)
    assert np.max(np.abs(w[:, 0] - expit(la - lb))) <= 2e-16
    assert np.max(np.abs(w.sum(1) - 1.0)) <= 4.5e-16


def pin_weights_sum_to_one(o):
    """The kept weights of every token sum to 1 (softmax over the kept logits)."""
    rng = _rng(5)
    l = rng.standard_normal((200, 8)) * 4.0
    for K in (1, 2, 4, 8):
        _, w, _ = o.topk(l, K)
        assert np.max(np.abs(w.sum(1) - 1.0)) <= 1e-15, K


def pin_full_softmax_when_K_equals_E(o):
    """K = E keeps every expert: the gate is the plain softmax of the logits."""
    rng = _rng(6)
    l = rng.standard_normal((100, 8))
    idx, w, margin = o.topk(l, 8)
    assert np.max(np.abs(_dense_gate(idx, w, 8) - softmax(l, axis=1))) <= 1e-15
    assert np.all(np.isinf(margin))


def pin_tie_break_and_margin(o):
    """Exact ties go to the lower expert index; margin = last kept minus the
    largest dropped logit (numpy sort)."""
    l = np.array([[0.5, 2.0, 2.0, 1.0, -1.0, 2.0, 0.0, 0.0],
                  [1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0],
                  [3.0, -1.0, 2.0, 2.0, 0.0, 0.0, 0.0, 0.0]])
    idx, w, margin = o.topk(l, 2)
    assert idx.tolist() == [[1, 2], [0, 1], [0, 2]], idx.tolist()
    assert margin.tolist() == [0.0, 0.0, 0.0], margin.tolist()
    rng = _rng(7)
    l = rng.standard_normal((300, 8))
    for K in (1, 2, 3):
        _, _, margin = o.topk(l, K)
        s = -np.sort(-l, axis=1)
        assert np.array_equal(margin, s[:, K - 1] - s[:, K]), K


def pin_shift_invariance(o):
    """Adding one constant to every logit (through a constant input feature and
    a constant W_g row) changes neither the sets nor the weights."""
    rng = _rng(8)
    T, d = 64, 32
    x = _rand_f32(rng, (T, d))
    x[:, 0] = 1.0
    wg = _rand_f32(rng, (d, 8), 0.3)
    wg[0, :] = 0.0
    idx0, w0, _ = o.topk(o.logits(x, wg, "f32"), 2)
    wg[0, :] = 0.75
    idx1, w1, _ = o.topk(o.logits(x, wg, "f32"), 2)
    assert np.array_equal(idx0, idx1)
    assert np.max(np.abs(w0 - w1)) <= 1e-14


def pin_set_weights(o):
    """Weights of a given set are the masked softmax over that set."""
    rng = _rng(9)
    l = rng.standard_normal((50, 8))
    idx, w, _ = o.topk(l, 2)
    assert np.max(np.abs(o.set_weights(l, idx) - w)) <= 1e-16
    other = np.stack([idx[:, 1], (idx[:, 1] + 1) % 8], 1).astype(np.int32)
    other[other[:, 1] == idx[:, 0], 1] = (other[other[:, 1] == idx[:, 0], 1] + 1) % 8
    ws = o.set_weights(l, other)
    la = np.take_along_axis(l, other[:, :1].astype(np.int64), 1)[:, 0]
    lb = np.take_along_axis(l, other[:, 1:].astype(np.int64), 1)[:, 0]
    assert np.max(np.abs(ws[:, 0] - expit(la - lb))) <= 2e-16


# --- permute -----------------------------------------------------------------

def pin_permute_is_stable_sort(o):
    """Gathering tokens by expert (ml-canon page, Questions worth asking) as a
    stable sort of the T*K slots by expert id equals numpy's stable argsort;
    offsets are the cumulative counts; slot_pos inverts perm."""
    rng = _rng(10)
    for (T, E, K) in ((1, 8, 2), (97, 8, 2), (50, 3, 1), (64, 8, 8)):
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
        off, perm, slot = o.permute(idx, E)
        flat = idx.reshape(-1)
        order = np.argsort(flat, kind="stable")
        assert np.array_equal(perm, order // K), (T, E, K)
        inv = np.empty_like(order)
        inv[order] = np.arange(order.size)
        assert np.array_equal(slot.reshape(-1), inv)
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))


# --- expert FFN and the whole layer ---------------------------------------------

def _tiny_layer(rng, T, d, h, E, dt, std=0.5):
    mk = _rand_bf16 if dt == "bf16" else _rand_f32
    return {"x": mk(rng, (T, d)), "w_g": mk(rng, (d, E), std),
            "w1": mk(rng, (E, h, d), std), "w3": mk(rng, (E, h, d), std),
            "w2": mk(rng, (E, d, h), std)}


def _f64(inp, dt):
    return {k: to_float64(v, dt) for k, v in inp.items()}


def pin_gate_up_and_down_match_matmul(o):
    """The expert's two halves: act = silu(W1 x) * (W3 x), out = W2 act, against
    numpy matrix products with silu(z) = z * expit(z); non-square (d != h)."""
    rng = _rng(11)
    for dt in ("bf16", "f32"):
        n, d, h = 21, 48, 80
        mk = _rand_bf16 if dt == "bf16" else _rand_f32
        x, w1, w3, w2 = mk(rng, (n, d)), mk(rng, (h, d), .3), mk(rng, (h, d), .3), mk(rng, (d, h), .3)
        xf, w1f, w3f, w2f = (to_float64(a, dt) for a in (x, w1, w3, w2))
        g, u = xf @ w1f.T, xf @ w3f.T
        act_ref = g * expit(g) * u
        act = o.gate_up(x, w1, w3, dt)
        _close(act, act_ref, 1e-13, f"gate_up {dt}")
        act32 = act_ref.astype(np.float32)
        act_st = f32_to_bf16_bits(act32) if dt == "bf16" else act32
        _close(o.down(act_st, dt, w2, dt), to_float64(act_st, dt) @ w2f.T, 1e-13, f"down {dt}")


def pin_E1_K1_is_dense_swiglu(o):
    """E = 1, K = 1: the gate weight is exactly 1 and the layer is one dense
    SwiGLU FFN (numpy matrix products); d != h catches transposed operands."""
    rng = _rng(12)
    T, d, h = 9, 24, 40
    inp = _tiny_layer(rng, T, d, h, 1, "f32")
    res = o.forward(inp, 1, "f32")
    assert np.all(res["w"] == 1.0) and np.all(res["idx"] == 0)
    f = _f64(inp, "f32")
    _close(res["y"], ref_numpy.dense_swiglu(f["x"], f["w1"][0], f["w3"][0], f["w2"][0]), 1e-12,
           "E=1,K=1 vs dense SwiGLU")


def pin_identical_experts(o):
    """All experts identical: y equals that one expert's output for any router
    (the weights sum to 1)."""
    rng = _rng(13)
    T, d, h, E = 20, 32, 48, 8
    inp = _tiny_layer(rng, T, d, h, E, "bf16")
    for k in ("w1", "w3", "w2"):
        inp[k] = np.ascontiguousarray(np.broadcast_to(inp[k][:1], inp[k].shape))
    res = o.forward(inp, 2, "bf16")
    f = _f64(inp, "bf16")
    _close(res["y"], ref_numpy.dense_swiglu(f["x"], f["w1"][0], f["w3"][0], f["w2"][0]), 1e-13,
           "identical experts")


def pin_brute_force_dense_masked_sum(o):
    """Tiny inputs: the oracle's sparse evaluation equals the brute-force dense
    sum over all n experts with the masked gate (notion page, output equation
    y = sum_i G(x)_i E_i(x))."""
    rng = _rng(14)
    for (T, d, h, E, K, dt) in ((16, 32, 64, 8, 2, "f32"), (13, 16, 32, 5, 2, "bf16"),
                                (8, 32, 16, 4, 1, "f32")):
        inp = _tiny_layer(rng, T, d, h, E, dt)
        res = o.forward(inp, K, dt)
        f = _f64(inp, dt)
        _close(res["y"], ref_numpy.dense_moe(f["x"], f["w_g"], f["w1"], f["w3"], f["w2"], K),
               1e-13, f"brute force {T},{d},{h},{E},{K},{dt}")


def pin_blocked_equals_plain_per_token_loop(o):
    """The oracle evaluates experts over blocks of up to 16 rows that share each
    weight row; every sum still runs over its own index in ascending order, so
    its output must equal, bit for bit, a plain per-token evaluation of the
    output equation (notion page, y = sum_i G(x)_i SwiGLU_i(x) with K nonzero
    gates) written as scalar float64 loops here. Segments of 20-30 rows per
    expert span two blocks and a ragged one."""
    import math

    rng = _rng(16)
    for (T, d, h, E, K, dt) in ((40, 12, 20, 3, 2, "bf16"), (23, 8, 12, 2, 2, "f32"),
                                (35, 16, 8, 2, 1, "bf16")):
        inp = _tiny_layer(rng, T, d, h, E, dt)
        f = _f64(inp, dt)
        l, idx, w, _ = o.route(inp["x"], inp["w_g"], K, dt)
        y = o.forward_tokens(np.arange(T), inp["x"], inp["w1"], inp["w3"], inp["w2"], idx, w,
                             dt)
        x = f["x"].tolist()
        for t in range(T):
            acc = [0.0] * d
            for k in range(K):
                e = int(idx[t, k])
                w1, w3, w2 = f["w1"][e].tolist(), f["w3"][e].tolist(), f["w2"][e].tolist()
                a = []
                for j in range(h):
                    g = 0.0
                    u = 0.0
                    for i in range(d):
                        g += x[t][i] * w1[j][i]
                    for i in range(d):
                        u += x[t][i] * w3[j][i]
                    a.append(g / (1.0 + math.exp(-g)) * u)
                for c in range(d):
                    s = 0.0
                    for j in range(h):
                        s += w2[c][j] * a[j]
                    acc[c] += float(w[t, k]) * s
            assert np.array_equal(np.array(acc), y[t]), (T, d, h, E, K, dt, t)


def pin_hand_examples(o):
    """Hand-derived closed-form examples (tests/golden/hand_examples.json)."""
    with open(GOLDEN) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        inp = {k: np.array(c[k], dtype=np.float32) for k in ("x", "w_g", "w1", "w3", "w2")}
        res = o.forward(inp, c["K"], "f32")
        assert res["idx"].tolist() == c["idx"], (c["name"], res["idx"])
        assert np.max(np.abs(res["w"] - np.array(c["w"]))) <= 2e-16, c["name"]
        assert np.max(np.abs(res["y"] - np.array(c["y"]))) <= 1e-15, (c["name"], res["y"])


def pin_token_subset_consistent(o):
    """Evaluating a subset of tokens gives the same rows as evaluating all (the
    layer is per token: crackai page, routing is independent per token)."""
    rng = _rng(15)
    inp = _tiny_layer(rng, 40, 32, 48, 8, "bf16")
    full = o.forward(inp, 2, "bf16")
    sub = [39, 3, 17, 3]
    part = o.forward(inp, 2, "bf16", tokens=sub)
    assert np.array_equal(part["y"], full["y"][sub])


# --- capacity variant (a cap on the rows per expert) ------------------------------

def _brute_capped(idx, E, C):
    """Walk the slots in (token, k) order and keep one while its expert holds < C."""
    T, K = idx.shape
    held = [0] * E
    kept = []
    for s in range(T * K):
        e = int(idx.flat[s])
        if C <= 0 or held[e] < C:
            kept.append((e, s))
        held[e] += 1
    offsets = [0] * (E + 1)
    for e, _ in kept:
        offsets[e + 1] += 1
    for e in range(E):
        offsets[e + 1] += offsets[e]
    slot = [-1] * (T * K)
    perm = [-1] * (T * K)
    nxt = offsets[:E]
    for e, s in kept:  # kept in slot order, so each expert's rows are in slot order
        slot[s] = nxt[e]
        perm[nxt[e]] = s // K
        nxt[e] += 1
    return np.array(offsets), np.array(perm), np.array(slot).reshape(T, K)


def pin_capacity_permute_brute_force(o):
    """Capacity cap (ml-canon page, "Questions worth asking": a cap on the tokens per
    expert): the capped stable sort equals a slot-by-slot walk that keeps a slot while
    its expert holds fewer than C rows; a cap at least T (or 0) changes nothing."""
    rng = _rng(31)
    for (T, E, K) in ((50, 8, 2), (9, 3, 2), (17, 4, 1)):
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
        idx[: T // 3, 0] = 0  # crowd expert 0 so that caps bite
        for C in (1, 2, 3, 7, T, 0):
            off, perm, slot = o.permute_capped(idx, E, C)
            boff, bperm, bslot = _brute_capped(idx, E, C)
            assert np.array_equal(off, boff), (T, E, K, C)
            assert np.array_equal(slot, bslot), (T, E, K, C)
            assert np.array_equal(perm[: off[-1]], bperm[: off[-1]]), (T, E, K, C)
            assert np.all(np.diff(off) <= (C if C > 0 else T * K))
        off0, perm0, slot0 = o.permute(idx, E)
        offT, permT, slotT = o.permute_capped(idx, E, T)
        assert np.array_equal(off0, offT) and np.array_equal(perm0, permT) and \
            np.array_equal(slot0, slotT)


def pin_capacity_forward_drops_without_renormalising(o):
    """Under a cap, a token's output is the sum over its kept slots of w_k E_k(x):
    all kept = the uncapped output, one dropped = the other slot's weighted expert
    alone (brute force with numpy), both dropped = 0."""
    rng = _rng(32)
    T, d, h, E, K = 24, 16, 24, 4, 2
    inp = _tiny_layer(rng, T, d, h, E, "f32")
    inp["w_g"][:, 0] += np.float32(3.0) * np.abs(inp["x"]).mean()  # crowd expert 0
    full = o.forward(inp, K, "f32")
    capped = o.forward(inp, K, "f32", capacity=5)
    slot = capped["slot_pos"]
    x64 = _f64(inp, "f32")
    n_one = n_both = 0
    for t in range(T):
        kept = [k for k in range(K) if slot[t, k] >= 0]
        if len(kept) == K:
            assert np.array_equal(capped["y"][t], full["y"][t])
        elif not kept:
            assert np.all(capped["y"][t] == 0.0)
            n_both += 1
        else:
            k = kept[0]
            e = int(full["idx"][t, k])
            want = full["w"][t, k] * ref_numpy.dense_swiglu(
                x64["x"][t:t + 1], x64["w1"][e], x64["w3"][e], x64["w2"][e])[0]
            _close(capped["y"][t], want, 1e-12, f"token {t} with one dropped slot")
            n_one += 1
    assert n_one > 0, "the cap dropped no slot: the pin would test nothing"
    assert n_both >= 0


# --- pre-norm block (RMSNorm before the layer, residual after) ------------------

def pin_rmsnorm_matches_torch(o):
    """RMSNorm of the block input (ml-canon page "52 Mixtral", Connections: the
    LLaMA-like blocks use RMSNorm) equals torch's float64 rms_norm on exactly
    widened inputs, for bf16 and fp32 storage, with a large and a small eps."""
    import torch

    rng = _rng(21)
    for dt in ("bf16", "f32"):
        for eps in (1e-5, 0.5):
            if dt == "bf16":
                h, g = _rand_bf16(rng, (9, 96)), _rand_bf16(rng, (96,), 0.7)
            else:
                h, g = _rand_f32(rng, (9, 96)), _rand_f32(rng, (96,), 0.7)
            _, exact = o.rmsnorm(h, g, eps, dt)
            ref = torch.nn.functional.rms_norm(torch.from_numpy(to_float64(h, dt)), (96,),
                                               torch.from_numpy(to_float64(g, dt)), eps).numpy()
            _close(exact, ref, 1e-14, f"rmsnorm {dt} eps={eps}")


def pin_rmsnorm_closed_forms(o):
    """Closed forms: a constant row c gives g * c / sqrt(c^2 + eps); a one-hot row
    a * e_j gives g_j * a / sqrt(a^2 / d + eps) at j and 0 elsewhere; with g = 1 and
    eps = 0 every row has mean square 1; scaling a row by s > 0 (eps = 0) changes
    nothing; negating it negates the output."""
    rng = _rng(22)
    d = 64
    g = _rand_f32(rng, (d,), 1.0)
    for c, eps in ((3.0, 1.0), (-0.25, 0.0625)):
        h = np.full((1, d), c, dtype=np.float32)
        _, x = o.rmsnorm(h, g, eps, "f32")
        _close(x[0], g.astype(np.float64) * c / np.sqrt(c * c + eps), 1e-15, "constant row")
    h = np.zeros((1, d), dtype=np.float32)
    h[0, 5] = 2.0
    _, x = o.rmsnorm(h, g, 0.5, "f32")
    want = np.zeros(d)
    want[5] = float(g[5]) * 2.0 / np.sqrt(4.0 / d + 0.5)
    _close(x[0], want, 1e-15, "one-hot row")
    h = _rand_f32(rng, (7, d))
    _, x = o.rmsnorm(h, np.ones(d, dtype=np.float32), 0.0, "f32")
    assert np.max(np.abs(np.mean(x * x, axis=1) - 1.0)) < 1e-14, "unit mean square"
    _, xs = o.rmsnorm((h * np.float32(4.0)).astype(np.float32), g, 0.0, "f32")
    _, x1 = o.rmsnorm(h, g, 0.0, "f32")
    _close(xs, x1, 1e-15, "scale invariance")
    _, xn = o.rmsnorm(-h, g, 0.0, "f32")
    assert np.array_equal(xn, -x1), "sign symmetry"


def pin_round_bf16_nearest_even(o):
    """The once-rounded bf16 values: exact values stay, a tie between two bf16
    neighbours goes to the one with an even last bit, anything else to the nearer
    one (hand-derived bit patterns)."""
    cases = [(1.0, 0x3F80), (1.0 + 2.0 ** -8, 0x3F80), (1.0 + 3 * 2.0 ** -8, 0x3F82),
             (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81), (-(1.0 + 2.0 ** -8), 0xBF80),
             (3.0, 0x4040), (0.1, 0x3DCD), (-2.0 ** -10, 0xBA80), (0.0, 0x0000),
             (255.5, 0x4380), (65280.0 + 128.0, 0x4780), (65280.0 + 127.0, 0x477F)]
    got = o.round_bf16([c[0] for c in cases])
    for (v, want), gbits in zip(cases, got):
        assert int(gbits) == want, f"round_bf16({v!r}) = {int(gbits):#06x}, want {want:#06x}"
    # x stored in bf16 is the once-rounded exact value
    rng = _rng(23)
    h, g = _rand_bf16(rng, (3, 32)), _rand_bf16(rng, (32,))
    xb, exact = o.rmsnorm(h, g, 1e-5, "bf16")
    assert np.array_equal(xb, o.round_bf16(exact))


def pin_block_residual(o):
    """The pre-norm block returns its input plus the layer's output on the
    normalised input: with every W2 = 0 the layer adds nothing and the block is the
    identity; otherwise block - input equals the plain layer on x = RMSNorm(h)."""
    rng = _rng(24)
    inp = _tiny_layer(rng, 12, 32, 48, 8, "bf16")
    inp["h"] = _rand_bf16(rng, (12, 32), 2.0)
    inp["norm_w"] = _rand_bf16(rng, (32,), 0.5)
    zero = dict(inp, w2=np.zeros_like(inp["w2"]))
    out = o.block_forward(zero, 2, "bf16", 1e-5)
    assert np.array_equal(out["y"], to_float64(inp["h"], "bf16"))
    out = o.block_forward(inp, 2, "bf16", 1e-5)
    plain = o.forward(dict(inp, x=out["x"]), 2, "bf16")
    assert np.array_equal(out["y"], to_float64(inp["h"], "bf16") + plain["y"])
    assert np.array_equal(out["idx"], plain["idx"])


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
