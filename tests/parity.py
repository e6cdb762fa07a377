"""Helpers shared by the GPU parity tests, the smoke check and the benchmark's
parity leg: host<->device marshalling of the generator's arrays and the
comparison rules.

Comparison rules
* Expert sets (rule R): for every token whose oracle 2nd-to-3rd logit margin
  exceeds 1e-3 the GPU's set must equal the oracle's. A token at or below that
  margin may get another set, but only a valid one: K distinct experts, every
  chosen logit >= every unchosen logit - 1e-3 (oracle logits). For such tokens
  the reference output is re-evaluated with the GPU's set.
* Gate weights: |w_gpu - w_ref(set)| <= 1e-5 (set = the GPU's set).
* Layer output: max |y_gpu - y_ref| <= tol * RMS(y_ref) with tol = 2e-2 for bf16
  inputs (float32 accumulation) and 1e-5 for float32 inputs; RMS over all the
  compared entries of y_ref.
"""
from __future__ import annotations

import numpy as np

MARGIN = 1e-3
W_TOL = 1e-5
Y_TOL = {"bf16": 2e-2, "f32": 1e-5}


def device_array(a: np.ndarray, dtype: str, device="cuda"):
    import torch

    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)
    if dtype == "i32":
        return torch.from_numpy(a.astype(np.int32, copy=False)).to(device)
    raise ValueError(dtype)


def host_array(t) -> np.ndarray:
    """bf16 tensors come back as uint16 bit patterns, others as numpy."""
    import torch

    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def upload_inputs(inp: dict, dtype: str, device="cuda") -> dict:
    return {k: device_array(v, dtype, device) for k, v in inp.items()}


def check_routing(idx_gpu, w_gpu, logits_ref, idx_ref, margin, K, oracle, tie_margin=None,
                  w_tol=None):
    """Apply rule R; returns (expert sets to evaluate the reference with, the
    tokens whose set differs from the oracle's)."""
    idx_gpu = np.asarray(idx_gpu)
    T, E = logits_ref.shape
    assert idx_gpu.shape == (T, K)
    assert idx_gpu.min() >= 0 and idx_gpu.max() < E, "expert id out of range"
    sg = np.sort(idx_gpu, 1)
    sr = np.sort(idx_ref, 1)
    diff = np.where(np.any(sg != sr, axis=1))[0]
    tie_margin = MARGIN if tie_margin is None else tie_margin
    w_tol = W_TOL if w_tol is None else w_tol
    strict = diff[margin[diff] > tie_margin]
    assert strict.size == 0, (
        f"{strict.size} tokens with margin > {tie_margin} got another expert set, e.g. token "
        f"{strict[0]}: gpu {idx_gpu[strict[0]].tolist()} oracle {idx_ref[strict[0]].tolist()} "
        f"margin {margin[strict[0]]:.3e}")
    for t in diff:
        chosen = set(idx_gpu[t].tolist())
        assert len(chosen) == K, f"token {t}: repeated expert {idx_gpu[t].tolist()}"
        lo = min(logits_ref[t, e] for e in chosen)
        hi = max((logits_ref[t, e] for e in range(E) if e not in chosen), default=-np.inf)
        assert lo >= hi - tie_margin, f"token {t}: invalid near-tie choice {idx_gpu[t].tolist()}"
    assert np.all(sg[:, 1:] != sg[:, :-1]) if K > 1 else True, "repeated expert in a set"
    idx_eval = np.array(idx_ref, dtype=np.int32, copy=True)
    idx_eval[diff] = idx_gpu[diff]
    w_ref = oracle.set_weights(logits_ref, idx_gpu.astype(np.int32))
    werr = np.max(np.abs(np.asarray(w_gpu, dtype=np.float64) - w_ref))
    assert werr <= w_tol, f"gate weights differ by {werr:.3e} > {w_tol}"
    return idx_eval, diff


def check_output(y_gpu, y_ref, dtype: str, what: str = "y"):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(y_ref * y_ref)))
    err = float(np.max(np.abs(y_gpu - y_ref)))
    rel = err / rms if rms > 0 else err
    assert rel <= Y_TOL[dtype], f"{what}: max|err| = {err:.4e} = {rel:.3e} x RMS > {Y_TOL[dtype]}"
    return rel


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    """A seeded sample of n tokens that always includes the first and last ones."""
    if n >= T:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    pick = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], pick])).astype(np.int64)
