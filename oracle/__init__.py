"""CPU oracle for the Mixtral sparse-MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does. It shares
no code with the GPU implementation.

``moe_oracle.c`` holds the arithmetic (float64, ascending-order sums, OpenMP over
rows); this module builds it with gcc and wraps it with ctypes. ``ref_numpy``
holds second formulations of the same layer used only to pin the C code.

Pins (tests/test_oracle_pins.py) check every function here against something
other than itself: library routines, closed forms, invariants and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "moe_oracle.c")
LIBRARY = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16 = 0, 1
_DT = {"f32": F32, "bf16": BF16}


def build(out: str = LIBRARY, mutant: Optional[int] = None, cc: str = "gcc") -> str:
    """Compile the oracle (plain C, no fast-math, no FMA contraction).

    -O3 without loop vectorisation: the 16 rows of a block that share a weight
    row are accumulated side by side in vector registers (each row's sum keeps
    its own ascending order, so the results are those of a scalar build bit for
    bit); vectorising the loop over the summation index instead would only
    shuffle registers."""
    cmd = [cc, "-std=c11", "-O3", "-fno-tree-loop-vectorize", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-o", out + ".tmp", SOURCE, "-lm"]
    if mutant is not None:
        cmd.insert(1, f"-DORACLE_MUTANT={int(mutant)}")
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes handle on one build of moe_oracle.c."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build(path)
        self.path = path
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.oracle_logits.argtypes = [i64, i64, i32, i32, vp, vp, vp]
        lib.oracle_topk.argtypes = [i64, i32, i32, vp, vp, vp, vp]
        lib.oracle_set_weights.argtypes = [i64, i32, i32, vp, vp, vp]
        lib.oracle_permute.argtypes = [i64, i32, i32, vp, vp, vp, vp]
        lib.oracle_gate_up.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp]
        lib.oracle_down.argtypes = [i64, i64, i64, i32, vp, i32, vp, vp]
        lib.oracle_forward_tokens.argtypes = [i64, vp, i64, i64, i32, i32, i32,
                                              vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_permute_capped.argtypes = [i64, i32, i32, vp, i64, vp, vp, vp]
        lib.oracle_permute_capped.restype = None
        lib.oracle_capped_weights.argtypes = [i64, i32, vp, vp, vp]
        lib.oracle_capped_weights.restype = None
        lib.oracle_rmsnorm.argtypes = [i64, i64, i32, vp, vp, ctypes.c_double, vp, vp]
        lib.oracle_rmsnorm.restype = None
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        for f in (lib.oracle_logits, lib.oracle_topk, lib.oracle_set_weights,
                  lib.oracle_permute, lib.oracle_gate_up, lib.oracle_down,
                  lib.oracle_forward_tokens):
            f.restype = None
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_mutant.restype = ctypes.c_int
        self.lib = lib

    @property
    def threads(self) -> int:
        return int(self.lib.oracle_threads())

    @property
    def mutant(self) -> int:
        return int(self.lib.oracle_mutant())

    # -- router -----------------------------------------------------------
    def logits(self, x: np.ndarray, w_g: np.ndarray, dtype: str) -> np.ndarray:
        x = np.ascontiguousarray(x)
        w_g = np.ascontiguousarray(w_g)
        T, d = x.shape
        E = w_g.shape[1]
        assert w_g.shape[0] == d
        out = np.empty((T, E), dtype=np.float64)
        self.lib.oracle_logits(T, d, E, _DT[dtype], _p(x), _p(w_g), _p(out))
        return out

    def topk(self, logits: np.ndarray, K: int):
        """(idx [T,K] int32, w [T,K] float64, margin [T] float64)."""
        logits = np.ascontiguousarray(logits, dtype=np.float64)
        T, E = logits.shape
        idx = np.empty((T, K), dtype=np.int32)
        w = np.empty((T, K), dtype=np.float64)
        margin = np.empty((T,), dtype=np.float64)
        self.lib.oracle_topk(T, E, K, _p(logits), _p(idx), _p(w), _p(margin))
        return idx, w, margin

    def set_weights(self, logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
        logits = np.ascontiguousarray(logits, dtype=np.float64)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        T, E = logits.shape
        K = idx.shape[1]
        w = np.empty((T, K), dtype=np.float64)
        self.lib.oracle_set_weights(T, E, K, _p(logits), _p(idx), _p(w))
        return w

    def route(self, x, w_g, K: int, dtype: str):
        l = self.logits(x, w_g, dtype)
        idx, w, margin = self.topk(l, K)
        return l, idx, w, margin

    # -- permute ----------------------------------------------------------
    def permute(self, idx: np.ndarray, E: int):
        """(offsets [E+1], perm_token [S], slot_pos [T,K]) of the stable sort by expert."""
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        T, K = idx.shape
        offsets = np.empty((E + 1,), dtype=np.int32)
        perm = np.empty((T * K,), dtype=np.int32)
        slot = np.empty((T, K), dtype=np.int32)
        self.lib.oracle_permute(T, E, K, _p(idx), _p(offsets), _p(perm), _p(slot))
        return offsets, perm, slot

    def permute_capped(self, idx: np.ndarray, E: int, capacity: int):
        """permute() with at most `capacity` rows per expert (earliest slots kept;
        dropped slots get slot_pos -1); capacity <= 0 means no cap."""
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        T, K = idx.shape
        offsets = np.empty((E + 1,), dtype=np.int32)
        perm = np.full((T * K,), -1, dtype=np.int32)
        slot = np.empty((T, K), dtype=np.int32)
        self.lib.oracle_permute_capped(T, E, K, _p(idx), int(capacity), _p(offsets), _p(perm),
                                       _p(slot))
        return offsets, perm, slot

    def capped_weights(self, slot_pos: np.ndarray, w: np.ndarray) -> np.ndarray:
        slot_pos = np.ascontiguousarray(slot_pos, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float64)
        T, K = w.shape
        out = np.empty_like(w)
        self.lib.oracle_capped_weights(T, K, _p(slot_pos), _p(w), _p(out))
        return out

    # -- expert FFN ---------------------------------------------------------
    def gate_up(self, xrows, w1e, w3e, dtype: str) -> np.ndarray:
        xrows = np.ascontiguousarray(xrows)
        n, d = xrows.shape
        h = w1e.shape[0]
        assert w1e.shape == (h, d) and w3e.shape == (h, d)
        act = np.empty((n, h), dtype=np.float64)
        self.lib.oracle_gate_up(n, d, h, _DT[dtype], _p(xrows),
                                _p(np.ascontiguousarray(w1e)), _p(np.ascontiguousarray(w3e)),
                                _p(act))
        return act

    def down(self, act, act_dtype: str, w2e, dtype: str) -> np.ndarray:
        act = np.ascontiguousarray(act)
        n, h = act.shape
        d = w2e.shape[0]
        assert w2e.shape == (d, h)
        out = np.empty((n, d), dtype=np.float64)
        self.lib.oracle_down(n, d, h, _DT[act_dtype], _p(act), _DT[dtype],
                             _p(np.ascontiguousarray(w2e)), _p(out))
        return out

    def forward_tokens(self, tokens: Sequence[int], x, w1, w3, w2, idx, w, dtype: str) -> np.ndarray:
        """y rows for the listed tokens with the given expert sets and weights."""
        tokens = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        x = np.ascontiguousarray(x)
        T, d = x.shape
        E, h, _ = w1.shape
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float64)
        K = idx.shape[1]
        assert idx.shape == (T, K) and w.shape == (T, K)
        assert w1.shape == (E, h, d) and w3.shape == (E, h, d) and w2.shape == (E, d, h)
        y = np.empty((len(tokens), d), dtype=np.float64)
        self.lib.oracle_forward_tokens(len(tokens), _p(tokens), d, h, E, K, _DT[dtype],
                                       _p(x), _p(np.ascontiguousarray(w1)),
                                       _p(np.ascontiguousarray(w3)),
                                       _p(np.ascontiguousarray(w2)), _p(idx), _p(w), _p(y))
        return y

    # -- pre-norm block -----------------------------------------------------
    def round_bf16(self, values) -> np.ndarray:
        """bf16 bit patterns of doubles rounded once (to nearest, ties to even)."""
        v = np.asarray(values, dtype=np.float64).ravel()
        return np.array([self.lib.oracle_round_bf16(float(a)) for a in v],
                        dtype=np.uint16).reshape(np.shape(values))

    def rmsnorm(self, h, g, eps: float, dtype: str):
        """(x in dtype storage [T, d], x_exact float64 [T, d]) of the block input h."""
        h = np.ascontiguousarray(h)
        g = np.ascontiguousarray(g)
        T, d = h.shape
        assert g.shape == (d,) and g.dtype == h.dtype
        exact = np.empty((T, d), dtype=np.float64)
        out = np.empty((T, d), dtype=h.dtype)
        self.lib.oracle_rmsnorm(T, d, _DT[dtype], _p(h), _p(g), float(eps), _p(exact), _p(out))
        return out, exact

    def block_forward(self, inputs, K: int, dtype: str, eps: float,
                      tokens: Optional[Sequence[int]] = None):
        """Pre-norm block h + y(RMSNorm(h) g): inputs hold h (block input) and norm_w
        beside the layer's weights. Returns dict(y, x, logits, idx, w, margin, tokens)."""
        x, _ = self.rmsnorm(inputs["h"], inputs["norm_w"], eps, dtype)
        out = self.forward(dict(inputs, x=x), K, dtype, tokens)
        hrows = np.stack([_widen(inputs["h"][t], dtype) for t in out["tokens"]]) \
            if len(out["tokens"]) else np.zeros((0, x.shape[1]))
        out["y"] = hrows + out["y"]
        out["x"] = x
        return out

    def forward(self, inputs, K: int, dtype: str, tokens: Optional[Sequence[int]] = None,
                capacity: int = 0):
        """Whole layer: returns dict(y, logits, idx, w, margin, tokens[, slot_pos]) (y for
        `tokens` or all). capacity > 0 caps the rows per expert (capacity variant)."""
        l, idx, w, margin = self.route(inputs["x"], inputs["w_g"], K, dtype)
        T = inputs["x"].shape[0]
        toks = np.arange(T) if tokens is None else np.asarray(tokens)
        out = {"logits": l, "idx": idx, "w": w, "margin": margin, "tokens": toks}
        w_eff = w
        if capacity > 0:
            E = inputs["w1"].shape[0]
            _, _, slot = self.permute_capped(idx, E, capacity)
            w_eff = self.capped_weights(slot, w)
            out["slot_pos"] = slot
        out["y"] = self.forward_tokens(toks, inputs["x"], inputs["w1"], inputs["w3"],
                                       inputs["w2"], idx, w_eff, dtype)
        return out


def _widen(row, dtype: str) -> np.ndarray:
    """Stored values (bf16 bits or float32) as float64, exactly."""
    if dtype == "bf16":
        return (np.asarray(row, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32) \
            .astype(np.float64)
    return np.asarray(row, dtype=np.float32).astype(np.float64)


_DEFAULT: Optional[Oracle] = None


def load() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
