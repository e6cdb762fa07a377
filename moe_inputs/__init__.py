"""Seeded synthetic inputs for the Mixtral sparse-MoE feed-forward layer.

This module is shared by the CPU oracle, the tests and the benchmark. It holds
random draws, scaling, the per-row normalisation that stands in for the RMSNorm
that precedes the layer in the Mistral-7B block, float32 -> bfloat16 rounding and
the workload table. It holds none of the layer's own arithmetic (no router,
top-k, softmax, SwiGLU or combine).

Shapes follow the problem statement on the pages (Mixtral of Experts, "Top-2
Routing in Detail" and the sparse-gating equation): tokens x [T, d], router
W_g [d, E] so that x . W_g is [T, E], expert matrices in column-vector form
W1, W3 [E, h, d] and W2 [E, d, h].

bfloat16 arrays are returned as ``np.uint16`` bit patterns; float32 arrays as
``np.float32``.
"""
from __future__ import annotations

import hashlib
import json
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

GENERATOR_VERSION = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
ZIPF_BIAS_FILE = os.path.join(_HERE, "zipf_bias.json")


@dataclass(frozen=True)
class Config:
    """One synthetic workload.

    x_kind: "normal" (iid N(0,1)) or "rmsnorm" (iid N(0,1) rows scaled to unit
    root-mean-square, the output of an RMSNorm without gain).
    *_std: standard deviations; the strings "fan_in_d" / "fan_in_h" mean
    d**-0.5 / h**-0.5 (variance 1/d or 1/h).
    zipf_bias: add the constant feature x[:, 0] = 1 and put a per-expert bias
    into W_g[0, :] so that expert popularity follows a Zipf law.
    """

    name: str
    T: int
    d: int
    h: int
    E: int = 8
    K: int = 2
    dtype: str = "bf16"  # "bf16" or "f32"
    x_kind: str = "normal"
    wg_std: object = "fan_in_d"
    w13_std: object = 0.02
    w2_std: object = 0.02
    zipf_bias: bool = False

    def std(self, which: str) -> float:
        v = {"wg": self.wg_std, "w13": self.w13_std, "w2": self.w2_std}[which]
        if v == "fan_in_d":
            return float(self.d) ** -0.5
        if v == "fan_in_h":
            return float(self.h) ** -0.5
        return float(v)

    @property
    def S(self) -> int:
        return self.T * self.K

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The five workloads. Mixtral-8x7B layer shape: d = 32 heads x 128 = 4096,
# expert inner dim 14336 (atlas page, "Design overview"); 8x22B shape
# d = 6144, h = 16384.
CONFIGS: Dict[str, Config] = {
    "tiny_f32": Config("tiny_f32", T=64, d=128, h=256, dtype="f32",
                       x_kind="normal", wg_std="fan_in_d", w13_std="fan_in_d",
                       w2_std="fan_in_h"),
    "decode_8x7b": Config("decode_8x7b", T=32, d=4096, h=14336,
                          x_kind="rmsnorm", wg_std=0.02),
    "prefill_8x7b": Config("prefill_8x7b", T=4096, d=4096, h=14336,
                           x_kind="rmsnorm", wg_std="fan_in_d"),
    "skew_8x7b": Config("skew_8x7b", T=16384, d=4096, h=14336,
                        x_kind="rmsnorm", wg_std="fan_in_d", zipf_bias=True),
    "prefill_8x22b": Config("prefill_8x22b", T=8192, d=6144, h=16384,
                            x_kind="normal", wg_std="fan_in_d"),
}

# Zipf(s = 1.2) popularity over the 8 experts, expert e has rank e + 1.
ZIPF_S = 1.2


def zipf_shares(E: int = 8, s: float = ZIPF_S) -> np.ndarray:
    r = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    return r / r.sum()


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); finite input."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else a32


def _normal(child: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(child))
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def load_zipf_bias(E: int = 8) -> np.ndarray:
    """Per-expert router bias (float32 values) for the Zipf workload."""
    with open(ZIPF_BIAS_FILE) as f:
        rec = json.load(f)
    b = np.array(rec["bias_f32"], dtype=np.float32)
    if b.shape != (E,):
        raise ValueError(f"zipf bias file has {b.shape[0]} experts, need {E}")
    return b


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_x(cfg: Config, seed: int = 0) -> np.ndarray:
    kids = np.random.SeedSequence(seed).spawn(2 + 3 * cfg.E)
    return _make_x(cfg, kids[0])


def _make_x(cfg: Config, child) -> np.ndarray:
    x = _normal(child, (cfg.T, cfg.d), 1.0)
    if cfg.x_kind == "rmsnorm":
        x64 = x.astype(np.float64)
        x64 /= np.sqrt(np.mean(x64 * x64, axis=1, keepdims=True) + 1e-6)
        x = x64.astype(np.float32)
    elif cfg.x_kind != "normal":
        raise ValueError(cfg.x_kind)
    if cfg.zipf_bias:
        x[:, 0] = 1.0  # constant feature; exact in bf16
    return _store(x, cfg.dtype)


def make_router(cfg: Config, seed: int = 0) -> np.ndarray:
    kids = np.random.SeedSequence(seed).spawn(2 + 3 * cfg.E)
    return _make_router(cfg, kids[1])


def _make_router(cfg: Config, child) -> np.ndarray:
    wg = _normal(child, (cfg.d, cfg.E), cfg.std("wg"))
    if cfg.zipf_bias:
        wg[0, :] = load_zipf_bias(cfg.E)
    return _store(wg, cfg.dtype)


def make_inputs(cfg: Config, seed: int = 0, experts: bool = True) -> Dict[str, np.ndarray]:
    """All inputs of one layer call.

    Streams: SeedSequence(seed).spawn(2 + 3E) in the order x, W_g, then for
    each expert e: W1[e], W3[e], W2[e]. Each draw is float32 standard normal
    times the configured std, then stored as bf16 (RNE) or float32.
    """
    kids = np.random.SeedSequence(seed).spawn(2 + 3 * cfg.E)
    out = {"x": _make_x(cfg, kids[0]), "w_g": _make_router(cfg, kids[1])}
    if not experts:
        return out
    st = np.uint16 if cfg.dtype == "bf16" else np.float32
    w1 = np.empty((cfg.E, cfg.h, cfg.d), dtype=st)
    w3 = np.empty((cfg.E, cfg.h, cfg.d), dtype=st)
    w2 = np.empty((cfg.E, cfg.d, cfg.h), dtype=st)
    jobs = []
    for e in range(cfg.E):
        jobs.append((w1, e, kids[2 + 3 * e], (cfg.h, cfg.d), cfg.std("w13")))
        jobs.append((w3, e, kids[3 + 3 * e], (cfg.h, cfg.d), cfg.std("w13")))
        jobs.append((w2, e, kids[4 + 3 * e], (cfg.d, cfg.h), cfg.std("w2")))

    def run(job):
        dst, e, child, shape, std = job
        dst[e] = _store(_normal(child, shape, std), cfg.dtype)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, jobs))
    out.update(w1=w1, w3=w3, w2=w2)
    return out


def make_act(n: int, h: int, dtype: str, seed: int = 0, std: float = 1.0) -> np.ndarray:
    """Synthetic hidden activations [n, h] for exercising the down projection alone."""
    child = np.random.SeedSequence([seed, 0xAC7]).spawn(1)[0]
    return _store(_normal(child, (n, h), std), dtype)


def make_block(cfg: Config, seed: int = 0, h_std: float = 2.0,
               w_std: float = 0.1) -> Dict[str, np.ndarray]:
    """Inputs of a pre-norm block around the layer: the block input h [T, d]
    (standard normal times h_std) and the norm gain norm_w [d] (1 + standard
    normal times w_std), stored in cfg.dtype. Streams SeedSequence([seed, 0xB10C])."""
    kids = np.random.SeedSequence([seed, 0xB10C]).spawn(2)
    h = _normal(kids[0], (cfg.T, cfg.d), h_std)
    g = (1.0 + _normal(kids[1], (cfg.d,), w_std)).astype(np.float32)
    return {"h": _store(h, cfg.dtype), "norm_w": _store(g, cfg.dtype)}


def make_routing(T: int, E: int, K: int, seed: int = 0) -> np.ndarray:
    """Random distinct expert ids per token, [T, K] int32 (for the permute alone)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x9E7])))
    keys = g.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :K].astype(np.int32)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def fingerprint(inputs: Dict[str, np.ndarray]) -> Dict[str, str]:
    return {k: sha256(v) for k, v in sorted(inputs.items())}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg
