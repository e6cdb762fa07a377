"""Calibrate the per-expert router bias of the skewed-routing workload.

Writes ``moe_inputs/zipf_bias.json``. The workload is the Mixtral-8x7B layer at
T = 16384 with expert popularity following Zipf(s = 1.2) over the 8 experts
(expert e has rank e + 1, so expert 0 takes about 43% of the slot assignments).

The router has no bias term (notion page, sparse-gating equation), so the bias
enters as a constant input feature: x[:, 0] = 1 and W_g[0, e] = b_e, which keeps
the logits exactly x . W_g. The bias is found by the fixed-point iteration
b <- b + 0.5 (ln p - ln share), 200 steps from b = 0, where ``share`` is the
fraction of top-2 slots each expert receives under the oracle's routing on the
workload's own x; b is then rounded to bf16 and the achieved shares recomputed
with that rounded bias.

Uses only the oracle and the seeded input generator.
Run:  python -m oracle.calibrate_zipf
"""
from __future__ import annotations

import json
import sys

import numpy as np

import moe_inputs
from oracle import load


def calibrate(iters: int = 200, seed: int = 0):
    o = load()
    cfg = moe_inputs.CONFIGS["skew_8x7b"]
    x = moe_inputs.make_x(cfg, seed)
    wg = moe_inputs.make_router(cfg.with_(zipf_bias=False), seed)
    wg[0, :] = 0  # bf16 +0.0; x[:, 0] is already the constant 1
    base = o.logits(x, wg, cfg.dtype)
    p = moe_inputs.zipf_shares(cfg.E)

    def shares(logits):
        idx, _, _ = o.topk(logits, cfg.K)
        return np.bincount(idx.reshape(-1), minlength=cfg.E) / idx.size

    b = np.zeros(cfg.E)
    for _ in range(iters):
        s = shares(base + b)
        b = b + 0.5 * (np.log(p) - np.log(np.maximum(s, 1e-12)))
        b -= b.mean()
    b32 = b.astype(np.float32)
    bits = moe_inputs.f32_to_bf16_bits(b32)
    b_bf16 = moe_inputs.bf16_bits_to_f32(bits)
    wg[0, :] = bits
    final = shares(o.logits(x, wg, cfg.dtype))
    return {
        "about": "Router bias for the Zipf(1.2) skewed-routing workload (T=16384, "
                 "d=4096, E=8, K=2, seed 0); realised as x[:,0]=1 and W_g[0,e]=b_e. "
                 "Written by oracle/calibrate_zipf.py.",
        "generator_version": moe_inputs.GENERATOR_VERSION,
        "seed": seed,
        "target_shares": p.tolist(),
        "bias_f32": [float(v) for v in b_bf16],
        "bias_bf16_bits": [int(v) for v in bits],
        "achieved_shares": final.tolist(),
        "max_share_error": float(np.max(np.abs(final - p))),
    }


def main(argv=None):
    rec = calibrate()
    with open(moe_inputs.ZIPF_BIAS_FILE, "w") as f:
        json.dump(rec, f, indent=2)
        f.write("\n")
    print(json.dumps({k: rec[k] for k in ("bias_f32", "achieved_shares", "max_share_error")}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
