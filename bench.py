"""Benchmark of the Mixtral sparse-MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one pass of the whole layer (route -> permute -> gate-up -> down ->
combine) over one batch of the workload's synthetic inputs, already resident in
HBM. The default workload is the Mixtral-8x7B decode batch (T = 32 tokens,
d = 4096, h = 14336, E = 8, K = 2, bf16), whose expert weights (2.82 GB) must be
streamed from HBM every step; other workloads: prefill_8x7b, skew_8x7b,
prefill_8x22b, tiny_f32.

Printed: ONE JSON line with tokens/s, the dominant kernel's roofline fraction
(HIP events around that kernel inside the timed region) and the CPU oracle
timed on a bounded sample of the same workload. The workloads named by --also
(default: the 8x7B prefill batch, T = 4096, whose expert GEMMs are bound by the
matrix cores rather than by HBM) are measured the same way in the same run and
reported under "sub_workloads" of that line, each after at least SUB_MIN_WARMUP
warm-up steps: the GPU sits idle while the CPU baseline of the workload before it
runs, and 5 warm-up steps left its clock still rising (prefill_8x7b gate-up 1.569 ms
per launch in the timed steps against 1.515 ms in the stage pass right after).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s on 1 MI355X; % bf16 MFMA peak (prefill), % HBM BW (decode)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
MFMA_F32_PEAK_TFLOPS = 157.3    # fp32 vector/matrix peak (fp32 problems)
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sparse_mixture_experts_wg_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_8x7b")
    ap.add_argument("--also", default="prefill_8x7b",
                    help="comma-separated workloads measured after the headline one in the same "
                         "run and reported as sub-records of its JSON line ('' for none)")
    ap.add_argument("--weight-copies", type=int, default=2,
                    help="rotate this many copies of the expert weights so that no step "
                         "finds them in the 256 MB last-level cache")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate budget of the CPU-oracle baseline leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", default="auto", choices=["auto", "stream", "tiled"])
    ap.add_argument("--capacity-factor", type=float, default=0.0,
                    help="capacity variant: cap every expert at ceil(cf*T*K/E) rows (0: no cap)")
    ap.add_argument("--block", action="store_true",
                    help="time the pre-norm block instead of the bare layer: RMSNorm of the "
                         "block input before routing, the residual added in the combine")
    ap.add_argument("--sweep", default="",
                    help="comma-separated batch sizes T: time moe_forward on both expert paths "
                         "at each T with the workload's d, h and distributions (prints one JSON "
                         "line with the table instead of the bench line)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the vendor GEMM library (torch.matmul, bf16) on the expert "
                         "projections' shapes of the workload, dense over all S = T*K rows and on "
                         "one expert's even share: the reference point for the tiled kernels")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (steps "
                         "times): the reference kernel for scaling HBM byte counters")
    return ap.parse_args()


def copy_probe(mib: int, steps: int):
    import torch

    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_probe_mib": mib, "read_bytes": n * 4, "write_bytes": n * 4,
                      "ms_per_copy": round(dt * 1e3, 4),
                      "GBps_read_plus_write": round(2 * n * 4 / dt / 1e9, 1)}), flush=True)
    return 0


def vendor_gemm(args):
    """torch.matmul (the vendor GEMM library) on the workload's projection shapes:
    gate-up [rows, d] x [d, 2h] and down [rows, h] x [h, d], for rows = S (the whole
    routed batch as one dense GEMM) and rows = S / E (one expert's even share)."""
    import torch

    import moe_inputs as mi

    cfg = mi.CONFIGS[args.workload]
    S, d, h, E = cfg.S, cfg.d, cfg.h, cfg.E
    g = torch.Generator(device="cuda").manual_seed(0)
    rows_out = []
    for name, M, K, N in (("gate_up_dense", S, d, 2 * h), ("gate_up_one_expert", S // E, d, 2 * h),
                          ("down_dense", S, h, d), ("down_one_expert", S // E, h, d)):
        a = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        b = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        for _ in range(3):
            a @ b.t()
        torch.cuda.synchronize()
        n = max(5, min(args.steps, 50))
        t0 = time.perf_counter()
        for _ in range(n):
            a @ b.t()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / n
        tf = 2.0 * M * N * K / (ms / 1e3) / 1e12
        rows_out.append({"gemm": name, "M": M, "K": K, "N": N, "ms": round(ms, 4),
                         "TFLOP/s": round(tf, 1), "frac_of_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        print(f"# {name}: {M} x {K} x {N}: {ms:.3f} ms, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del a, b
    print(json.dumps({"vendor_gemm": cfg.name, "rows": rows_out}), flush=True)
    return 0


def sweep(args):
    """Tokens/s of the whole layer (one moe_forward call per step) against the batch
    size, for the streaming and the tiled expert path and for the automatic choice."""
    import numpy as np
    import torch

    import moe_inputs as mi
    import sparse_mixture_experts_wg_amd as moe
    from tests import parity

    Ts = sorted({int(t) for t in args.sweep.split(",") if t.strip()})
    base = mi.CONFIGS[args.workload]
    cfg = base.with_(name=f"{base.name}_sweep", T=max(Ts))
    print(f"# sweep over T={Ts} with d={cfg.d} h={cfg.h} E={cfg.E} K={cfg.K} {cfg.dtype}",
          file=sys.stderr, flush=True)
    inp = mi.make_inputs(cfg, seed=0)
    copies = max(1, args.weight_copies)
    wsets = [{k: parity.device_array(inp[k], cfg.dtype) for k in ("w1", "w3", "w2")}
             for _ in range(copies)]
    w_g = parity.device_array(inp["w_g"], cfg.dtype)
    rows = []
    for T in Ts:
        x = parity.device_array(np.ascontiguousarray(inp["x"][:T]), cfg.dtype)
        y = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
        row = {"T": T}
        for path in ("stream", "tiled", "auto"):
            p = moe.problem(T, cfg.d, cfg.h, cfg.E, cfg.K, cfg.dtype, "f32", path)
            if path == "auto":
                row["auto"] = "stream" if moe.resolve_path(p) == moe.PATH_STREAM else "tiled"
                continue
            wsb = torch.empty((moe.forward_workspace_bytes(p),), dtype=torch.uint8, device="cuda")
            for i in range(3):
                ws = wsets[i % copies]
                moe.forward(p, x, w_g, ws["w1"], ws["w3"], ws["w2"], y, ws=wsb)
            torch.cuda.synchronize()
            n = max(5, min(args.steps, 40))
            t0 = time.perf_counter()
            for i in range(n):
                ws = wsets[i % copies]
                moe.forward(p, x, w_g, ws["w1"], ws["w3"], ws["w2"], y, ws=wsb)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / n
            row[f"{path}_ms"] = round(ms, 4)
            row[f"{path}_tokens_per_s"] = round(T / (ms / 1e3), 1)
        row["best"] = "stream" if row["stream_ms"] <= row["tiled_ms"] else "tiled"
        print(f"# T={T:5d} stream {row['stream_ms']:8.3f} ms  tiled {row['tiled_ms']:8.3f} ms  "
              f"auto={row['auto']}", file=sys.stderr, flush=True)
        rows.append(row)
    print(json.dumps({"sweep": cfg.name, "d": cfg.d, "h": cfg.h, "E": cfg.E, "K": cfg.K,
                      "dtype": cfg.dtype, "weight_copies": copies, "rows": rows}), flush=True)
    return 0


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# the dominant kernel is bracketed by HIP events on every GU_EVERY-th timed step
GU_EVERY = 8


def kernel_files(path: str):
    return ["gemm_stream.hip"] if path == "stream" else ["gemm_tiled.hip"]


def load_traffic(workload: str, kernel: str, sha: str):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3
    counter runs, if they were taken on the current kernel source."""
    f = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != sha:
        return None
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this layer has no "
              "multi-GPU path", file=sys.stderr)
        return 2

    if args.copy_probe_mib:
        return copy_probe(args.copy_probe_mib, max(1, args.steps))
    if args.sweep:
        return sweep(args)
    if args.vendor_gemm:
        return vendor_gemm(args)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    out = measure(args.workload, args, args.cpu_seconds)
    subs = {}
    for name in [s.strip() for s in args.also.split(",") if s.strip()]:
        if name == args.workload:
            continue
        torch.cuda.empty_cache()
        rec = measure(name, args, min(args.cpu_seconds, 3.0),
                      warmup=max(args.warmup, SUB_MIN_WARMUP))
        for k in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data",
                  "unit", "steps"):
            rec.pop(k, None)
        subs[name] = rec
    if subs:
        out["sub_workloads"] = subs
    print(json.dumps(out), flush=True)
    return 0


SUB_MIN_WARMUP = 20


def measure(workload: str, args, cpu_seconds: float, warmup: int | None = None) -> dict:
    """One workload: warm-up (args.warmup steps unless warmup is given), exactly
    args.steps timed steps (each one call of the
    whole layer, moe_forward or moe_block_forward), the dominant kernel's roofline
    from HIP events the library records around it inside the timed region, a stage
    breakdown pass and a timing of the staged entry points, and the CPU oracle on a
    bounded sample with a parity spot check of the timed run's output."""
    import numpy as np
    import torch

    import moe_inputs as mi
    import sparse_mixture_experts_wg_amd as moe
    from tests import parity

    cfg = mi.CONFIGS[workload]
    T, d, h, E, K, S = cfg.T, cfg.d, cfg.h, cfg.E, cfg.K, cfg.S
    print(f"# workload {cfg.name}: T={T} d={d} h={h} E={E} K={K} {cfg.dtype}; generating",
          file=sys.stderr, flush=True)
    inp = mi.make_inputs(cfg, seed=0)
    dev = parity.upload_inputs({k: inp[k] for k in ("x", "w_g")}, cfg.dtype)
    copies = max(1, args.weight_copies)
    wsets = []
    for c in range(copies):
        wsets.append({k: parity.device_array(inp[k], cfg.dtype) for k in ("w1", "w3", "w2")})
    # the staged calls let the down projection leave partial sums for the combine, as
    # the one-call entry point does internally
    cap = moe.capacity_rows(T, K, E, args.capacity_factor) if args.capacity_factor > 0 else 0
    p = moe.problem(T, d, h, E, K, cfg.dtype, "f32", args.path, moe.FLAG_DOWN_PARTIALS,
                    capacity=cap)
    path = "stream" if moe.resolve_path(p) == moe.PATH_STREAM else "tiled"
    parts = moe.down_parts(p)
    if cfg.dtype == "f32":
        path = "f32"
    f32 = torch.float32
    dt = torch.bfloat16 if cfg.dtype == "bf16" else f32
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=f32, device="cuda")
    offsets = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    perm = torch.empty((S,), dtype=torch.int32, device="cuda")
    slot = torch.empty((T, K), dtype=torch.int32, device="cuda")
    # bf16: the gate-up kernels read the token rows through perm_token (no x_perm
    # copy), as moe_forward does; float32 gathers x_perm in the permute
    rows_direct = cfg.dtype == "bf16"
    x_perm = None if rows_direct else torch.empty((S, d), dtype=dt, device="cuda")
    act = torch.empty((S, h), dtype=dt, device="cuda")
    o_perm = torch.empty((S, d) if parts == 1 else (parts, S, d), dtype=f32, device="cuda")
    y = torch.empty((T, d), dtype=f32, device="cuda")
    BLOCK_EPS = 1e-5
    if args.block:
        blk = mi.make_block(cfg, seed=0)
        h_in = parity.device_array(blk["h"], cfg.dtype)
        norm_w = parity.device_array(blk["norm_w"], cfg.dtype)
        x_in = torch.empty((T, d), dtype=dt, device="cuda")  # normalised block input
    else:
        x_in = dev["x"]

    # the timed step: one call of the whole layer (the library records the gate-up
    # events inside it when `gu` is given)
    if args.block:
        ws_fwd = torch.empty((moe.block_workspace_bytes(p),), dtype=torch.uint8, device="cuda")
    else:
        ws_fwd = torch.empty((moe.forward_workspace_bytes(p),), dtype=torch.uint8, device="cuda")

    def step(i, gu=None):
        ws = wsets[i % copies]
        if args.block:
            moe.block_forward(p, h_in, norm_w, BLOCK_EPS, dev["w_g"], ws["w1"], ws["w3"], ws["w2"],
                              y, topk_idx=idx, topk_w=w, ws=ws_fwd, events=gu)
        else:
            moe.forward(p, x_in, dev["w_g"], ws["w1"], ws["w3"], ws["w2"], y, topk_idx=idx,
                        topk_w=w, ws=ws_fwd, events=gu)

    # the same layer through the staged entry points, for the stage breakdown
    def step_staged(i, ev=None):
        ws = wsets[i % copies]
        if ev is not None:
            ev[0].record()
        if args.block:
            moe.rmsnorm(p, h_in, norm_w, BLOCK_EPS, x_in)
            if ev is not None:
                ev[5].record()
        moe.route(p, x_in, dev["w_g"], idx, w)
        moe.permute(p, x_in, idx, offsets, perm, slot, x_perm, gather=not rows_direct)
        if ev is not None:
            ev[1].record()
        if rows_direct:
            moe.expert_gate_up_rows(p, x_in, perm, offsets, ws["w1"], ws["w3"], act)
        else:
            moe.expert_gate_up(p, x_perm, offsets, ws["w1"], ws["w3"], act)
        if ev is not None:
            ev[2].record()
        moe.expert_down(p, act, offsets, ws["w2"], o_perm)
        if ev is not None:
            ev[3].record()
        if args.block:
            moe.combine_residual(p, o_perm, slot, w, h_in, y)
        else:
            moe.combine(p, o_perm, slot, w, y)
        if ev is not None:
            ev[4].record()

    n_warm = args.warmup if warmup is None else warmup
    print(f"# path {path}; {n_warm} warm-up steps", file=sys.stderr, flush=True)
    for i in range(n_warm):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps. The only events inside it bracket the
    # dominant kernel (gate-up): the library records them on the stream it launches
    # on (torch's current stream, which the binding passes), on every GU_EVERY-th
    # step from the first; a pair of events costs about 6 us of a 430 us decode
    # step. Recording each event once beforehand creates it.
    gu_steps = list(range(0, args.steps, GU_EVERY))
    gu_events = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in gu_steps}
    for evs in gu_events.values():
        for ev in evs:
            ev.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, gu=gu_events.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    gu_ms_live = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in gu_events.values()]))
    tokens_per_s = T / (ms_step / 1e3)

    # Stage breakdown: a separate, shorter pass with events between all stages
    # (events add a few microseconds each, so this pass is not the timed one).
    n_diag = max(3, min(args.steps, 30))
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n_diag)]
    for i in range(n_diag):
        step_staged(i, events[i])
    torch.cuda.synchronize()
    counts = np.diff(parity.host_array(offsets).astype(np.int64))
    stage = np.array([[ev[j].elapsed_time(ev[j + 1]) for j in range(4)] for ev in events])
    stage_ms = stage.mean(axis=0)
    norm_ms = float(np.mean([ev[0].elapsed_time(ev[5]) for ev in events])) if args.block else None
    step_ms = np.array([ev[0].elapsed_time(ev[4]) for ev in events])
    gpu_ms_step = float(np.mean(step_ms))

    # the staged entry points, one call per stage, for comparison (not part of the
    # timed region)
    n_st = max(5, min(args.steps, 50))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(n_st):
        step_staged(i)
    torch.cuda.synchronize()
    ms_staged = (time.perf_counter() - t1) * 1e3 / n_st
    # the timed run's output again for the spot check below (the staged passes
    # write the same buffers with bitwise the same values)
    step(0)
    torch.cuda.synchronize()

    # ---- roofline of the dominant kernel (gate-up) --------------------------------
    es = 2 if cfg.dtype == "bf16" else 4
    hit = int(np.sum(counts > 0))
    gu_ms = gu_ms_live
    S_rows = int(counts.sum())  # rows the experts run: S, or fewer under a capacity cap
    gu_bytes = hit * 2 * h * d * es + S_rows * d * es + S_rows * h * es
    gu_flop = 2.0 * S_rows * d * 2 * h
    layer_bytes = hit * 3 * h * d * es + d * E * es + T * d * es + T * d * 4
    layer_flop = 2.0 * S_rows * 3 * d * h + 2.0 * T * d * E
    kernel = {"stream": "stream_gate_up", "tiled": "tiled_gate_up", "f32": "f32_gate_up"}[path]
    sha = source_hash(kernel_files(path)) if path != "f32" else None
    traffic_rec = load_traffic(cfg.name, kernel, sha) if sha else None
    traffic = None
    traffic_detail = None
    if traffic_rec:
        # HBM bytes per launch from rocprofv3: reads from the L2's sized read requests
        # (exact for a 1 GiB device copy), writes from WRITE_SIZE scaled by what it reads
        # for that copy
        traffic = traffic_rec["read_bytes_per_launch"] + traffic_rec["write_bytes_per_launch"]
        traffic_detail = {"read_bytes": traffic_rec["read_bytes_per_launch"],
                          "write_bytes": traffic_rec["write_bytes_per_launch"],
                          "fetch_size_kib_raw": traffic_rec["fetch_size_kib_per_dispatch_raw"],
                          "write_scale": traffic_rec["write_scale"],
                          "over_algorithmic": traffic_rec["traffic_over_algorithmic"],
                          "source": f"profiles/traffic_{kernel}_{cfg.name}.json"}
    if path == "stream":
        achieved = gu_bytes / (gu_ms / 1e3) / 1e9
        roof = {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": gu_bytes, "avg_launch_ms": round(gu_ms, 5),
                "launches_timed": len(gu_steps), "traffic": traffic,
                "traffic_detail": traffic_detail}
        layer = {"hbm_frac": round(layer_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                 "algorithmic_bytes": layer_bytes}
    else:
        peak = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
        achieved = gu_flop / (gu_ms / 1e3) / 1e12
        roof = {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "algorithmic_flop": gu_flop,
                "avg_launch_ms": round(gu_ms, 5), "launches_timed": len(gu_steps),
                "traffic": traffic, "traffic_detail": traffic_detail}
        layer = {"mfma_frac": round(layer_flop / (ms_step / 1e3) / 1e12 / peak, 4),
                 "algorithmic_flop": layer_flop}

    # ---- CPU oracle baseline on a bounded sample, plus a parity spot check ---------
    cpu = None
    spot = None
    if not args.no_cpu_baseline:
        import oracle

        o = oracle.load()
        per_tok = 2.0 * K * 3 * d * h
        n = int(min(T, max(8, round(cpu_seconds * 2.0e9 * o.threads / per_tok))))
        toks = np.arange(n)
        print(f"# CPU oracle on {n} tokens x {o.threads} threads", file=sys.stderr, flush=True)
        c0 = time.perf_counter()
        passes = 0
        while True:
            if args.block:
                xs, _ = o.rmsnorm(np.ascontiguousarray(blk["h"][:n]), blk["norm_w"], BLOCK_EPS,
                                  cfg.dtype)
            else:
                xs = np.ascontiguousarray(inp["x"][:n])
            l, idx_r, w_r, margin = o.route(xs, inp["w_g"], K, cfg.dtype)
            y_ref = o.forward_tokens(toks, xs, inp["w1"], inp["w3"], inp["w2"], idx_r, w_r,
                                     cfg.dtype)
            passes += 1
            if time.perf_counter() - c0 >= cpu_seconds or passes >= 100:
                break
        cpu_s = (time.perf_counter() - c0) / passes
        cpu = {"value": round(n / cpu_s, 3), "unit": "tokens/s", "cores": o.threads,
               "kind": "oracle",
               "sample": f"first {n} of {T} tokens of {cfg.name} (route + all K experts + "
                         f"combine{', with the RMSNorm and residual of the block' if args.block else ''}"
                         f", float64), {passes} pass(es), {cpu_s:.2f} s per pass"}
        # parity of the timed run's output on the same tokens (rule R applied)
        ih = parity.host_array(idx)[:n]
        wh = parity.host_array(w)[:n]
        # (block: x is normalised in float32 on the GPU and in float64 here, both rounded
        # once to bf16, so routing is compared with the block's wider near-tie margin)
        tol = dict(tie_margin=1e-2, w_tol=2e-3) if args.block and cfg.dtype == "bf16" else {}
        idx_eval, diff = parity.check_routing(ih, wh, l, idx_r, margin, K, o, **tol)
        if len(diff) or cap:
            w_eval = o.set_weights(l, idx_eval)
            if cap:  # the cap keeps the earliest slots, so the first n tokens decide alone
                w_eval = o.capped_weights(o.permute_capped(idx_eval, E, cap)[2], w_eval)
            y_ref = o.forward_tokens(toks, xs, inp["w1"], inp["w3"], inp["w2"], idx_eval,
                                     w_eval, cfg.dtype)
        y_gpu = parity.host_array(y)[:n].astype(np.float64)
        if args.block:  # compare the MoE part; the residual is added exactly in float32
            y_gpu = y_gpu - mi.to_float64(blk["h"][:n], cfg.dtype)
        spot_rel = parity.check_output(y_gpu, y_ref, cfg.dtype, "bench")
        spot = {"tokens": n, "max_err_over_rms": float(f"{spot_rel:.4e}"),
                "tolerance": parity.Y_TOL[cfg.dtype]}

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded generator; random-init weights of the layer's shape)",
        "config": {"workload": cfg.name, "T": T, "d": d, "h": h, "E": E, "K": K,
                   "path": path, "down_partial_sums": parts, "weight_copies": copies,
                   "block": bool(args.block), "capacity": cap,
                   "capacity_factor": args.capacity_factor},
        "roofline": roof,
        "layer": layer,
        "cpu_baseline": cpu,
        "stages_ms": {("rmsnorm+route+permute" if args.block else "route+permute"):
                      round(float(stage_ms[0]), 5),
                      "gate_up": round(float(stage_ms[1]), 5),
                      "down": round(float(stage_ms[2]), 5),
                      "combine": round(float(stage_ms[3]), 5)},
        "gpu_ms_per_step_events": round(gpu_ms_step, 5),
        "gpu_ms_per_step_events_stats": {"median": round(float(np.median(step_ms)), 5),
                                         "min": round(float(np.min(step_ms)), 5),
                                         "p90": round(float(np.percentile(step_ms, 90)), 5),
                                         "steps": int(step_ms.size)},
        "block_rmsnorm": None if norm_ms is None else {
            "ms": round(norm_ms, 5),
            "hbm_bytes": T * d * es * 2 + d * es,
            "achieved_GBps": round((T * d * es * 2 + d * es) / (norm_ms / 1e3) / 1e9, 1),
            "frac_of_hbm_peak": round((T * d * es * 2 + d * es) / (norm_ms / 1e3) / 1e9
                                      / HBM_PEAK_GBS, 4)},
        "stages_note": f"separate pass of {n_diag} steps with events between the stages",
        "ms_per_step_staged_api": round(ms_staged, 5),
        "rows_per_expert": counts.tolist(),
        "parity_spot_check": spot,
    }
    del wsets, dev
    return out


if __name__ == "__main__":
    sys.exit(main())
