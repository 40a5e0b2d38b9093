"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--entry E] [--lse] [--backward] [--no-cpu]

One step is one launch of the fused forward over one batch of the workload
(default: SD2.1 512x512 UNet self-attention, B2 H5 N4096 d64, no mask),
through attn_fwd_ws (keys split evenly over the resident work-groups when
that balances the chip; --entry attn_fwd for one work-group per query tile;
attn_fwd_ex, the default for cross-attention, also writes the logsumexp with
--lse). With --backward a step is one attn_bwd call (gradients of Q, K and V
from the forward's output and logsumexp, computed once before timing). Inputs
and the workspace are resident in HBM before timing starts. Prints one JSON
line on stdout.

FLOP accounting (the metric of the workload): 4 Nq Nkv d per head without a
mask, half of 4 N^2 d with the causal mask, 4 N (window cells) d per head for
neighbourhood attention (the window-sized work); the backward counts its five
products, 10 Nq Nkv d per head (half with the causal mask, window-sized for
neighbourhood attention). Algorithmic bytes:
q, k, v read once and o (and the float32 logsumexp, if asked for) written once;
the backward reads q, k, v, o, dO and the logsumexp and writes dq, dk, dv.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

# MI355X published dense bf16 MFMA peak (256 CUs x 2.4 GHz x 4096 FLOP/clk) and HBM3E bandwidth
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0


def flops(w: workloads.Workload) -> float:
    per_head = 4.0 * w.N * w.n_kv * w.d
    if w.mask == "causal":
        assert w.n_kv == w.N, "causal metric defined for self-attention"
        per_head /= 2
    elif w.mask in ("na2d", "na3d"):
        cells = w.na.get("kernel_d", 1) * w.na["kernel_h"] * w.na["kernel_w"]
        per_head = 4.0 * w.N * cells * w.d
    return per_head * w.B * w.H


def backward_flops(w: workloads.Workload) -> float:
    per_head = 10.0 * w.N * w.n_kv * w.d
    if w.mask == "causal":
        per_head /= 2
    elif w.mask in ("na2d", "na3d"):
        per_head = 10.0 * w.N * w.na.get("kernel_d", 1) * w.na["kernel_h"] * w.na["kernel_w"] * w.d
    return per_head * w.B * w.H


def backward_bytes(w: workloads.Workload) -> float:
    return w.B * w.H * ((4.0 * w.N + 4.0 * w.n_kv) * w.d * 2 + 4.0 * w.N)


def algorithmic_bytes(w: workloads.Workload, lse: bool = False) -> float:
    return w.B * w.H * (2.0 * (w.N + w.n_kv) * w.d * 2 + (4.0 * w.N if lse else 0.0))


RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")
KERNEL_SOURCES = ["attn_fwd.hip", "kernel_common.hpp", "launch.hpp", "tile_plan.hpp"]
BWD_KERNEL_SOURCES = ["attn_bwd.hip", "kernel_common.hpp", "launch.hpp", "tile_plan.hpp"]


def recorded_traffic(name: str, sources=KERNEL_SOURCES):
    """Calibrated HBM bytes of one launch from profiles/traffic.txt, if taken on the current kernel sources."""
    import hashlib

    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "exact_attention_68_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    digest = h.hexdigest()[:16]
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        parts = ln.split()
        if len(parts) == 4 and not ln.startswith("#") and parts[0] == name and parts[1] == digest:
            return (float(parts[2]) + float(parts[3])) * 1024.0
    return None


def mask_mode(A, w):
    return {"none": A.ATTN_MASK_NONE, "causal": A.ATTN_MASK_CAUSAL, "na2d": A.ATTN_MASK_NA2D,
            "na3d": A.ATTN_MASK_NA3D}[w.mask]


def window_params(A, w):
    if w.mask == "na2d":
        return A.na2d_params(**w.na)
    if w.mask == "na3d":
        return A.na3d_params(**w.na)
    return None


def cpu_baseline(w: workloads.Workload, q, k, v, budget_s: float = 12.0) -> dict:
    """Time the float64 oracle on the host cores: whole heads, repeated until about budget_s has passed."""
    import oracle

    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((p.get("num_threads", 1) for p in info), default=1)
    except Exception:  # threadpoolctl missing or unable to inspect
        threads = os.cpu_count() or 1
    qf, kf, vf = (t.float().numpy() for t in (q, k, v))
    na = None
    if w.na:
        kind = oracle.NA3D if w.mask == "na3d" else oracle.NA2D
        na = kind(**{kk: (bool(vv) if kk.startswith("wrap") else vv) for kk, vv in w.na.items()})
    heads = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b, h = divmod(heads % (w.B * w.H), w.H)
        oracle.attention(qf[b:b + 1, h:h + 1], kf[b:b + 1, h:h + 1], vf[b:b + 1, h:h + 1], w.scale, w.mask, na)
        heads += 1
    dt = time.perf_counter() - t0
    f = flops(w) * heads / (w.B * w.H)
    return {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} heads of {w.name} ({heads / (w.B * w.H):.1f} passes over its {w.B * w.H} heads; "
                      f"float64 NumPy, S materialised per head) in {dt:.1f} s; host has {os.cpu_count()} logical CPUs"}


def copy_calibration(nbytes: int = 256 << 20, reps: int = 3) -> None:
    """A plain device-to-device copy of known size, for scaling memory-traffic counters."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {reps} copies of {nbytes} bytes", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=workloads.HEADLINE, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--entry", default=None, choices=["attn_fwd_ws", "attn_fwd", "attn_fwd_ex"],
                    help="C entry point (default attn_fwd_ws, attn_fwd_ex for cross-attention)")
    ap.add_argument("--lse", action="store_true", help="attn_fwd_ex also writes the logsumexp")
    ap.add_argument("--backward", action="store_true", help="time attn_bwd (the gradients) instead of the forward")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for traffic counters)")
    ap.add_argument("--traffic-kib", type=float, nargs=2, metavar=("FETCH", "WRITE"), default=None,
                    help="FETCH_SIZE and WRITE_SIZE of one launch in KiB, already scaled by the copy calibration")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    from exact_attention_68_amd.build import ensure_built
    ensure_built()
    import exact_attention_68_amd as A

    w = workloads.WORKLOADS[args.workload]
    entry = args.entry or ("attn_fwd_ex" if (w.n_kv != w.N or args.lse) else "attn_fwd_ws")
    if entry != "attn_fwd_ex" and (w.n_kv != w.N or args.lse):
        ap.error("cross-attention and --lse need --entry attn_fwd_ex")
    q, k, v = workloads.workload_qkv(w)
    dev = torch.device("cuda:0")
    dq, dk, dv = (t.to(dev) for t in (q, k, v))
    do = torch.empty_like(dq)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev) if args.lse else None
    params = window_params(A, w)
    mode = mask_mode(A, w)
    stream = torch.cuda.current_stream(dev)

    ws = None
    if entry != "attn_fwd":
        nbytes = A.attn_fwd_ex_workspace_size(w.B, w.H, w.N, w.n_kv, w.d, mode, params)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev) if nbytes else None

    def step():
        if entry == "attn_fwd_ws":
            A.attn_fwd_ws(dq, dk, dv, do, w.scale, mode, params, ws, stream.cuda_stream)
        elif entry == "attn_fwd_ex":
            A.attn_fwd_ex(dq, dk, dv, do, lse, w.scale, mode, params, ws, stream.cuda_stream)
        else:
            A.attn_fwd(dq, dk, dv, do, w.scale, mode, params, stream.cuda_stream)

    if args.backward:
        g = torch.Generator(device="cpu").manual_seed(w.seed + 1)
        ddo = torch.randn(w.B, w.H, w.N, w.d, generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev)
        lse_f = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
        nf = A.attn_fwd_ex_workspace_size(w.B, w.H, w.N, w.n_kv, w.d, mode, params)
        wsf = torch.zeros(nf, dtype=torch.uint8, device=dev) if nf else None
        A.attn_fwd_ex(dq, dk, dv, do, lse_f, w.scale, mode, params, wsf, stream.cuda_stream)
        wsb = torch.zeros(A.attn_bwd_workspace_size(w.B, w.H, w.N, w.n_kv, w.d, mode, params), dtype=torch.uint8,
                          device=dev)
        gq, gk, gv = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
        ws = wsb
        entry = "attn_bwd"

        def step():
            A.attn_bwd(dq, dk, dv, do, ddo, lse_f, gq, gk, gv, w.scale, mode, params, wsb, stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: warmup {args.warmup} done, timing {args.steps} steps", file=sys.stderr, flush=True)

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps

    F = backward_flops(w) if args.backward else flops(w)
    value = F * args.steps / wall / 1e12
    achieved = F / (kernel_ms * 1e-3) / 1e12
    nbytes = backward_bytes(w) if args.backward else algorithmic_bytes(w, args.lse)
    # neighbourhood windows and short key sequences sit below the ridge of the roofline: HBM-bound
    if w.mask in ("na2d", "na3d") or F / nbytes < RIDGE_FLOP_PER_BYTE:  # (forward and backward alike)
        roof = {"bound": "hbm", "achieved": nbytes / (kernel_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # what the event-timed step contains: the attention kernel, plus the merge kernel of a split launch
    split = ws is not None and not args.backward
    roof["kernels"] = (f"attn_bwd_dq_kernel<{w.d},{w.mask}> + attn_bwd_dkv_kernel<{w.d},{w.mask}>"
                       if args.backward else
                       (f"attn_fwd_kernel<{w.d},none,split> + attn_merge_kernel" if split
                        else f"attn_fwd_kernel<{w.d},{w.mask}>"))
    roof["traffic"] = (sum(args.traffic_kib) * 1024.0 if args.traffic_kib
                       else recorded_traffic(f"{w.name}:{entry}{':lse' if args.lse else ''}"))
    if args.backward:
        roof["traffic"] = recorded_traffic(f"{w.name}:attn_bwd", BWD_KERNEL_SOURCES)

    line = {
        "metric": "attention fwd TFLOP/s and % of bf16 MFMA peak, SD2.1 B2 H5 N4096 d64",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "pct_of_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "kernel_us": kernel_ms * 1e3,
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "Nkv": w.n_kv, "d": w.d, "mask": w.mask,
                   "scale": w.scale, **({"window": w.na} if w.na else {}), "entry": entry, "lse": args.lse,
                   "workspace_bytes": 0 if ws is None else ws.numel()},
        "roofline": roof,
    }
    if args.copy_calibration:
        copy_calibration()
    if args.backward:
        line["metric"] = "attention bwd TFLOP/s (dQ, dK, dV) and % of bf16 MFMA peak"
        line["pct_of_peak"] = 100.0 * value / PEAK_BF16_TFLOPS
    if not args.no_cpu and not args.backward:
        line["cpu_baseline"] = cpu_baseline(w, q, k, v)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
