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
line on stdout. Before the warm-up steps the step is repeated, untimed, for
--spinup-ms (300 ms by default; reported as "spinup"): timed right after idle,
a few milliseconds of work run while the GPU's clocks are still ramping up.

Before timing, the run measures its own workload under rocprofv3 in child
processes (this script with --child, placed after `--`): a kernel trace (the
per-dispatch durations; their median per step is reported beside the HIP-event
time), a counter pass for the matrix cores (mfma_util) and FETCH_SIZE and
WRITE_SIZE passes scaled by a plain 256 MiB device copy (roofline.traffic and
hbm_gbs). --no-prof skips them; a pass that fails leaves its fields null.

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


# ---------------------------------------------------------------- live profiler passes
# The default run measures its own workload under rocprofv3 in child processes (the
# program itself after `--`, never a relaunch of this process), before this process
# touches the GPU: a kernel trace (per-dispatch durations, median over steps, as the
# headline's cross-check of the HIP-event time), one counter pass for the matrix
# cores (SQ_VALU_MFMA_BUSY_CYCLES against GRBM_GUI_ACTIVE) and one each for
# FETCH_SIZE and WRITE_SIZE, scaled by a plain device copy of known size in the same
# run. Each field states its source; a pass that fails leaves its fields null.
PROF_TIMEOUT_S = 180
XCD_CUS = 32  # CUs per XCD on MI355X (GRBM_GUI_ACTIVE is summed over the XCDs)


def _child_cmd(args, steps: int, warmup: int, calibrate: bool = False, spinup: bool = False) -> list:
    cmd = [sys.executable, os.path.abspath(__file__), "--child", "--no-cpu", "--workload", args.workload,
           "--steps", str(steps), "--warmup", str(warmup), "--spinup-ms", str(args.spinup_ms if spinup else 0)]
    if args.entry:
        cmd += ["--entry", args.entry]
    if args.lse:
        cmd.append("--lse")
    if args.backward:
        cmd.append("--backward")
    if calibrate:
        cmd.append("--copy-calibration")
    return cmd


def _rocprof(prof_args: list, child: list, out_dir: str):
    """Run rocprofv3 <prof_args> -d out_dir -o run -- child; returns the list of its csv files, or
    None. rocprofv3 may exit non-zero after a complete run (its own teardown); the files decide."""
    import glob
    import signal
    import subprocess

    cmd = ["rocprofv3", *prof_args, "--output-format", "csv", "-d", out_dir, "-o", "run", "--", *child]
    env = dict(os.environ, TMPDIR="/tmp")
    try:
        proc = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True, cwd="/tmp",
                                env=env, start_new_session=True)
        try:
            _, err = proc.communicate(timeout=PROF_TIMEOUT_S)
        except subprocess.TimeoutExpired:
            os.killpg(proc.pid, signal.SIGKILL)
            proc.communicate()
            print(f"[bench] rocprofv3 {' '.join(prof_args)}: timed out", file=sys.stderr, flush=True)
            return None
    except OSError as e:
        print(f"[bench] rocprofv3 not runnable: {e}", file=sys.stderr, flush=True)
        return None
    files = glob.glob(os.path.join(out_dir, "**", "*.csv"), recursive=True)
    if not files:
        print(f"[bench] rocprofv3 {' '.join(prof_args)}: no output (rc {proc.returncode}): {err[-400:]}",
              file=sys.stderr, flush=True)
        return None
    return files


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return None if n == 0 else (xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2]))


def _counter_rows(files):
    """{dispatch id: (kernel name, {counter: value})} from rocprofv3 counter-collection csv files."""
    import csv

    out = {}
    for f in files:
        if not f.endswith("counter_collection.csv"):
            continue
        for row in csv.DictReader(open(f)):
            did = (f, row.get("Dispatch_Id"))
            name, ctr = out.setdefault(did, (row.get("Kernel_Name", ""), {}))
            ctr[row["Counter_Name"]] = ctr.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return out


def live_profile(args, steps_per_call_kernels: int, cus: int) -> dict:
    """The profiler passes of one workload; returns the fields of the bench line."""
    import csv
    import shutil
    import tempfile

    res = {"kernel_trace": None, "mfma_util": None, "traffic_bytes": None}
    # the kernels of one step (the backward run also holds the one forward call made before timing)
    step_kernel = ("attn_bwd_",) if args.backward else ("attn_fwd_", "attn_split_clear_kernel")
    main_kernel = "attn_bwd_dkv" if args.backward else "attn_fwd_"
    if shutil.which("rocprofv3") is None:
        return res
    work = tempfile.mkdtemp(prefix="attn_bench_prof_")
    try:
        # kernel trace: 30 timed calls after the clock spin-up and 5 warm-up calls; the last 30 calls' dispatches
        files = _rocprof(["--kernel-trace"], _child_cmd(args, 30, 5, spinup=True), os.path.join(work, "trace"))
        if files:
            rows = []
            for f in files:
                if f.endswith("kernel_trace.csv"):
                    rows += [r for r in csv.DictReader(open(f))
                             if any(k in r.get("Kernel_Name", "") for k in step_kernel)]
            rows.sort(key=lambda r: int(r["Start_Timestamp"]))
            rows = rows[-30 * steps_per_call_kernels:]
            per_kernel = {}
            for r in rows:
                short = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("attn::", "")
                per_kernel.setdefault(short, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            steps = [sum((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                         for r in rows[i:i + steps_per_call_kernels])
                     for i in range(0, len(rows) - steps_per_call_kernels + 1, steps_per_call_kernels)]
            if steps:
                res["kernel_trace"] = {
                    "step_us_median": _median(steps), "steps": len(steps),
                    "kernels": {k: {"median_us": _median(v), "calls": len(v)} for k, v in per_kernel.items()},
                    "source": "rocprofv3 --kernel-trace of this run (child process), median over steps"}
        # matrix-core busy cycles of the dominant kernel, per dispatch
        files = _rocprof(["--pmc", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
                         _child_cmd(args, 5, 2), os.path.join(work, "mfma"))
        if files:
            utils = []
            for name, ctr in _counter_rows(files).values():
                if main_kernel in name:
                    xcds = max(1, cus // XCD_CUS)
                    cycles = ctr.get("GRBM_GUI_ACTIVE", 0.0) / xcds
                    if cycles > 0:
                        utils.append(ctr.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4 * cus) / cycles)
            if utils:
                res["mfma_util"] = _median(utils)
        # HBM traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) in separate passes, each scaled by
        # what the counter reads for a plain device copy of 256 MiB in the same run
        traffic = 0.0
        for ctr_name in ("FETCH_SIZE", "WRITE_SIZE"):
            files = _rocprof(["--pmc", ctr_name], _child_cmd(args, 5, 2, calibrate=True),
                             os.path.join(work, ctr_name))
            if not files:
                traffic = None
                break
            att, calib = {}, []
            for name, ctr in _counter_rows(files).values():
                if any(k in name for k in step_kernel):
                    att.setdefault(name.split("(")[0], []).append(ctr.get(ctr_name, 0.0))
                elif "copy" in name.lower():
                    calib.append(ctr.get(ctr_name, 0.0))
            if not att or not calib:
                traffic = None
                break
            factor = (256 << 10) / _median(calib)  # KiB moved per KiB counted
            traffic += sum(_median(v) for v in att.values()) * 1024.0 * factor
            res[f"{ctr_name.lower()}_factor"] = factor
            for name, v in att.items():
                short = name.replace("void ", "").replace("attn::", "")
                res.setdefault("traffic_kernels", {}).setdefault(short, {})[ctr_name] = _median(v) * 1024.0 * factor
        res["traffic_bytes"] = traffic
    finally:
        shutil.rmtree(work, ignore_errors=True)
    return res


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
    ap.add_argument("--no-prof", action="store_true",
                    help="skip the live rocprofv3 passes (kernel trace, MFMA busy, HBM traffic)")
    ap.add_argument("--spinup-ms", type=float, default=300.0,
                    help="before the warm-up steps, repeat the step for this long so that the GPU's clocks "
                         "leave their idle state (0: none)")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)  # a profiled pass of the parent
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

    prof = None
    if not args.child and not args.no_prof:
        split_call = ws is not None and not args.backward
        kernels_per_call = 2 if (args.backward or split_call) else 1
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        print(f"[bench] {w.name}: rocprofv3 passes (kernel trace, MFMA busy, FETCH_SIZE, WRITE_SIZE)", file=sys.stderr,
              flush=True)
        prof = live_profile(args, kernels_per_call, cus)

    # Clock spin-up: the GPU leaves idle at reduced clocks and needs some tens of milliseconds of
    # load to reach its steady state; a step of 50-200 us timed over a few milliseconds right after
    # idle measures that ramp, not the kernels. The step is repeated (untimed) for spinup_ms first.
    spin_calls, t_spin = 0, time.perf_counter()
    while args.spinup_ms > 0 and (time.perf_counter() - t_spin) * 1e3 < args.spinup_ms:
        for _ in range(16):
            step()
        spin_calls += 16
        torch.cuda.synchronize()
    spin_ms = (time.perf_counter() - t_spin) * 1e3
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
    # what the event-timed step contains: the attention kernel, after the counter clear of a split launch
    split = ws is not None and not args.backward
    roof["kernels"] = (f"attn_bwd_dq_kernel<{w.d},{w.mask}> + attn_bwd_dkv_kernel<{w.d},{w.mask}>"
                       if args.backward else
                       (f"attn_split_clear_kernel + attn_fwd_kernel<{w.d},none,split>" if split
                        else f"attn_fwd_kernel<{w.d},{w.mask}>"))
    if prof and prof.get("kernel_trace"):  # the names the kernel trace recorded
        roof["kernels"] = " + ".join(prof["kernel_trace"]["kernels"])
    # HBM bytes of one step, from this run's FETCH_SIZE and WRITE_SIZE passes (or given on the command line)
    roof["traffic"] = None
    if prof and prof.get("traffic_bytes"):
        roof["traffic"] = prof["traffic_bytes"]
        roof["traffic_source"] = ("rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE passes of this run, per dispatch, "
                                  "scaled by a 256 MiB device copy in the same pass")
        roof["traffic_kernels"] = prof.get("traffic_kernels")
    elif args.traffic_kib:
        roof["traffic"] = sum(args.traffic_kib) * 1024.0
        roof["traffic_source"] = "--traffic-kib"

    line = {
        "metric": "attention fwd TFLOP/s and % of bf16 MFMA peak, SD2.1 B2 H5 N4096 d64",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "spinup": {"ms": spin_ms, "calls": spin_calls},
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "pct_of_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "kernel_us": kernel_ms * 1e3,
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "Nkv": w.n_kv, "d": w.d, "mask": w.mask,
                   "scale": w.scale, **({"window": w.na} if w.na else {}), "entry": entry, "lse": args.lse,
                   "workspace_bytes": 0 if ws is None else ws.numel()},
        "roofline": roof,
    }
    # matrix-core utilisation and HBM bandwidth (the measurement contract), from the live passes
    line["mfma_util"] = prof.get("mfma_util") if prof else None
    line["mfma_util_source"] = ("rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES / (4 x CUs) / (GRBM_GUI_ACTIVE / XCDs) of "
                                "the attention kernel, median over dispatches" if line["mfma_util"] is not None
                                else None)
    line["hbm_gbs"] = roof["traffic"] / (kernel_ms * 1e-3) / 1e9 if roof["traffic"] else None
    if prof and prof.get("kernel_trace"):
        kt = prof["kernel_trace"]
        line["kernel_trace"] = kt
        line["kernel_trace_tflops"] = F / (kt["step_us_median"] * 1e-6) / 1e12
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
