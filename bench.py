#!/usr/bin/env python3
"""Monarch attention forward on one MI355X: ms/call, TFLOP/s, % of bf16 MFMA peak.

A step is one full forward (stage 1 + stage 2 of the Monarch product) over one
batch of seeded synthetic inputs that are already resident in device memory.
The default workload is the frame-aligned 21x30x52-token grid, 12 heads,
d=128, bf16 (b = 1560 tokens per block, m = 21 blocks per group).

Prints ONE JSON line. Besides the contract fields it carries:
  roofline      the dominant kernel's achieved rate against its roofline,
                timed with HIP events on the stream the kernels run on;
  cpu_baseline  the fp64 oracle timed on a bounded sample on the host cores;
  stages_two_launch  per-stage ms and rates of the two-launch path (stage 1
                then stage 2), timed separately; dense: the library's own
                dense softmax-attention kernel at the same shape; backward:
                the gradient pass at the same shape; chunk: one frame-causal
                chunk of three frames after a cache of the earlier frames;
                refine_one_step: the forward with one refinement step.
A call is stage 1 then stage 2 (two launches); --fused auto/on times the
library's one-launch fused variant instead where it applies (frame and tiled
alignments). call_ms_events: per-call device time from HIP events in a second
loop (the timed loop itself has nothing between the calls).

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 30] [--config frame_bf16]
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

METRIC = "Monarch-attn ms/call + TFLOP/s (% bf16 MFMA peak), N=32760 12h d128"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop per byte


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="frame_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--forward-only", action="store_true",
                    help="time the forward only: skip the other forward variant, the backward, the chunk and "
                         "the dense comparison (profiling runs: every launch of a kernel is then the same workload)")
    ap.add_argument("--fused", choices=["auto", "on", "off"], default="off",
                    help="one fused launch for both stages: where it applies (auto), required (on), "
                         "never (off, the default: the two-launch path measures faster)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for HBM counter scaling)")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of untimed forward calls before the warm-up calls (the first ~10 ms of "
                         "load after idle run in a power-management transient)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="only summarise a rocprofv3 kernel-trace CSV of a run of this bench (no GPU): "
                         "per-kernel launch statistics and the dominant kernel's roofline fraction")
    ap.add_argument("--trace-kernel", default="flash_kernel<128, false, false",
                    help="with --trace-summary / --traffic-summary: substring of the kernel's name")
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV",
                    help="only summarise rocprofv3 --pmc CSVs (no GPU): per kernel and grid, the mean of "
                         "every counter over its dispatches")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="only summarise HBM traffic (no GPU) from four rocprofv3 --pmc CSVs: FETCH_SIZE and "
                         "WRITE_SIZE of a run of this bench, and of a --copy-calibration run")
    return ap.parse_args()


def source_digest() -> str:
    """Digest of the device-code sources (kernel_*.hip and the headers they include; not the
    host-only C-ABI source); stored HBM counter figures are valid only for it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "structured_attention_video_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith(".h") or (f.startswith("kernel_") and f.endswith(".hip")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, config: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if still current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{config}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def trace_summary(path: str, config: str, kernel: str) -> None:
    """Per-kernel statistics of a rocprofv3 --kernel-trace CSV of a run of this bench, and the
    roofline fraction of the stage-1 kernel at this workload from its mean launch duration.
    Launches are grouped by kernel and grid size (the dense comparison and the chunk use the
    same kernel on other grids); the stage-1 group is the most-launched one whose kernel name
    contains `kernel`, and its mean is over every launch in it."""
    import csv
    import statistics
    import datagen
    c = datagen.CONFIGS[config]
    T, H, W = c["grid"]
    N = T * H * W
    b = {"frame": H * W, "row": W, "dense": N, "token": 1}[c["align"]]
    m = (c["tile_tokens"] or N) // b
    # the MFMA flash kernel takes the stage whose problems exceed 128 rows (stage 1: b rows,
    # stage 2: m_tau rows); its algorithmic FLOP per launch are that stage's
    stage, L = ("stage-1", b) if b > 128 else ("stage-2", m)
    if "fused" in kernel:  # the one-launch forward does both stages
        stage, L = "fused", b + m
    flops1 = 4 * c["batch"] * c["heads"] * N * L * c["d"]
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    by = {}
    for r in rows:
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]))
        by.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"# {os.path.basename(path)}: {len(rows)} dispatches; durations in us")
    print(f"{'calls':>5} {'mean':>9} {'median':>9} {'min':>9} {'max':>9} {'threads':>9}  kernel")
    for (name, grid), d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        print(f"{len(d):5d} {statistics.mean(d):9.1f} {statistics.median(d):9.1f} {min(d):9.1f} {max(d):9.1f} "
              f"{grid:9d}  {name[:90]}")
    cand = [(k, d) for k, d in by.items() if kernel in k[0]]
    if not cand:
        print(f"# no kernel matching {kernel!r}")
        return
    (name, grid), d = max(cand, key=lambda kv: len(kv[1]))
    mean = statistics.mean(d)
    tf = flops1 / (mean * 1e-6) / 1e12
    print(f"# {stage} kernel {name[:70]} (grid {grid} threads): {len(d)} launches, mean {mean:.1f} us, "
          f"median {statistics.median(d):.1f} us")
    print(f"# {stage} algorithmic FLOP per launch {flops1} / mean -> {tf:.1f} TFLOP/s = frac "
          f"{tf / PEAK_BF16_TFLOPS:.4f} of {PEAK_BF16_TFLOPS:.0f} TFLOP/s")


def _pmc_rows(path):
    import csv
    by = {}
    for r in csv.DictReader(open(path)):
        key = (r["Kernel_Name"], int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0))
        d = by.setdefault(key, {})
        d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return by


def counter_summary(paths) -> None:
    """Mean of every counter per (kernel, grid size) over its dispatches, per CSV."""
    for path in paths:
        print(f"# {os.path.basename(os.path.dirname(path))}/{os.path.basename(path)}")
        for (name, grid), d in sorted(_pmc_rows(path).items(), key=lambda kv: kv[0]):
            vals = ", ".join(f"{k}={sum(v) / len(v):.4g}" for k, v in sorted(d.items()))
            n = max(len(v) for v in d.values())
            print(f"{name[:70]:70s} grid={grid:<8d} dispatches={n:<4d} {vals}")


def traffic_summary(paths, config: str, kernel: str) -> None:
    """HBM bytes per launch of the kernels of a bench run: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) scaled by what the same counters read for a plain device copy of known size."""
    fetch, write, cfetch, cwrite = (_pmc_rows(p) for p in paths)
    copy_bytes = 1 << 30

    def one(rows, counter):
        vals = [v for d in rows.values() for v in d.get(counter, [])]
        return max(vals) if vals else float("nan")
    f_copy = copy_bytes / (one(cfetch, "FETCH_SIZE") * 1024)
    w_copy = copy_bytes / (one(cwrite, "WRITE_SIZE") * 1024)
    print(f"# copy calibration ({copy_bytes} B read and written): FETCH_SIZE factor {f_copy:.3f}, "
          f"WRITE_SIZE factor {w_copy:.3f}")
    print(f"source_digest: {source_digest()}")
    for (name, grid), d in sorted(fetch.items(), key=lambda kv: kv[0]):
        fv = d.get("FETCH_SIZE", [])
        wv = write.get((name, grid), {}).get("WRITE_SIZE", [])
        if not fv or not wv:
            continue
        fb = sum(fv) / len(fv) * 1024 * f_copy
        wb = sum(wv) / len(wv) * 1024 * w_copy
        tag = "  <- hbm_bytes_per_launch" if kernel in name else ""
        print(f"# {name[:70]} grid={grid}: read {fb:.4g} B, written {wb:.4g} B per launch{tag}")
        if tag:
            print(f"hbm_bytes_per_launch: {fb + wb:.6g}")
            tag = ""


def settle(fn, seconds: float) -> int:
    """Untimed calls of fn for about `seconds` of wall time; returns how many."""
    import torch
    if seconds <= 0:
        return 0
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds and n < 100000:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
    return n


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def cpu_baseline(cfg_name, q, k, v, b, tile, budget_s, gpu_out):
    """Time the fp64 oracle on the first heads of the workload (bounded sample)."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        threads = max((p.get("num_threads", 0) for p in threadpoolctl.threadpool_info()), default=0)
    except Exception:  # pragma: no cover
        threads = 0
    if not threads:
        threads = len(os.sched_getaffinity(0))
    heads_total = q.shape[0] * q.shape[1]
    qf, kf, vf = (x.reshape(-1, *x.shape[2:]) for x in (q, k, v))
    gf = gpu_out.reshape(-1, *gpu_out.shape[2:])
    done, t_total, worst_rel, worst_abs = 0, 0.0, 0.0, 0.0
    while done < heads_total and (done == 0 or t_total < budget_s):
        t0 = time.perf_counter()
        ref = oracle.monarch_forward(qf[done], kf[done], vf[done], b, tile or None)
        t_total += time.perf_counter() - t0
        got = gf[done].double().numpy()
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        worst_rel, worst_abs = max(worst_rel, rel), max(worst_abs, float(np.abs(got - ref).max()))
        done += 1
    ms_per_call = t_total / done * heads_total * 1e3
    return {
        "value": round(ms_per_call, 1), "unit": "ms/call", "cores": threads, "kind": "oracle",
        "sample": f"{done} of {heads_total} heads of {cfg_name} (fp64 NumPy, {t_total:.1f} s), "
                  f"scaled to all heads",
    }, {"heads_checked": done, "rel_l2": worst_rel, "max_abs": worst_abs}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(json.dumps({"error": "this build runs on one GPU only; the Monarch forward is not "
                          "sharded across GPUs (see the multi-GPU design note)", "n_gpus": args.gpus}))
        sys.exit(2)

    if args.trace_summary:
        trace_summary(args.trace_summary, args.config, args.trace_kernel)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.traffic_summary:
        traffic_summary(args.traffic_summary, args.config, args.trace_kernel)
        return

    import torch
    import datagen
    from structured_attention_video_amd import MonarchPlan

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return

    c = datagen.CONFIGS[args.config]
    dt = datagen.torch_dtype(c["dtype"])
    q_cpu, k_cpu, v_cpu = datagen.config_inputs(args.config)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (q_cpu, k_cpu, v_cpu))
    mk = lambda fused: MonarchPlan(c["batch"], c["heads"], c["d"], c["grid"], align=c["align"],
                                   tile_tokens=c["tile_tokens"], dtype=dt, fused=fused)
    plan = mk(args.fused != "off")
    if args.fused == "on" and not plan.fused:
        print(json.dumps({"error": f"the fused launch does not apply to {args.config}"}))
        sys.exit(2)
    split = mk(False)  # the two-launch path, timed per stage for context
    info = plan.info
    k1, k2 = split.kernel_names()
    has1, has2 = info["b"] > 1, info["m_tau"] > 1
    o = torch.empty_like(q)
    ws = plan.new_workspace(dev)
    y = torch.empty(q.shape, dtype=split.y_dtype, device=dev) if (has1 and has2) else None

    def call():
        plan.forward(q, k, v, out=o, workspace=ws)

    def timed(fn, n):
        """n calls of fn with HIP events around each (torch's current stream,
        where the library launches): per-call device times, sorted."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize()
        return sorted(e[0].elapsed_time(e[1]) for e in ev)

    # The first ~10 ms of load after idle run in a power-management transient (launches up
    # to ~30% slower, then back to the sustained rate): settle first, untimed, so that the
    # warm-up and the timed calls see the sustained clock.
    settle_calls = settle(call, args.settle_s)
    for _ in range(args.warmup):
        call()
    # the timed region: exactly `steps` calls, nothing else enqueued between them
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    per_call = timed(call, args.steps)
    pct = lambda xs, f: xs[min(len(xs) - 1, int(f * len(xs)))]

    # per-stage times of the two-launch path (context, and the roofline when not
    # fused): the two launches alternate as in a forward call, with HIP events
    # between them, so each launch runs in the conditions of the timed calls
    # (back-to-back launches of one stage alone run hotter and slower)
    stage_ms = {}
    if has1 and has2:
        for _ in range(2):
            split.stage1(q, k, v, y)
            split.stage2(q, k, y, o)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record()
            split.stage1(q, k, v, y)
            e[1].record()
            split.stage2(q, k, y, o)
            e[2].record()
        torch.cuda.synchronize()
        t1 = [e[0].elapsed_time(e[1]) for e in ev]
        t2 = [e[1].elapsed_time(e[2]) for e in ev]
        stage_ms = {"stage1": sum(t1) / len(t1), "stage2": sum(t2) / len(t2)}
        call()  # leave o = the measured path's output
    else:
        stage_ms = {"stage1" if has1 or not has2 else "stage2": sum(per_call) / len(per_call)}

    flops = info["flops_stage1"] + info["flops_stage2"]
    tflops = flops / (ms_step * 1e-3) / 1e12
    esz = 2 if c["dtype"] == "bf16" else 4
    tensor_b = c["batch"] * c["heads"] * info["N"] * c["d"] * esz
    yb = tensor_b if split.y_dtype == dt else tensor_b * 2
    # algorithmic bytes per launch: stage 1 reads Q,K,V writes Y; stage 2 reads Q,K,Y writes O
    bytes1 = 3 * tensor_b + (yb if has2 else 0) if has1 or not has2 else 0
    bytes2 = 2 * tensor_b + (yb if has1 else tensor_b) + tensor_b if has2 else 0
    stages = []
    if "stage1" in stage_ms:
        stages.append(dict(kernel=k1, launch="stage1", flops=info["flops_stage1"] or flops, bytes=bytes1,
                           ms=stage_ms["stage1"]))
    if "stage2" in stage_ms:
        stages.append(dict(kernel=k2, launch="stage2", flops=info["flops_stage2"], bytes=bytes2,
                           ms=stage_ms["stage2"]))
    for st in stages:
        st["tflops"] = st["flops"] / (st["ms"] * 1e-3) / 1e12
        st["gbs"] = st["bytes"] / (st["ms"] * 1e-3) / 1e9
        st["bound"] = "mfma" if st["flops"] / max(st["bytes"], 1) > RIDGE else "hbm"
    if plan.fused:
        # one persistent launch (after a control-block reset) does all the work:
        # it is the dominant kernel; its bytes are Q, K, V read and O written
        # (Y is produced and consumed inside the launch)
        dom = dict(kernel="fused_mfma_bf16", launch="forward", flops=flops, bytes=4 * tensor_b,
                   ms=sum(per_call) / len(per_call))
        dom["tflops"] = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
        dom["gbs"] = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        dom["bound"] = "mfma"
    else:
        dom = max(stages, key=lambda st: st["ms"])
    peak_mfma = PEAK_BF16_TFLOPS if c["dtype"] == "bf16" else PEAK_FP32_TFLOPS
    if dom["bound"] == "mfma":
        achieved, peak, unit = dom["tflops"], peak_mfma, "TFLOP/s"
    else:
        achieved, peak, unit = dom["gbs"], PEAK_HBM_GBS, "GB/s"
    traffic = stored_traffic(dom["kernel"], args.config)
    roofline = {"bound": dom["bound"], "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom["kernel"],
                "launch": dom["launch"], "avg_ms": round(dom["ms"], 4),
                "algorithmic_per_launch": dom["flops"] if dom["bound"] == "mfma" else dom["bytes"]}

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_calls": settle_calls,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c["dtype"],
        "data": "synthetic (seeded N(0,1) + 0.5 sinusoidal (t,h,w) code)" if c["pe_scale"] else "synthetic (seeded N(0,1))",
        "config": {"workload": args.config, "batch": c["batch"], "heads": c["heads"], "head_dim": c["d"],
                   "grid": list(c["grid"]), "N": info["N"], "b": info["b"], "m_tau": info["m_tau"],
                   "tile_tokens": info["tau"], "align": c["align"],
                   "y_dtype": "fp32" if split.y_dtype == torch.float32 else c["dtype"],
                   "fused": bool(plan.fused), "kernels": ["fused_mfma_bf16"] if plan.fused else [k1, k2]},
        "ms_per_call": round(ms_step, 4),
        "call_ms_events": {"p10": round(pct(per_call, 0.1), 4), "p50": round(pct(per_call, 0.5), 4),
                           "p90": round(pct(per_call, 0.9), 4)},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "flops_per_call": flops,
        "roofline": roofline,
        "stages_two_launch": [{k_: (round(v_, 4) if isinstance(v_, float) else v_) for k_, v_ in st.items()}
                              for st in stages],
    }

    # the other forward variant (fused one-launch vs two launches), for context
    alt = mk(not plan.fused)
    if alt.fused != plan.fused and not args.forward_only:
        alt_ws = alt.new_workspace(dev)
        oa = torch.empty_like(q)
        for _ in range(2):
            alt.forward(q, k, v, out=oa, workspace=alt_ws)
        ta = timed(lambda: alt.forward(q, k, v, out=oa, workspace=alt_ws), args.steps)
        out["other_variant"] = {"fused": bool(alt.fused), "ms_per_call_p50": round(pct(ta, 0.5), 4),
                                "tflops_p50": round(flops / (pct(ta, 0.5) * 1e-3) / 1e12, 2),
                                "bitwise_equal_to_timed_output": bool(torch.equal(oa, o))}
        del oa, alt_ws
    alt.close()

    # the forward with one refinement step of the factors at the same shape, for context
    rplan = MonarchPlan(c["batch"], c["heads"], c["d"], c["grid"], align=c["align"],
                        tile_tokens=c["tile_tokens"], dtype=dt, refine=True)
    if rplan.info["refine_steps"] and not args.forward_only:
        rws = rplan.new_workspace(dev)
        orf = torch.empty_like(q)
        for _ in range(2):
            rplan.forward(q, k, v, out=orf, workspace=rws)
        tr = timed(lambda: rplan.forward(q, k, v, out=orf, workspace=rws), args.steps)
        k1r, k2r = rplan.kernel_names()
        out["refine_one_step"] = {"ms_per_call_p50": round(pct(tr, 0.5), 4),
                                  "kernels": [k1r, k1r, k2r], "launches": "Y = R V; R K with row entropies; stage 2"}
        del rws, orf
    rplan.close()

    # the backward pass (gradients of all three inputs) at the same shape, for context:
    # time per call and the rate at 2.5x the forward FLOPs (five products of the
    # forward's size: the usual accounting for attention backward; the library
    # additionally recomputes the forward)
    if split.backward_workspace_bytes and not args.forward_only:
        bws = torch.empty(split.backward_workspace_bytes, dtype=torch.uint8, device=dev)
        go = torch.randn(q.shape, generator=torch.Generator().manual_seed(77)).to(dt).to(dev)
        gq, gk, gv = (torch.empty_like(q) for _ in range(3))
        ob = split.forward(q, k, v)
        for _ in range(2):
            split.backward(q, k, v, ob, go, workspace=bws, grads=(gq, gk, gv))
        tb = timed(lambda: split.backward(q, k, v, ob, go, workspace=bws, grads=(gq, gk, gv)),
                   max(3, args.steps // 5))
        # from a training forward's saved state (no forward recompute)
        split.forward_train(q, k, v, out=ob, workspace=bws)
        ts = timed(lambda: split.backward(q, k, v, ob, go, workspace=bws, grads=(gq, gk, gv), saved=True),
                   max(3, args.steps // 5))
        tt = timed(lambda: split.forward_train(q, k, v, out=ob, workspace=bws), max(3, args.steps // 5))
        out["backward"] = {"ms_per_call_p50": round(pct(tb, 0.5), 4),
                           "tflops_at_2p5x_forward": round(2.5 * flops / (pct(tb, 0.5) * 1e-3) / 1e12, 2),
                           "saved_state_ms_per_call_p50": round(pct(ts, 0.5), 4),
                           "forward_train_ms_per_call_p50": round(pct(tt, 0.5), 4)}
        del bws, go, gq, gk, gv, ob

    # one frame-causal chunk (the last three frames against the cache of all earlier
    # frames: autoregressive generation, three frames per chunk) at the same shape
    T = c["grid"][0]
    if (info["tiles"] == 1 and info["m_tau"] > 1 and T >= 4 and (c["grid"][1] * c["grid"][2]) % info["b"] == 0
            and not args.forward_only):
        yc = torch.zeros(q.shape, dtype=split.y_dtype, device=dev) if info["b"] > 1 else None
        oc = torch.empty_like(q)
        split.chunk_forward(q, k, v, yc, oc, 0, T - 3)
        for _ in range(2):
            split.chunk_forward(q, k, v, yc, oc, T - 3, T)
        tc = timed(lambda: split.chunk_forward(q, k, v, yc, oc, T - 3, T), args.steps)
        out["chunk"] = {"frames": [T - 3, T], "cached_frames": T - 3, "ms_per_call_p50": round(pct(tc, 0.5), 4)}
        del yc, oc

    if not args.no_dense and not args.forward_only:
        dplan = MonarchPlan(c["batch"], c["heads"], c["d"], c["grid"], align="dense", dtype=dt)
        od = torch.empty_like(q)
        dplan.forward(q, k, v, out=od)
        torch.cuda.synchronize()
        n_d = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_d):
            dplan.forward(q, k, v, out=od)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / n_d
        out["dense"] = {"kernel": dplan.kernel_names()[0], "ms_per_call": round(dms, 3),
                        "tflops": round(dplan.flops / (dms * 1e-3) / 1e12, 2),
                        "monarch_speedup": round(dms / ms_step, 2)}
        dplan.close()
        del od

    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        base, parity = cpu_baseline(args.config, q_cpu, k_cpu, v_cpu, info["b"], c["tile_tokens"],
                                    args.cpu_seconds, o.cpu())
        out["cpu_baseline"] = base
        out["parity_vs_oracle"] = parity
    else:
        out["cpu_baseline"] = None
    plan.close()
    split.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
