#!/usr/bin/env python
"""Throughput of range-masked flash attention on one MI355X.

One step = the whole hot path of a training step over one batch of seeded
synthetic input that is already resident in HBM: validate and plan the
slices on the host, copy the plan to the device, run the training forward
(out, lse and the record the backward reads), run the backward.  Default
workload: 8 packed causal sequences of 8192 tokens (65536 tokens), 32 q heads,
8 kv heads, head size 128, bf16.

Reported (one JSON line):
  value        forward TFLOP/s over unmasked pairs: 4 * d * hq * pairs divided
               by the mean duration of ffa_fwd (out and lse: v's fp16 copy and
               the forward kernel), timed after the steps with HIP events
               recorded on the stream the kernels run on
  fwd_train_*  the same for the step's training forward (ffa_fwd_ex with a
               saved record: fp16 copy of v, P V in fp16, out's residual)
  bwd_tflops   backward TFLOP/s, 10 * d * hq * pairs over the backward kernels
  ms_per_step  wall-clock milliseconds per step, planning included
  roofline     the forward kernel against the bf16 MFMA peak
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402

METRIC = "fwd TFLOP/s over unmasked pairs + % bf16 MFMA peak (bwd TFLOP/s too)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FWD_SOURCE = os.path.join(ROOT, "range_masked_attention_amd", "csrc", "fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_long_packed_traffic.json")


def visible_pairs(w: W.Workload) -> int:
    """Number of visible (i, j) cells of the slice mask, in closed form per slice.

    Slices are disjoint, so the count is a sum over slices: a FULL slice is a
    rectangle; in a CAUSAL slice row i sees keys [ks, min(ke, i + 1 + ke - qe)).
    """
    qr, kr, ty = w.slices()
    n = 0
    for (qs, qe), (ks, ke), t in zip(qr.tolist(), kr.tolist(), ty.tolist()):
        if qs == qe or ks == ke:
            continue
        if t == W.FULL:
            n += (qe - qs) * (ke - ks)
            continue
        rows = np.arange(qs, qe, dtype=np.int64)
        n += int(np.clip(np.minimum(ke, rows + 1 + ke - qe) - ks, 0, None).sum())
    return n


def source_hash(path: str) -> str:
    """Hash of a kernel source with its comments and spacing dropped, so an
    edit of the comments alone does not count as a change of the kernel."""
    with open(path, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def measured_traffic(per_launch_algo_bytes: float):
    """HBM bytes per forward launch from the committed rocprofv3 counter runs,
    if they were taken on the current forward kernel source (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != source_hash(FWD_SOURCE):
        return None
    return t.get("hbm_bytes_per_launch")


def fwd_kernel_name(w: W.Workload, alibi: bool) -> str:
    """The forward kernel ffa_fwd launches for this workload, as the profiler
    names it: two q heads per workgroup when q heads pair up within a kv head
    and there are at least 512 such workgroups.  Work items are at least one
    per q tile and kv head (cutting long lists only adds some), which decides
    it for every workload here."""
    grp = w.hq // w.hkv
    units = ((w.Tq + 127) // 128) * w.hkv
    hpw = 2 if grp % 2 == 0 and units * (grp // 2) >= 512 else 1
    return f"fwd_kernel<{w.d}, {str(w.softcap > 0).lower()}, {str(alibi).lower()}, {hpw}>"


def cpu_baseline(w: W.Workload, q, k, v, budget_s: float):
    """Time the fp64 oracle on whole 256-row blocks spread over the sequence."""
    from oracle import ffa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    qr, kr, ty = w.slices()
    q64, k64, v64 = q.double().numpy(), k.double().numpy(), v.double().numpy()
    n_blocks = (w.Tq + 255) // 256
    order = np.random.default_rng(0).permutation(n_blocks)
    sl = O.normalise_slices(qr, kr, ty, w.Tq, w.Tk)
    pairs, done, t0 = 0, 0, time.perf_counter()
    for b in order:
        rows = np.arange(b * 256, min(w.Tq, b * 256 + 256))
        O.attention_fwd(q64, k64, v64, qr, kr, ty, w.scale, w.softcap, rows=rows)
        pairs += int((O.visibility(sl, rows, np.arange(w.Tk)) > 0).sum())
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(4.0 * w.d * w.hq * pairs / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"forward of {done} random 256-row blocks of {n_blocks} ({pairs} visible pairs, "
                      f"all {w.hq} heads) in {dt:.1f} s, fp64 NumPy"}


def mfma_ceiling() -> int:
    """The matrix cores' rate on their own, by operand values (probe library
    range_masked_attention_amd/_lib/libffa_probe.so): one JSON line.  With the
    pipes busy all the time, the rate over the nominal peak is the clock over
    the nominal 2.4 GHz, which the GPU's power limit lowers as the operands'
    bits get busier."""
    import ctypes
    from range_masked_attention_amd import _build
    if not os.path.exists(_build.PROBE_LIB):
        _build.build()
    lib = ctypes.CDLL(_build.PROBE_LIB)
    lib.ffa_probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.ffa_probe_mfma_rate.restype = ctypes.c_int
    res = []
    for f16, dtype in ((0, "bf16"), (1, "f16")):
        for kind, name in ((0, "N(0,1)"), (1, "constant 0.7"), (2, "zeros")):
            t = ctypes.c_double(0.0)
            rc = lib.ffa_probe_mfma_rate(f16, kind, 2000, ctypes.byref(t))
            if rc != 0:
                print(json.dumps({"error": f"probe failed ({rc})", "dtype": dtype, "operands": name}))
                return 1
            res.append({"dtype": dtype, "operands": name, "value": round(t.value, 1),
                        "frac": round(t.value / PEAK_BF16_TFLOPS, 4)})
    print(json.dumps({"metric": "matrix-core TFLOP/s, 32x32x16 products on register operands", "unit": "TFLOP/s",
                      "peak": PEAK_BF16_TFLOPS, "waves_per_simd": 2, "results": res}))
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, help="workload number (1-5); 4 is the 64K-token batch")
    ap.add_argument("--no-bwd", action="store_true", help="time the forward only")
    ap.add_argument("--alibi", action="store_true",
                    help="add the distance bias with ALiBi's geometric slopes (a variant, not the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="time budget of the oracle sample")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the benchmark: matrix-core TFLOP/s of 32x32x16 products on register "
                         "operands (bf16 and fp16; N(0,1), constant and zero values)")
    args = ap.parse_args()
    if args.mfma_ceiling:
        sys.exit(mfma_ceiling())

    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; pass --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import range_masked_attention_amd as ffa
    if not os.path.exists(ffa.lib_path()):
        from range_masked_attention_amd import _build
        _build.build()
    ffa.load_library()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)

    w = W.config(args.config)
    do_bwd = w.backward and not args.no_bwd
    dev = torch.device("cuda:0")
    q, k, v, do = W.workload_tensors(w, with_dout=True)
    qd, kd, vd, od = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    out = torch.empty_like(qd)
    lse = torch.empty((w.Tq, w.hq), dtype=torch.float32, device=dev)
    # a training step runs the training forward, which saves a record (out's
    # rounding residual, v's fp16 copy) for the backward
    saved = (torch.empty(ffa.ffa_saved_size(w.Tq, w.Tk, w.hq, w.hkv, w.d), dtype=torch.uint8, device=dev)
             if do_bwd else None)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = torch.empty(max(ffa.ffa_bwd_workspace_size(w.Tq, w.Tk, w.hq, w.hkv, w.d), 16), dtype=torch.uint8, device=dev)
    qr, kr, ty = w.slices()
    slopes = (torch.tensor(ffa.alibi_geometric_slopes(w.hq), dtype=torch.float32, device=dev)
              if args.alibi else None)
    pairs = visible_pairs(w)
    fwd_flop = 4.0 * w.d * w.hq * pairs
    bwd_flop = 10.0 * w.d * w.hq * pairs

    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        t_plan = time.perf_counter()
        plan = ffa.ffa_plan_create(w.Tq, w.Tk, qr, kr, ty)
        t_plan = time.perf_counter() - t_plan
        if events:
            events[0].record(stream)
        ffa.ffa_fwd_planned(plan, qd, kd, vd, w.scale, w.softcap, out=out, lse=lse, alibi_slopes=slopes,
                            saved=saved)
        if events:
            events[1].record(stream)
        if do_bwd:
            ffa.ffa_bwd_planned(plan, qd, kd, vd, out, lse, od, w.scale, w.softcap,
                                dq=dq, dk=dk, dv=dv, workspace=ws, alibi_slopes=slopes, saved=saved)
            if events:
                events[2].record(stream)
        ffa.ffa_plan_destroy(plan)
        return t_plan

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    plan_s = 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        plan_s += step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the device-side planner on the same slices (outside the timed steps):
    # HIP events around repeated ffa_plan_refresh on the launch stream
    sl_dev = [torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=dev) for a in (qr, kr, ty)]
    dplan, dws = ffa.ffa_plan_create_device(w.Tq, w.Tk, *sl_dev)
    for _ in range(3):
        ffa.ffa_plan_refresh(dplan)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(20):
        ffa.ffa_plan_refresh(dplan)
    e1.record(stream)
    torch.cuda.synchronize()
    plan_device_ms = e0.elapsed_time(e1) / 20
    if ffa.ffa_plan_status(dplan) != 0:
        raise RuntimeError("device planner reported a bad status on the bench slices")
    ffa.ffa_plan_destroy(dplan)
    del dws

    # the forward as ffa_fwd runs it (out and lse only): the same number of
    # launches as steps, each between HIP events on the launch stream
    plan = ffa.ffa_plan_create(w.Tq, w.Tk, qr, kr, ty)
    for _ in range(2):
        ffa.ffa_fwd_planned(plan, qd, kd, vd, w.scale, w.softcap, out=out, lse=lse, alibi_slopes=slopes)
    fevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e in fevs:
        e[0].record(stream)
        ffa.ffa_fwd_planned(plan, qd, kd, vd, w.scale, w.softcap, out=out, lse=lse, alibi_slopes=slopes)
        e[1].record(stream)
    torch.cuda.synchronize()
    ffa.ffa_plan_destroy(plan)

    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in fevs]))
    fwd_train_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) if do_bwd else None
    ms_step = 1e3 * wall / args.steps
    fwd_tflops = fwd_flop / (fwd_ms * 1e-3) / 1e12
    fwd_train_tflops = fwd_flop / (fwd_train_ms * 1e-3) / 1e12
    bwd_tflops = bwd_flop / (bwd_ms * 1e-3) / 1e12 if do_bwd else None

    res = {
        "metric": METRIC,
        "value": round(fwd_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v/dO drawn on the CPU)",
        "config": {
            "workload": f"{w.name}: {w.Tq} tokens, {len(w.slices(padded=False)[0])} slices, "
                        f"hq={w.hq} hkv={w.hkv} d={w.d} softcap={w.softcap}"
                        + (", ALiBi slopes" if args.alibi else ""),
            "tokens": w.Tq, "hq": w.hq, "hkv": w.hkv, "head_dim": w.d,
            "visible_pairs": pairs,
            "step": "plan + fwd" + (" (training forward, saved record) + bwd" if do_bwd else ""),
        },
        "value_is": "ffa_fwd (out, lse) on the step's plan and inputs, timed after the steps",
        "fwd_ms": round(fwd_ms, 4),
        "fwd_frac_of_bf16_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
        "fwd_train_ms": round(fwd_train_ms, 4),
        "fwd_train_tflops": round(fwd_train_tflops, 2),
        "bwd_ms": round(bwd_ms, 4) if do_bwd else None,
        "bwd_tflops": round(bwd_tflops, 2) if do_bwd else None,
        "plan_ms": round(1e3 * plan_s / args.steps, 4),
        "plan_device_ms": round(plan_device_ms, 4),
        "step_tflops": round((fwd_flop + (bwd_flop if do_bwd else 0.0)) / (ms_step * 1e-3) / 1e12, 2),
    }
    algo_bytes = 2.0 * (w.Tq * w.hq * w.d * 2 + 2 * w.Tk * w.hkv * w.d) + 4.0 * w.Tq * w.hq
    res["roofline"] = {
        "bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s", "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
        "traffic": measured_traffic(algo_bytes),
        "kernel": fwd_kernel_name(w, args.alibi),
        "flop_per_launch": fwd_flop, "min_hbm_bytes_per_launch": algo_bytes,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
