#!/usr/bin/env python3
"""Throughput of HSTU jagged attention on one MI355X (gfx950).

One step = the whole path for one batch of the long-sequence forward+backward workload (batch 16,
lengths uniform in [1024, 8192], 8 heads of width 128, 8 context tokens and 64 candidates per
sequence, position + time relative bias, bf16 inputs with fp32 accumulation): build the work-list
plan on the host and upload it, attention forward, then the dK/dV and dQ + bias-gradient
backward passes (the dK/dV pass stores dS, bf16, for the dQ pass to read back).  Inputs are
resident in HBM before timing starts.

FLOPs are counted on visible (unmasked) pairs only: 4d per pair per head forward, 10d backward.

Prints one JSON line.  Besides the headline workload it reports the forward-only workloads
(ranking-shaped, long-tail, full layer) with warm and cold-cache timings, the full layer's
backward, candidate scoring against cached history, Stochastic Length compaction, the dominant
kernel's roofline, and the fp64 CPU oracle timed on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "HSTU jagged attn fwd+bwd TFLOP/s (unmasked FLOPs), % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE = "long_fwdbwd"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# What a kernel's HBM traffic depends on: its source, the shared device helpers and the plan
# code that fixes the launch order (the L2 hits across work units).
_CSRC = "hstu_jagged_pointwise_amd/csrc/"
KERNEL_SOURCES = {
    "fwd": (_CSRC + "attn_fwd.hip", _CSRC + "device_common.h", _CSRC + "hstu_api.hip"),
    "bwd_dkdv": (_CSRC + "attn_bwd.hip", _CSRC + "device_common.h", _CSRC + "hstu_api.hip"),
    "bwd_dq": (_CSRC + "attn_bwd.hip", _CSRC + "device_common.h", _CSRC + "hstu_api.hip"),
}
# Algorithmic MFMA work per visible pair per head, in units of d: forward S and P.V; the dK/dV
# pass S, dP, dV, dK (it also stores dS); the dQ pass dS.K from the stored dS.
FLOPS_PER_PAIR_D = {"fwd": 4, "bwd_dkdv": 8, "bwd_dq": 2}


def describe(w):
    return (f"{w['name']}: batch {w['batch']}, total tokens {w['total_tokens']}, heads {w['heads']}, "
            f"head dim {w['d']}, max_seqlen {w['max_seqlen']}, contexts {w['num_contexts']}, "
            f"candidates {int(w['num_targets'][0]) if len(w['num_targets']) else 0}, "
            f"position+time bias {'yes' if w.get('rab_pos') is not None else 'no'}")


def sha256(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if the kernel source, the
    device helpers and the plan code are unchanged since they were taken; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != sha256(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


KERNEL_NAMES = {"fwd": "fwd_bf16_kernel<128", "bwd_dkdv": "bwd_dkdv_kernel<128",
                "bwd_dq": "bwd_dq_stored_kernel<128"}


def write_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, out=TRAFFIC_FILE):
    """HBM bytes per launch of the headline kernels from rocprofv3 counter runs.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) come from separate runs of
    `bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-extra`; each is scaled by bytes / counter
    for a plain 1 GiB device copy (`bench.py --copy-calibration`) profiled with the same counter.
    """
    import csv

    def per_kernel(path, counter):
        vals = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] == counter:
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return vals

    def copy_scale(path, counter):
        v = [x for k, xs in per_kernel(path, counter).items() if "copyBuffer" in k for x in xs]
        return (1 << 30) / (1024.0 * float(np.median(v)))

    fs, ws = copy_scale(copy_fetch_csv, "FETCH_SIZE"), copy_scale(copy_write_csv, "WRITE_SIZE")
    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    rec = {"_calibration": {"fetch_bytes_per_kib": round(1024 * fs, 3),
                            "write_bytes_per_kib": round(1024 * ws, 3),
                            "copy": "1 GiB device-to-device copy, 5 launches"}}
    for kernel, pattern in KERNEL_NAMES.items():
        f = [x for k, xs in fetch.items() if pattern in k for x in xs]
        wr = [x for k, xs in write.items() if pattern in k for x in xs]
        if not f or not wr:
            continue
        rb, wb = 1024 * fs * float(np.mean(f)), 1024 * ws * float(np.mean(wr))
        rec[kernel] = {"bytes_per_launch": int(rb + wb), "read_bytes": int(rb), "write_bytes": int(wb),
                       "fetch_kib_raw": float(np.mean(f)), "write_kib_raw": float(np.mean(wr)),
                       "dispatches": len(f), "source_sha256": sha256(KERNEL_SOURCES[kernel])}
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def cpu_baseline(w_full, budget_pairs=60_000_000):
    """The oracle (fp64 loops, OpenMP) on a bounded sample of the workload: the first sequence,
    with as many heads as fit the pair budget (heads are independent)."""
    import oracle
    off = w_full["seq_offsets"]
    d = w_full["d"]
    per_head = oracle.count_pairs(off[:2], w_full["num_contexts"], w_full["num_targets"][:1])
    hs_ = int(max(1, min(w_full["heads"], budget_pairs // max(per_head, 1))))
    e = int(off[1])
    w = dict(w_full)
    w.update(batch=1, heads=hs_, seq_offsets=off[:2].copy(), num_targets=w_full["num_targets"][:1],
             total_tokens=e, timestamps=w_full["timestamps"][:e],
             rab_pos=w_full["rab_pos"][:hs_], rab_ts=w_full["rab_ts"][:hs_])
    for key in ("q", "k", "v", "dout"):
        w[key] = np.ascontiguousarray(w_full[key][:e, :hs_])
    pairs = per_head * hs_
    t0 = time.perf_counter()
    oracle.attn_fwd(w)
    oracle.attn_bwd(w)
    dt = time.perf_counter() - t0
    flops = pairs * 14 * d
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"forward+backward of sequence 0 ({e} tokens) on heads 0..{hs_ - 1}: "
                      f"{pairs} visible pairs of the same workload, fp64"}


class Timer:
    """HIP events on torch's current stream (the stream every library call is enqueued on)."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = {}

    def record(self, name, fn):
        ev0 = self.torch.cuda.Event(enable_timing=True)
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev0.record()
        fn()
        ev1.record()
        self.marks.setdefault(name, []).append((ev0, ev1))

    def ms(self, name):
        return [a.elapsed_time(b) for a, b in self.marks.get(name, [])]


def bench_headline(args, torch, hj, runner, w):
    dev = runner.to_device(w)
    base_args = runner.args_for(w, dev)
    T, H, d = w["total_tokens"], w["heads"], w["d"]
    out = runner.empty_like_thd(w, dev)
    dq, dk, dv = (runner.empty_like_thd(w, dev) for _ in range(3))
    drp = torch.empty((H, 128), dtype=torch.float32, device=out.device)
    drt = torch.empty((H, 128), dtype=torch.float32, device=out.device)
    timer = Timer(torch)
    plan_host_s = []
    # stored dS: the same size for every step's plan of this batch
    p0 = runner.plan_for(w, base_args)
    ws = torch.empty(max(hj.hstu_workspace_bytes(p0, hj.OP_BWD), 16), dtype=torch.uint8,
                     device=out.device)
    info = hj.hstu_plan_info(p0)
    p0.close()

    def build():
        return runner.plan_for(w, base_args)

    # host planning time on its own (a host-only plan: no upload, which in the loop below waits
    # for the previous step's kernels)
    for _ in range(5):
        t0 = time.perf_counter()
        runner.plan_for(w, base_args, hj.HSTU_PLAN_HOST_ONLY).close()
        plan_host_s.append(time.perf_counter() - t0)

    def launch(plan, record):
        def fwd():
            hj.hstu_attn_fwd(plan, base_args, dev["q"], dev["k"], dev["v"], out)

        def dkdv():
            hj.hstu_attn_bwd_dkdv(plan, base_args, dev["q"], dev["k"], dev["v"], dev["dout"], dk, dv,
                                  ws=ws)

        def dqp():
            hj.hstu_attn_bwd_dq(plan, base_args, dev["q"], dev["k"], dev["v"], dev["dout"], dq, drp, drt,
                                ws=ws)

        if record:
            timer.record("fwd", fwd)
            timer.record("bwd_dkdv", dkdv)
            timer.record("bwd_dq", dqp)
        else:
            fwd(); dkdv(); dqp()

    for _ in range(args.warmup):
        plan = build()
        launch(plan, False)
        torch.cuda.current_stream().synchronize()
        plan.close()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # Every step builds its own plan on the host.  A step's plan is built, and uploaded through
    # the library's own stream, while the previous step's kernels run (as a data loader prepares
    # the next batch).  A plan is destroyed after the next step is queued: its buffer goes back in
    # the order of this (default) stream, after the kernels that read it.
    plan, prev = build(), None
    for k in range(args.steps):
        launch(plan, True)
        nxt = build() if k + 1 < args.steps else None
        if prev is not None:
            prev.close()
        prev, plan = plan, nxt
    torch.cuda.synchronize()
    prev.close()
    wall = time.perf_counter() - t0
    assert torch.isfinite(out.float()).all() and torch.isfinite(dq.float()).all()

    pairs = info["visible_pairs"]
    flops = pairs * 14 * d
    ms_step = wall * 1e3 / args.steps
    kern = {name: float(np.mean(timer.ms(name))) for name in ("fwd", "bwd_dkdv", "bwd_dq")}
    gpu_ms = sum(kern.values())
    return dict(info=info, pairs=pairs, flops=flops, ms_step=ms_step, kern=kern, gpu_ms=gpu_ms,
                plan_ms=1e3 * float(np.median(plan_host_s)), tokens=T)


def roofline(kern, pairs, d):
    name = max(kern, key=kern.get)
    flops = pairs * FLOPS_PER_PAIR_D[name] * d
    achieved = flops / (kern[name] * 1e-3) / 1e12
    traffic = measured_traffic(name)
    return {"kernel": name, "bound": "mfma", "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": flops,
            "per_unit": f"{FLOPS_PER_PAIR_D[name]}*d flops per visible pair per head"}


def bench_forward(torch, hj, runner, name, iters=20, cold=False):
    import hstu_synth as hs
    w = hs.make_workload(name)
    dev = runner.to_device(w)
    a = runner.args_for(w, dev)
    plan = runner.plan_for(w, a)
    info = hj.hstu_plan_info(plan)
    T, H, d = w["total_tokens"], w["heads"], w["d"]
    layer = bool(w.get("layer_dim"))
    if layer:
        D = w["layer_dim"]
        y = torch.empty((T, D), dtype=torch.bfloat16, device="cuda:0")
        ws = torch.empty(hj.hstu_workspace_bytes(plan, hj.OP_LAYER, D), dtype=torch.uint8, device="cuda:0")
        call = lambda: hj.hstu_layer_fwd(plan, a, D, dev["x"], dev["w1"], dev["w2"], y, ws=ws)
        flops = info["visible_pairs"] * 4 * d + 2 * T * D * 4 * H * d + 2 * T * H * d * D
        nbytes = 2 * (2 * T * D + D * 4 * H * d + H * d * D)
    else:
        out = runner.empty_like_thd(w, dev)
        call = lambda: hj.hstu_attn_fwd(plan, a, dev["q"], dev["k"], dev["v"], out)
        flops = info["visible_pairs"] * 4 * d
        nbytes = T * H * d * 2 * 4 + (T * 8 if w.get("timestamps") is not None else 0)
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0") if cold else None
    for _ in range(5):
        call()
    timer = Timer(torch)
    for _ in range(iters):
        if cold:
            scratch.fill_(1.0)  # 1 GiB written between timed calls evicts the 256 MB cache
        timer.record("x", call)
    torch.cuda.synchronize()
    ms = timer.ms("x")
    med = float(np.median(ms))
    plan.close()
    return {"ms_median": round(med, 4), "ms_p10": round(float(np.percentile(ms, 10)), 4),
            "ms_p90": round(float(np.percentile(ms, 90)), 4),
            "tflops": round(flops / med / 1e9, 2), "pct_bf16_peak": round(100 * flops / med / 1e9 / PEAK_BF16_TFLOPS, 2),
            "tokens_per_s": round(T / med * 1e3, 1), "algorithmic_GBps": round(nbytes / med / 1e6, 1),
            "pct_hbm_peak": round(100 * nbytes / med / 1e6 / PEAK_HBM_GBS, 2),
            "visible_pairs": info["visible_pairs"], "flops": flops, "bytes": nbytes}


def bench_cached(torch, hj, runner, iters=20):
    """Candidate scoring against cached history: 128 users with long-tail history lengths, 64
    candidates each (4 heads of width 128).  FLOPs: 4d per visible (candidate, key) pair per
    head; bytes: candidate q, k, v and output, cached k and v, and the timestamps."""
    import hstu_synth as hs
    w = hs.make_cached_workload()
    dev = runner.to_device(w)
    a = runner.args_for(w, dev)
    plan = hj.hstu_plan_create_cached(a, w["cand_offsets"], w["cache_offsets"])
    info = hj.hstu_plan_info(plan)
    out = runner.empty_like_thd(w, dev)
    ws = torch.empty(max(hj.hstu_workspace_bytes(plan, hj.OP_CACHED), 16), dtype=torch.uint8,
                     device="cuda:0")
    call = lambda: hj.hstu_attn_fwd_cached(plan, a, dev["q"], dev["k"], dev["v"], dev["k_cache"],
                                           dev["v_cache"], dev["cache_timestamps"], out, ws=ws)
    T, Tc, H, d = w["total_tokens"], w["cache_tokens"], w["heads"], w["d"]
    flops = info["visible_pairs"] * 4 * d
    nbytes = (4 * T + 2 * Tc) * H * d * 2 + 8 * (T + Tc)
    for _ in range(5):
        call()
    timer = Timer(torch)
    for _ in range(iters):
        timer.record("x", call)
    torch.cuda.synchronize()
    med = float(np.median(timer.ms("x")))
    plan.close()
    return {"ms_median": round(med, 4), "tflops": round(flops / med / 1e9, 2),
            "pct_bf16_peak": round(100 * flops / med / 1e9 / PEAK_BF16_TFLOPS, 2),
            "candidates_per_s": round(T / med * 1e3, 1),
            "algorithmic_GBps": round(nbytes / med / 1e6, 1),
            "pct_hbm_peak": round(100 * nbytes / med / 1e6 / PEAK_HBM_GBS, 2),
            "visible_pairs": info["visible_pairs"], "flops": flops, "bytes": nbytes}


def bench_select(torch, hj, iters=20):
    """Stochastic Length compaction of one THD tensor of the long-sequence workload (74k tokens,
    8 x 128 bf16 per token), every sequence cut to its 2048 most recent tokens.  Bytes: the kept
    rows read once and written once (an HBM-bound copy)."""
    import hstu_synth as hs
    spec = hs.WORKLOADS[HEADLINE]
    L = hs.draw_lengths(np.random.default_rng(0), spec, spec.batch)
    keep = np.minimum(L, 2048)
    so, do = hs.offsets_from_lengths(L), hs.offsets_from_lengths(keep)
    row = (spec.heads, spec.d)
    src = torch.empty((int(so[-1]),) + row, dtype=torch.bfloat16, device="cuda:0").normal_()
    dst = torch.empty((int(do[-1]),) + row, dtype=torch.bfloat16, device="cuda:0")
    dso = torch.from_numpy(so).cuda()
    ddo = torch.from_numpy(do).cuda()
    call = lambda: hj.hstu_jagged_select(dso, ddo, src, dst)
    for _ in range(5):
        call()
    timer = Timer(torch)
    for _ in range(iters):
        timer.record("x", call)
    torch.cuda.synchronize()
    med = float(np.median(timer.ms("x")))
    nbytes = 2 * dst.numel() * dst.element_size()
    return {"ms_median": round(med, 4), "algorithmic_GBps": round(nbytes / med / 1e6, 1),
            "pct_hbm_peak": round(100 * nbytes / med / 1e6 / PEAK_HBM_GBS, 2),
            "rows_kept": int(do[-1]), "rows_in": int(so[-1]), "bytes": nbytes}


def bench_layer_bwd(torch, hj, runner, iters=20):
    """Full layer backward (recompute of the forward's intermediates included) on the full-layer
    workload with dY ~ N(0, 1).  FLOPs counted: the backward's own products only, i.e. dG, dW2,
    dW1, dX (2 T D Hd (1 + 1 + 4 + 4)) and 10d per visible pair per head for the attention; the
    recomputed X W1 and attention forward are work done but not counted."""
    import hstu_synth as hs
    w = hs.make_workload("layer_fwd")
    T, H, d, D = w["total_tokens"], w["heads"], w["d"], w["layer_dim"]
    w["dy"] = hs.round_bf16(np.random.default_rng(1).normal(0.0, 1.0, (T, D)).astype(np.float32))
    dev = runner.to_device(w)
    a = runner.args_for(w, dev)
    plan = runner.plan_for(w, a)
    info = hj.hstu_plan_info(plan)
    ws = torch.empty(hj.hstu_workspace_bytes(plan, hj.OP_LAYER_BWD, D), dtype=torch.uint8,
                     device="cuda:0")
    f32 = dict(dtype=torch.float32, device="cuda:0")
    dx = torch.empty((T, D), dtype=torch.bfloat16, device="cuda:0")
    dw1, dw2 = torch.empty((D, 4 * H * d), **f32), torch.empty((H * d, D), **f32)
    drp, drt = torch.empty((H, 128), **f32), torch.empty((H, 128), **f32)
    call = lambda: hj.hstu_layer_bwd(plan, a, D, dev["x"], dev["w1"], dev["w2"], dev["dy"], dx,
                                     dw1, dw2, drp, drt, ws=ws)
    flops = 20 * T * D * H * d + 10 * d * info["visible_pairs"]
    for _ in range(5):
        call()
    timer = Timer(torch)
    for _ in range(iters):
        timer.record("x", call)
    torch.cuda.synchronize()
    med = float(np.median(timer.ms("x")))
    plan.close()
    return {"ms_median": round(med, 4), "tflops": round(flops / med / 1e9, 2),
            "pct_bf16_peak": round(100 * flops / med / 1e9 / PEAK_BF16_TFLOPS, 2),
            "tokens_per_s": round(T / med * 1e3, 1), "flops": flops,
            "flops_counted": "dG, dW2, dW1, dX products and 10d per visible pair per head"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the forward-only workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                         "COPY_WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter files into the per-kernel "
                         "HBM traffic record (no GPU use)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only; this implementation has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4,
                          "launches": 5}))
        return

    import hstu_jagged_pointwise_amd as hj
    import hstu_synth as hs
    from hstu_jagged_pointwise_amd import runner
    hj.load_library()

    w = hs.make_workload(HEADLINE)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w)
    r = bench_headline(args, torch, hj, runner, w)
    d = w["d"]
    value = r["flops"] / (r["ms_step"] * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(w), "global_batch": w["batch"],
                   "seq_len": f"uniform [1024, 8192], max {w['max_seqlen']}",
                   "parallelism": "single GPU"},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(r["tokens"] / (r["ms_step"] * 1e-3), 1),
        "visible_pairs": r["pairs"],
        "flops_per_step": r["flops"],
        "kernel_ms": {k: round(v, 4) for k, v in r["kern"].items()},
        "kernel_sum_ms": round(r["gpu_ms"], 4),
        "kernel_only_tflops": round(r["flops"] / (r["gpu_ms"] * 1e-3) / 1e12, 2),
        "plan_host_ms": round(r["plan_ms"], 4),
        "roofline": roofline(r["kern"], r["pairs"], d),
        "cpu_baseline": cpu,
    }
    if not args.no_extra:
        extra = {}
        for name in ("ranking_fwd", "longtail_fwd", "layer_fwd"):
            extra[name] = {"warm": bench_forward(torch, hj, runner, name)}
        extra["longtail_fwd"]["cold"] = bench_forward(torch, hj, runner, "longtail_fwd", cold=True)
        result["forward_workloads"] = extra
        result["layer_backward"] = bench_layer_bwd(torch, hj, runner)
        result["cached_scoring"] = bench_cached(torch, hj, runner)
        result["stochastic_length_select"] = bench_select(torch, hj)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
