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

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) come from separate rocprofv3 --pmc runs of
    `bench.py --only long_fwdbwd --steps 5 --warmup 2`; each is scaled by bytes / counter for a
    plain 1 GiB device copy (`bench.py --copy-calibration`) profiled with the same counter.
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


def cpu_baseline(w_full, budget_pairs=250_000_000):
    """The oracle (fp64 loops, OpenMP over (sequence, head) units) on a bounded sample of the
    workload: its first sequences, all heads, as many as fit the pair budget (at least the
    first).  `cores` is the number of threads that had work: one unit per thread at most."""
    import oracle
    off = w_full["seq_offsets"]
    d, H = w_full["d"], w_full["heads"]
    nb, pairs = 0, 0
    for b in range(w_full["batch"]):
        p = H * oracle.count_pairs(off[b:b + 2] - off[b], w_full["num_contexts"],
                                   w_full["num_targets"][b:b + 1])
        if nb > 0 and pairs + p > budget_pairs:
            break
        nb, pairs = nb + 1, pairs + p
    e = int(off[nb])
    w = dict(w_full)
    w.update(batch=nb, seq_offsets=off[:nb + 1].copy(), num_targets=w_full["num_targets"][:nb],
             total_tokens=e, timestamps=w_full["timestamps"][:e])
    for key in ("q", "k", "v", "dout"):
        w[key] = np.ascontiguousarray(w_full[key][:e])
    t0 = time.perf_counter()
    oracle.attn_fwd(w)
    oracle.attn_bwd(w)
    dt = time.perf_counter() - t0
    flops = pairs * 14 * d
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": min(oracle.num_threads(), nb * H), "threads_available": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"forward+backward of the first {nb} sequence(s) ({e} tokens), all {H} heads: "
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
        if record:
            ev0 = torch.cuda.Event(enable_timing=True)
            ev0.record()

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
            ev1 = torch.cuda.Event(enable_timing=True)
            ev1.record()
            timer.marks.setdefault("step", []).append((ev0, ev1))
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
    # the next batch).  A plan is destroyed after the next step is queued, in the order of the
    # stream its kernels run on (hstu_plan_destroy_on): its buffer goes back after them, and the
    # host does not wait.
    stream = torch.cuda.current_stream()
    plan, prev = build(), None
    for k in range(args.steps):
        launch(plan, True)
        nxt = build() if k + 1 < args.steps else None
        if prev is not None:
            prev.close(stream)
        prev, plan = plan, nxt
    torch.cuda.synchronize()
    prev.close(stream)
    wall = time.perf_counter() - t0
    assert torch.isfinite(out.float()).all() and torch.isfinite(dq.float()).all()

    pairs = info["visible_pairs"]
    flops = pairs * 14 * d
    ms_step = wall * 1e3 / args.steps
    kern = {name: float(np.mean(timer.ms(name))) for name in ("fwd", "bwd_dkdv", "bwd_dq")}
    gpu_ms = sum(kern.values())
    step_ms = timer.ms("step")
    return dict(info=info, pairs=pairs, flops=flops, ms_step=ms_step, kern=kern, gpu_ms=gpu_ms,
                plan_ms=1e3 * float(np.median(plan_host_s)), tokens=T, step_ms=step_ms)


def algorithmic_bytes(name, T, H, d, s=2):
    """HBM bytes a kernel must move by the survey's definition: the forward reads q, k, v and
    writes o (4 T H d s); the backward reads q, k, v, dO and writes dq, dk, dv (7 T H d s), split
    between the passes as dK/dV: q, k, v, dO in, dk, dv out (6 T H d s) and dQ: k in, dq out
    (2 T H d s).  The stored dS (2 bytes per visible pair, written by dK/dV and read by dQ) is not
    algorithmic; it is reported as a separate overhead."""
    return {"fwd": 4, "bwd_dkdv": 6, "bwd_dq": 2}[name] * T * H * d * s


def roofline(kern, pairs, T, H, d, peaks=None):
    name = max(kern, key=kern.get)
    flops = pairs * FLOPS_PER_PAIR_D[name] * d
    achieved = flops / (kern[name] * 1e-3) / 1e12
    traffic = measured_traffic(name)
    alg = algorithmic_bytes(name, T, H, d)
    ds_bytes = 2 * pairs if name in ("bwd_dkdv", "bwd_dq") else 0
    r = {"kernel": name, "bound": "mfma", "achieved": round(achieved, 2),
         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
         "traffic": traffic,
         "algorithmic_flops_per_launch": flops,
         "per_unit": f"{FLOPS_PER_PAIR_D[name]}*d flops per visible pair per head",
         "algorithmic_bytes": alg,
         "stored_ds_overhead_bytes": ds_bytes,
         "traffic_over_algorithmic": round(traffic / alg, 2) if traffic else None}
    if peaks and peaks.get("bf16_gemm_tflops"):
        r["frac_of_measured_gemm_peak"] = round(achieved / peaks["bf16_gemm_tflops"], 4)
    return r


def measure_peaks(torch):
    """Attainable rates measured on this GPU in the same run: a 1 GiB device-to-device copy
    (bytes read + written per second) and a bf16 8192^3 matrix product through torch (the
    vendor BLAS), as empirical ceilings next to the published peaks."""
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    timer = Timer(torch)
    for _ in range(3):
        b.copy_(a)
    for _ in range(10):
        timer.record("copy", lambda: b.copy_(a))
    torch.cuda.synchronize()
    copy_ms = float(np.median(timer.ms("copy")))
    del a, b
    n = 8192
    x = torch.randn((n, n), device="cuda:0").to(torch.bfloat16)
    y = torch.randn((n, n), device="cuda:0").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(x, y)
    for _ in range(10):
        timer.record("gemm", lambda: torch.matmul(x, y))
    torch.cuda.synchronize()
    gemm_ms = float(np.median(timer.ms("gemm")))
    del x, y
    # the floor of the event timing itself: a one-element kernel, timed alone and back to back
    z = torch.zeros(1, device="cuda:0")
    tiny = lambda: z.add_(1.0)
    for _ in range(10):
        tiny()
    for _ in range(20):
        timer.record("tiny", tiny)
    torch.cuda.synchronize()
    return {"copy_GBps": round(2 * (1 << 30) / copy_ms / 1e6, 1),
            "bf16_gemm_tflops": round(2 * n ** 3 / gemm_ms / 1e9, 1),
            "tiny_kernel_ms": round(float(np.median(timer.ms("tiny"))), 4),
            "tiny_kernel_back_to_back_ms": round(back_to_back_ms(torch, tiny), 4),
            "how": "1 GiB device copy (read + write bytes); torch.matmul bf16 8192^3; a one-element "
                   "kernel timed like the forward workloads (alone, and 50 back to back); medians "
                   "of 10 or 20"}


def back_to_back_ms(torch, call, reps=50):
    """Time per call of `reps` calls queued back to back between two events: what a call
    occupies the GPU when the launches overlap (latency-bound workloads)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def pctl(ms):
    return {"median": round(float(np.median(ms)), 4), "p10": round(float(np.percentile(ms, 10)), 4),
            "p90": round(float(np.percentile(ms, 90)), 4)}


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
        esize = 4 if w["dtype"] == "fp32" else 2
        nbytes = T * H * d * esize * 4 + (T * 8 if w.get("timestamps") is not None else 0)
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
    b2b = None if cold else round(back_to_back_ms(torch, call), 4)
    plan.close()
    return {"ms_median": round(med, 4), "ms_p10": round(float(np.percentile(ms, 10)), 4),
            "ms_p90": round(float(np.percentile(ms, 90)), 4), "ms_back_to_back": b2b,
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
    b2b = round(back_to_back_ms(torch, call), 4)
    plan.close()
    return {"ms_median": round(med, 4), "ms_back_to_back": b2b, "tflops": round(flops / med / 1e9, 2),
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


ONLY = ("long_fwdbwd", "tiny_fp32", "ranking_fwd", "longtail_fwd", "layer_fwd", "layer_bwd",
        "cached_scoring", "stochastic_length")


def profile_md(folder, out):
    """Markdown summary of one profiled bench run (no GPU use).

    `folder` holds the rocprofv3 outputs of one workload, each pass in its own subfolder as the
    profile commands written into the summary produce them: trace/ (--kernel-trace --stats),
    fetch/ and write/ (--pmc FETCH_SIZE, --pmc WRITE_SIZE), copyf/ and copyw/ (the same counters
    on `bench.py --copy-calibration`), sq/ and sq2/ (issue counters), and bench.json, the JSON
    line the traced run printed.  Missing passes are left out of the summary."""
    import csv
    import glob

    def rows(sub, suffix):
        paths = sorted(glob.glob(os.path.join(folder, sub, f"*{suffix}")))
        return list(csv.DictReader(open(paths[0]))) if paths else []

    def short(name):
        return name.replace("hstu::(anonymous namespace)::", "").replace("(hstu::AttnParams)", "") \
                   .replace("(hstu::GemmArgs)", "").replace("void ", "")

    bench = {}
    bj = os.path.join(folder, "bench.json")
    if os.path.exists(bj):
        lines = [x for x in open(bj) if x.startswith("{")]
        bench = json.loads(lines[-1]) if lines else {}
    only = bench.get("only", HEADLINE)
    flags = f"--only {only} --steps 5 --warmup 2"
    L = [f"# Kernel profile: {only}", ""]
    if bench.get("config"):
        L += [f"Workload: {bench['config'].get('workload', '')}", ""]
    L += ["Commands (from the repository root on the GPU host; R = the repository root):", "", "```",
          "cd /tmp && export TMPDIR=/tmp",
          f"rocprofv3 --kernel-trace --stats -f csv -d P/trace -o trace -- python3 $R/bench.py {flags} > P/bench.json",
          f"rocprofv3 --pmc FETCH_SIZE -f csv -d P/fetch -o fetch -- python3 $R/bench.py {flags}",
          f"rocprofv3 --pmc WRITE_SIZE -f csv -d P/write -o write -- python3 $R/bench.py {flags}",
          "rocprofv3 --pmc FETCH_SIZE -f csv -d P/copyf -o copyf -- python3 $R/bench.py --copy-calibration",
          "rocprofv3 --pmc WRITE_SIZE -f csv -d P/copyw -o copyw -- python3 $R/bench.py --copy-calibration",
          f"rocprofv3 --pmc {' '.join(SQ1)} -f csv -d P/sq -o sq -- python3 $R/bench.py {flags}",
          f"rocprofv3 --pmc {' '.join(SQ2)} -f csv -d P/sq2 -o sq2 -- python3 $R/bench.py {flags}",
          "python3 $R/bench.py --profile-md P profiles/<this file>",
          "```", ""]
    trace = rows("trace", "_kernel_trace.csv")
    per = {}
    for r in trace:
        per.setdefault(r["Kernel_Name"], []).append(r)
    order = sorted(per, key=lambda k: -sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in per[k]))
    if trace:
        total = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace)
        L += ["## Kernel trace", "",
              "All dispatches of the traced run (warm-up steps included, so the average sits above the "
              "median; the live figures below cover the timed steps only). Register and LDS columns as "
              "rocprofv3 reports them.", "",
              "| kernel | dispatches | average (us) | median (us) | min (us) | max (us) | share | VGPR | AGPR | SGPR | LDS (B) | scratch (B/lane) |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for k in order[:12]:
            ds = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in per[k]]
            r0 = per[k][0]
            L.append(f"| `{short(k)[:100]}` | {len(ds)} | {np.mean(ds) / 1e3:.1f} | {np.median(ds) / 1e3:.1f} | {min(ds) / 1e3:.1f} | "
                     f"{max(ds) / 1e3:.1f} | {100 * sum(ds) / total:.1f}% | {r0['VGPR_Count']} | "
                     f"{r0['Accum_VGPR_Count']} | {r0['SGPR_Count']} | {r0['LDS_Block_Size']} | {r0['Scratch_Size']} |")
        L.append("")
    if bench:
        keep = {k: bench[k] for k in ("kernel_ms", "ms_per_step", "value", "roofline", "warm", "cold")
                if k in bench}
        L += ["Live HIP-event figures printed by the same traced run:", "", "```",
              json.dumps(keep, indent=1)[:3000], "```", ""]

    def counters(sub):
        out = {}
        for r in rows(sub, "_counter_collection.csv"):
            out.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        return out

    fetch, write = counters("fetch"), counters("write")
    copyf, copyw = counters("copyf"), counters("copyw")
    if fetch and write and copyf and copyw:
        def scale(c, name):
            v = [x for k, d in c.items() if "copyBuffer" in k for x in d.get(name, [])]
            return (1 << 30) / (1024.0 * float(np.median(v)))
        fs, ws = scale(copyf, "FETCH_SIZE"), scale(copyw, "WRITE_SIZE")
        L += ["## HBM traffic per dispatch", "",
              f"FETCH_SIZE and WRITE_SIZE (KiB) scaled by a 1 GiB device copy profiled the same way: "
              f"{1024 * fs:.0f} bytes per KiB read, {1024 * ws:.0f} per KiB written.", "",
              "| kernel | dispatches | HBM read (MB) | HBM write (MB) |", "|---|---|---|---|"]
        for k in order[:8]:
            if k in fetch and k in write:
                L.append(f"| `{short(k)[:100]}` | {len(fetch[k]['FETCH_SIZE'])} | "
                         f"{1024 * fs * np.mean(fetch[k]['FETCH_SIZE']) / 1e6:.2f} | "
                         f"{1024 * ws * np.mean(write[k]['WRITE_SIZE']) / 1e6:.2f} |")
        L.append("")
    sq = counters("sq")
    for k, d in counters("sq2").items():
        sq.setdefault(k, {}).update(d)
    if sq:
        names = [k for k in order[:4] if k in sq]
        L += ["## Issue counters per dispatch", "",
              "| counter | " + " | ".join(f"`{short(k)[:40]}`" for k in names) + " |",
              "|---|" + "---|" * len(names)]
        for c in SQ1 + SQ2:
            L.append(f"| {c} | " + " | ".join(f"{np.mean(sq[k].get(c, [0])):.3g}" for k in names) + " |")
        def ratio(k, a, b):
            x, y = np.mean(sq[k].get(a, [0])), np.mean(sq[k].get(b, [0]))
            return f"{x / y:.2f}" if y else "-"
        for a, b in (("SQ_INSTS_VALU", "SQ_INSTS_MFMA"), ("SQ_INSTS_SALU", "SQ_INSTS_MFMA"),
                     ("SQ_INSTS_LDS", "SQ_INSTS_MFMA"), ("SQ_WAIT_ANY", "SQ_WAVE_CYCLES")):
            L.append(f"| {a} / {b} | " + " | ".join(ratio(k, a, b) for k in names) + " |")
        L.append("")
    with open(out, "w") as f:
        f.write("\n".join(L) + "\n")
    print(out)


SQ1 = ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
       "SQ_INSTS_LDS", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT"]
SQ2 = ["SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_INST_LEVEL_VMEM", "SQ_ACTIVE_INST_VALU",
       "SQ_ACTIVE_INST_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU", "SQ_BUSY_CU_CYCLES"]


def run_only(args, torch, hj, runner, hs):
    """One workload alone (for profiling it on its own): prints its figures as one JSON line."""
    name = args.only
    if name == "long_fwdbwd":
        w = hs.make_workload(HEADLINE)
        r = bench_headline(args, torch, hj, runner, w)
        res = {"kernel_ms": {k: round(v, 4) for k, v in r["kern"].items()},
               "ms_per_step": round(r["ms_step"], 4),
               "value": round(r["flops"] / (r["ms_step"] * 1e-3) / 1e12, 2),
               "step_event_ms": pctl(r["step_ms"]),
               "roofline": roofline(r["kern"], r["pairs"], w["total_tokens"], w["heads"], w["d"]),
               "config": {"workload": describe(w)}}
    elif name == "layer_bwd":
        res = bench_layer_bwd(torch, hj, runner, iters=args.steps)
    elif name == "cached_scoring":
        res = bench_cached(torch, hj, runner, iters=args.steps)
    elif name == "stochastic_length":
        res = bench_select(torch, hj, iters=args.steps)
    else:
        res = {"warm": bench_forward(torch, hj, runner, name, iters=args.steps)}
        if args.cold:
            res["cold"] = bench_forward(torch, hj, runner, name, iters=args.steps, cold=True)
        w = hs.make_workload(name)
        res["config"] = {"workload": describe(w)}
    res["only"] = name
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the forward-only workloads")
    ap.add_argument("--only", choices=ONLY,
                    help="run one workload alone (its figures only; for profiling it on its own)")
    ap.add_argument("--cold", action="store_true", help="with --only: also time cold-cache calls")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                         "COPY_WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter files into the per-kernel "
                         "HBM traffic record (no GPU use)")
    ap.add_argument("--profile-md", nargs=2, metavar=("FOLDER", "OUT"),
                    help="summarize the rocprofv3 outputs of one profiled workload as markdown "
                         "(no GPU use)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.profile_md:
        profile_md(*args.profile_md)
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
    if args.only:
        run_only(args, torch, hj, runner, hs)
        return

    w = hs.make_workload(HEADLINE)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w)
    r = bench_headline(args, torch, hj, runner, w)
    peaks = None if args.no_extra else measure_peaks(torch)
    T, H, d = w["total_tokens"], w["heads"], w["d"]
    value = r["flops"] / (r["ms_step"] * 1e-3) / 1e12
    step = pctl(r["step_ms"])
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
        # GPU time of each step (HIP events around its three launches); the wall-clock
        # ms_per_step above also holds the gaps between steps
        "step_event_ms": step,
        "step_event_tflops": {k: round(r["flops"] / (v * 1e-3) / 1e12, 2) for k, v in step.items()},
        "visible_pairs": r["pairs"],
        "flops_per_step": r["flops"],
        "bytes_per_step": {"forward": algorithmic_bytes("fwd", T, H, d),
                           "backward": 7 * T * H * d * 2,
                           "stored_ds_overhead": 2 * 2 * r["pairs"]},
        "kernel_ms": {k: round(v, 4) for k, v in r["kern"].items()},
        "kernel_sum_ms": round(r["gpu_ms"], 4),
        "kernel_only_tflops": round(r["flops"] / (r["gpu_ms"] * 1e-3) / 1e12, 2),
        "plan_host_ms": round(r["plan_ms"], 4),
        "roofline": roofline(r["kern"], r["pairs"], T, H, d, peaks),
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    if peaks:
        result["pct_of_measured_gemm_peak"] = round(100 * value / peaks["bf16_gemm_tflops"], 2)
    if not args.no_extra:
        extra = {"tiny_fp32": {"warm": bench_forward(torch, hj, runner, "tiny_fp32")}}
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
