"""Seeded synthetic inputs for HSTU jagged attention.

This module only draws random inputs; it holds none of the method's arithmetic (no mask, no
bucketing, no attention).  Both the fp64 oracle (``oracle/``) and the HIP path
(``hstu_jagged_pointwise_amd``) consume what it produces, so neither depends on the other.

Workloads follow the shapes the pages describe for generative-recommender user histories:
jagged sequences stored back to back with start offsets (TorchRec KeyedJaggedTensor layout,
page 1 section 3.1.2), mostly short sequences with a few long ones (page 1 section 2.1.3,
"sparse optimisation"), one timestamp per token (page 1 section 2.1.2, the sequential
transduction formulation), and candidate items appended at the end of each sequence (page 1
section 2.1.2, ranking task).

Recipe (one ``numpy.random.default_rng(seed)`` per workload, draws in this order):
  1. sequence lengths;
  2. per sequence, timestamps = base + cumsum(max(1, ceil(Exponential(mean 3600 s))));
  3. relative-bias tables, position table then time table, each N(0, 0.02^2) of shape (H, 128);
  4. q, k, v each N(0, 0.5^2) of shape (T, H, d)  -- or, for the layer workload, X ~ N(0, 1) of
     shape (T, D), W1 ~ N(0, 0.02^2) of shape (D, 4*H*d), W2 ~ N(0, 0.02^2) of shape (H*d, D);
  5. for the forward+backward workload, the upstream gradient dO ~ N(0, 1) of shape (T, H, d);
     for a layer backward, dY ~ N(0, 1) of shape (T, D).
bf16 workloads round every floating-point tensor except the bias tables to bf16 (round to
nearest even, done by torch) and return the rounded values as float32 arrays, so both sides see
the same numbers.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np

TIME_BASE = 1_700_000_000  # seconds; large enough that timestamps need 64-bit storage
NUM_BUCKETS = 128


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    dtype: str                 # "fp32" or "bf16"
    batch: int
    heads: int
    d: int
    lengths: str               # "fixed", "uniform", "lognormal"
    len_args: tuple
    num_contexts: int = 0
    num_targets: int = 0
    rab: bool = False
    layer_dim: int = 0         # D for the full-layer workload, else 0
    backward: bool = False
    alpha: Optional[float] = None  # default 1/sqrt(d)
    max_seqlen: Optional[int] = None  # default max generated length


# The five workloads, in order: tiny fp32 check, ranking-shaped forward, long-tail forward,
# full layer forward, long-sequence forward+backward.
WORKLOADS: Dict[str, WorkloadSpec] = {
    "tiny_fp32": WorkloadSpec("tiny_fp32", "fp32", 4, 2, 32, "fixed", ((7, 16, 33, 64),),
                              max_seqlen=64),
    "ranking_fwd": WorkloadSpec("ranking_fwd", "bf16", 32, 4, 64, "uniform", (16, 256), rab=True),
    "longtail_fwd": WorkloadSpec("longtail_fwd", "bf16", 128, 4, 128, "lognormal",
                                 (5.0, 1.0, 8, 4096), num_targets=16, rab=True),
    "layer_fwd": WorkloadSpec("layer_fwd", "bf16", 64, 4, 128, "lognormal", (5.3, 0.8, 16, 1024),
                              num_contexts=4, num_targets=16, rab=True, layer_dim=512),
    "long_fwdbwd": WorkloadSpec("long_fwdbwd", "bf16", 16, 8, 128, "uniform", (1024, 8192),
                                num_contexts=8, num_targets=64, rab=True, backward=True),
}
WORKLOAD_ORDER = ["tiny_fp32", "ranking_fwd", "longtail_fwd", "layer_fwd", "long_fwdbwd"]


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even) and return them widened back to float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def draw_lengths(rng: np.random.Generator, spec: WorkloadSpec, batch: int) -> np.ndarray:
    kind, args = spec.lengths, spec.len_args
    if kind == "fixed":
        return np.asarray(args[0], dtype=np.int64)
    if kind == "uniform":
        lo, hi = args
        return rng.integers(lo, hi + 1, batch).astype(np.int64)  # inclusive bounds
    if kind == "lognormal":
        mu, sigma, lo, hi = args
        return np.clip(np.rint(rng.lognormal(mu, sigma, batch)), lo, hi).astype(np.int64)
    raise ValueError(kind)


def draw_timestamps(rng: np.random.Generator, lengths: Sequence[int]) -> np.ndarray:
    parts = []
    for n in lengths:
        gaps = np.maximum(1, np.ceil(rng.exponential(3600.0, int(n)))).astype(np.int64)
        parts.append(TIME_BASE + np.cumsum(gaps))
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def offsets_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    """Start of each sequence in the packed token dimension, plus the total at the end."""
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return off


def make_inputs(lengths: Sequence[int], heads: int, d: int, *, dtype: str = "bf16", seed: int = 0,
                rab: bool = True, num_contexts: int = 0, num_targets: int = 0,
                max_seqlen: Optional[int] = None, alpha: Optional[float] = None,
                layer_dim: int = 0, backward: bool = False,
                rng: Optional[np.random.Generator] = None, name: str = "custom") -> dict:
    """Draw one batch for explicit lengths (steps 2-5 of the recipe)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lengths = np.asarray(lengths, dtype=np.int64)
    B = len(lengths)
    T = int(lengths.sum())
    off = offsets_from_lengths(lengths)
    out = dict(name=name, dtype=dtype, batch=B, heads=heads, d=d, lengths=lengths, seq_offsets=off,
               total_tokens=T, num_contexts=int(num_contexts),
               num_targets=np.full(B, int(num_targets), dtype=np.int32),
               max_seqlen=int(max_seqlen if max_seqlen is not None
                              else (int(lengths.max()) if B else 0)),
               alpha=float(alpha if alpha is not None else 1.0 / math.sqrt(d)),
               timestamps=None, rab_pos=None, rab_ts=None)
    rnd = round_bf16 if dtype == "bf16" else (lambda a: np.asarray(a, dtype=np.float32))
    if rab:
        out["timestamps"] = draw_timestamps(rng, lengths)
        out["rab_pos"] = rng.normal(0.0, 0.02, (heads, NUM_BUCKETS)).astype(np.float32)
        out["rab_ts"] = rng.normal(0.0, 0.02, (heads, NUM_BUCKETS)).astype(np.float32)
    if layer_dim:
        D, Hd = layer_dim, heads * d
        out["layer_dim"] = D
        out["x"] = rnd(rng.normal(0.0, 1.0, (T, D)).astype(np.float32))
        out["w1"] = rnd(rng.normal(0.0, 0.02, (D, 4 * Hd)).astype(np.float32))
        out["w2"] = rnd(rng.normal(0.0, 0.02, (Hd, D)).astype(np.float32))
    else:
        for key in ("q", "k", "v"):
            out[key] = rnd(rng.normal(0.0, 0.5, (T, heads, d)).astype(np.float32))
    if backward:
        if layer_dim:
            out["dy"] = rnd(rng.normal(0.0, 1.0, (T, layer_dim)).astype(np.float32))
        else:
            out["dout"] = rnd(rng.normal(0.0, 1.0, (T, heads, d)).astype(np.float32))
    return out


def make_cached_inputs(cache_lengths: Sequence[int], num_cands: Sequence[int], heads: int, d: int,
                       *, seed: int = 0, rab: bool = True, max_seqlen: Optional[int] = None,
                       alpha: Optional[float] = None, name: str = "cached") -> dict:
    """Candidate scoring against a key/value cache, bf16: per user a cached history of
    cache_lengths[b] tokens (k_cache, v_cache, cache_timestamps) and num_cands[b] candidates
    (q, k, v, timestamps) that follow it.  Timestamps run through history then candidates as in
    step 2 of the recipe; then the bias tables, the cached k and v, then candidate q, k, v, all
    drawn as in steps 3-4."""
    rng = np.random.default_rng(seed)
    hl = np.asarray(cache_lengths, dtype=np.int64)
    mc = np.asarray(num_cands, dtype=np.int64)
    B = len(hl)
    full = draw_timestamps(rng, hl + mc) if rab else None
    out = dict(name=name, dtype="bf16", batch=B, heads=heads, d=d,
               cache_offsets=offsets_from_lengths(hl), cand_offsets=offsets_from_lengths(mc),
               total_tokens=int(mc.sum()), cache_tokens=int(hl.sum()),
               max_seqlen=int(max_seqlen if max_seqlen is not None
                              else (int((hl + mc).max()) if B else 1)),
               alpha=float(alpha if alpha is not None else 1.0 / math.sqrt(d)),
               timestamps=None, cache_timestamps=None, rab_pos=None, rab_ts=None)
    if rab:
        fo = offsets_from_lengths(hl + mc)
        out["cache_timestamps"] = np.concatenate(
            [full[fo[b]:fo[b] + hl[b]] for b in range(B)] or [np.zeros(0, np.int64)])
        out["timestamps"] = np.concatenate(
            [full[fo[b] + hl[b]:fo[b + 1]] for b in range(B)] or [np.zeros(0, np.int64)])
        out["rab_pos"] = rng.normal(0.0, 0.02, (heads, NUM_BUCKETS)).astype(np.float32)
        out["rab_ts"] = rng.normal(0.0, 0.02, (heads, NUM_BUCKETS)).astype(np.float32)
    Tc, T = int(hl.sum()), int(mc.sum())
    for key, n in (("k_cache", Tc), ("v_cache", Tc), ("q", T), ("k", T), ("v", T)):
        out[key] = round_bf16(rng.normal(0.0, 0.5, (n, heads, d)).astype(np.float32))
    return out


def make_cached_workload(seed: int = 0, batch: int = 128, num_cands: int = 64) -> dict:
    """Candidate scoring at ranking scale: per user a cached history with the long-tail length
    mix (lognormal(5, 1) clipped to [8, 4096], as the long-tail forward workload), 64
    candidates, 4 heads of width 128, position and time bias."""
    rng = np.random.default_rng(seed)
    spec = WORKLOADS["longtail_fwd"]
    hl = draw_lengths(rng, spec, batch)
    return make_cached_inputs(hl, np.full(batch, num_cands), spec.heads, spec.d,
                              seed=seed + 1, name="cached_scoring")


def make_workload(name: str, seed: int = 0, *, batch: Optional[int] = None,
                  len_cap: Optional[int] = None) -> dict:
    """Draw one of the named workloads.

    ``batch`` and ``len_cap`` shrink a workload for tests the oracle must finish quickly: the
    length distribution is drawn as specified for ``batch`` sequences and then clipped to
    ``len_cap``.  ``max_seqlen`` follows the (clipped) maximum unless the workload fixes it.
    """
    spec = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    B = spec.batch if batch is None else batch
    lengths = draw_lengths(rng, spec, B)
    if spec.lengths == "fixed" and batch is not None:
        lengths = lengths[:batch]
    if len_cap is not None:
        lengths = np.minimum(lengths, len_cap)
    max_seqlen = spec.max_seqlen if spec.max_seqlen is not None else None
    w = make_inputs(lengths, spec.heads, spec.d, dtype=spec.dtype, rab=spec.rab,
                    num_contexts=spec.num_contexts, num_targets=spec.num_targets,
                    max_seqlen=max_seqlen, alpha=spec.alpha, layer_dim=spec.layer_dim,
                    backward=spec.backward, rng=rng, name=name)
    return w
