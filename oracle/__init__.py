"""fp64 CPU oracle for HSTU jagged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product (``hstu_jagged_pointwise_amd``) never does, and this
package never imports the product.

``hstu_ref.c`` holds the plain loop definitions (see its header for the formulas and the passages
they follow); this module compiles it with gcc and exposes it to numpy through ctypes.
``brute.py`` is a second, independent formulation (padded dense numpy) used to pin the loops.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hstu_ref.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "libhstu_ref.so")
_lib = None

# -march=x86-64-v3 rather than native: the library is built in one place and may run on another
# host.  -ffp-contract=off keeps every multiply and add rounded as written.
CFLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/_build/libhstu_ref.so``."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, i32, f64, p = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        common = [i64, i64, i64, i64, p, i64, i64, p, p, p, p, f64, p, p, p]
        lib.hstu_ref_bucket.argtypes = [i64]
        lib.hstu_ref_bucket.restype = i32
        lib.hstu_ref_visible.argtypes = [i64, i64, i64, i64, i64]
        lib.hstu_ref_visible.restype = i32
        lib.hstu_ref_count_pairs.argtypes = [i64, p, i64, p]
        lib.hstu_ref_count_pairs.restype = i64
        lib.hstu_ref_attn_fwd.argtypes = common + [p, i32]
        lib.hstu_ref_attn_fwd_rows.argtypes = common + [i64, p, p, p, i32]
        lib.hstu_ref_attn_bwd.argtypes = common + [p, p, p, p, p, p, i32]
        lib.hstu_ref_attn_bwd_rows.argtypes = common + [p, i64, p, p, p, p, p, i32]
        lib.hstu_ref_layer_fwd.argtypes = [i64, i64, i64, i64, p, i64, i64, p, p, p, p, f64,
                                           p, p, p, f64, p, p, i32]
        lib.hstu_ref_layer_bwd.argtypes = [i64, i64, i64, i64, p, i64, i64, p, p, p, p, f64,
                                           p, p, p, p, f64, p, p, p, p, p, i32]
        lib.hstu_ref_attn_fwd_cached.argtypes = [i64, i64, i64, p, p, i64, p, p, p, p, f64,
                                                 p, p, p, p, p, p, i32]
        lib.hstu_ref_num_threads.restype = i32
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _i64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int64)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def num_threads() -> int:
    return int(_load().hstu_ref_num_threads())


def bucket(x: int) -> int:
    return int(_load().hstu_ref_bucket(int(x)))


def visible(n: int, num_contexts: int, num_targets: int, i: int, j: int) -> bool:
    return bool(_load().hstu_ref_visible(n, num_contexts, num_targets, i, j))


def count_pairs(seq_offsets, num_contexts: int, num_targets=None) -> int:
    off = _i64(seq_offsets)
    nt = _i32(num_targets)
    return int(_load().hstu_ref_count_pairs(len(off) - 1, _ptr(off), num_contexts, _ptr(nt)))


class _Args:
    """Holds contiguous copies of one problem's inputs for the C calls."""

    def __init__(self, w: dict, q=None, k=None, v=None):
        self.off = _i64(w["seq_offsets"])
        self.B = len(self.off) - 1
        self.H = int(w["heads"])
        self.nt = _i32(w.get("num_targets"))
        self.ts = _i64(w.get("timestamps"))
        self.rp = _f64(w.get("rab_pos"))
        self.rt = _f64(w.get("rab_ts"))
        if self.rt is not None and self.ts is None:
            raise ValueError("a time bias needs timestamps")
        self.q = _f64(w["q"] if q is None else q)
        self.k = _f64(w["k"] if k is None else k)
        self.v = _f64(w["v"] if v is None else v)
        self.dqk = self.q.shape[-1]
        self.dv = self.v.shape[-1]
        self.T = int(self.off[-1])
        self.head = [self.B, self.H, self.dqk, self.dv, _ptr(self.off), int(w["max_seqlen"]),
                     int(w.get("num_contexts", 0)), _ptr(self.nt), _ptr(self.ts), _ptr(self.rp),
                     _ptr(self.rt), float(w["alpha"]), _ptr(self.q), _ptr(self.k), _ptr(self.v)]


def attn_fwd(w: dict, q=None, k=None, v=None, nthreads: int = 0) -> np.ndarray:
    """O = sum_j vis * SiLU(S_ij) / N * v_j for every (token, head); shape (T, H, dv), fp64."""
    a = _Args(w, q, k, v)
    out = np.zeros((a.T, a.H, a.dv), np.float64)
    _load().hstu_ref_attn_fwd(*a.head, _ptr(out), nthreads)
    return out


def attn_fwd_rows(w: dict, row_tok, row_head, nthreads: int = 0) -> np.ndarray:
    """Forward output for selected (token, head) rows; shape (nrows, dv)."""
    a = _Args(w)
    rt, rh = _i64(row_tok), _i64(row_head)
    out = np.zeros((len(rt), a.dv), np.float64)
    _load().hstu_ref_attn_fwd_rows(*a.head, len(rt), _ptr(rt), _ptr(rh), _ptr(out), nthreads)
    return out


def attn_fwd_cached(w: dict, nthreads: int = 0) -> np.ndarray:
    """Candidate rows scored against cached history keys and values (see hstu_ref.c); w holds
    cand_offsets / cache_offsets, q, k, v (candidates), k_cache, v_cache, timestamps (candidates),
    cache_timestamps and the bias tables.  Returns (T_cand, H, d), fp64."""
    co, ho = _i64(w["cand_offsets"]), _i64(w["cache_offsets"])
    q, k, v = _f64(w["q"]), _f64(w["k"]), _f64(w["v"])
    kc, vc = _f64(w["k_cache"]), _f64(w["v_cache"])
    B, H, d = len(co) - 1, int(w["heads"]), int(w["d"])
    ts, tsc = _i64(w.get("timestamps")), _i64(w.get("cache_timestamps"))
    rp, rt = _f64(w.get("rab_pos")), _f64(w.get("rab_ts"))
    out = np.zeros((int(co[-1]), H, d))
    _load().hstu_ref_attn_fwd_cached(B, H, d, _ptr(co), _ptr(ho), int(w["max_seqlen"]), _ptr(ts),
                                     _ptr(tsc), _ptr(rp), _ptr(rt), float(w["alpha"]), _ptr(q),
                                     _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(out), nthreads)
    return out


def jagged_select(src, src_offsets, dst_offsets, keep_start=None) -> np.ndarray:
    """Stochastic Length compaction (page 1 section 2.1.3, algorithm-level optimisation: each
    training sequence is cut to a randomly drawn length before the encoder runs).  Sequence b
    keeps the dst_offsets[b + 1] - dst_offsets[b] consecutive tokens starting at keep_start[b]
    within it (default: the most recent ones, i.e. its last tokens), in order; the result is the
    jagged tensor of the kept tokens.  Plain slicing of the rows."""
    so, do = np.asarray(src_offsets, np.int64), np.asarray(dst_offsets, np.int64)
    src = np.asarray(src)
    out = np.zeros((int(do[-1]),) + src.shape[1:], dtype=src.dtype)
    for b in range(len(so) - 1):
        n, m = so[b + 1] - so[b], do[b + 1] - do[b]
        st = n - m if keep_start is None else int(keep_start[b])
        assert 0 <= st and st + m <= n, "window outside the sequence"
        out[do[b]:do[b + 1]] = src[so[b] + st:so[b] + st + m]
    return out


def attn_bwd(w: dict, dout=None, q=None, k=None, v=None, nthreads: int = 0) -> dict:
    """Gradients of sum(dout * O) w.r.t. q, k, v and the two bias tables (fp64)."""
    a = _Args(w, q, k, v)
    do = _f64(w["dout"] if dout is None else dout)
    dq = np.zeros((a.T, a.H, a.dqk)); dk = np.zeros((a.T, a.H, a.dqk))
    dvv = np.zeros((a.T, a.H, a.dv))
    drp = np.zeros((a.H, 128)) if a.rp is not None else None
    drt = np.zeros((a.H, 128)) if a.rt is not None else None
    _load().hstu_ref_attn_bwd(*a.head, _ptr(do), _ptr(dq), _ptr(dk), _ptr(dvv), _ptr(drp),
                              _ptr(drt), nthreads)
    return dict(dq=dq, dk=dk, dv=dvv, drab_pos=drp, drab_ts=drt)


def attn_bwd_rows(w: dict, row_tok, row_head, dout=None, nthreads: int = 0) -> dict:
    """dq of the selected rows as queries and dk, dv of the same rows as keys."""
    a = _Args(w)
    do = _f64(w["dout"] if dout is None else dout)
    rt, rh = _i64(row_tok), _i64(row_head)
    dq = np.zeros((len(rt), a.dqk)); dk = np.zeros((len(rt), a.dqk)); dvv = np.zeros((len(rt), a.dv))
    _load().hstu_ref_attn_bwd_rows(*a.head, _ptr(do), len(rt), _ptr(rt), _ptr(rh), _ptr(dq),
                                   _ptr(dk), _ptr(dvv), nthreads)
    return dict(dq=dq, dk=dk, dv=dvv)


def layer_fwd(w: dict, eps: float = 1e-5, nthreads: int = 0):
    """Y = (LayerNorm(A) * U) W2 + X with Q, K, V, U from SiLU(X W1); returns (Y, A)."""
    off = _i64(w["seq_offsets"])
    B, H, d, D = len(off) - 1, int(w["heads"]), int(w["d"]), int(w["layer_dim"])
    T = int(off[-1])
    x, w1, w2 = _f64(w["x"]), _f64(w["w1"]), _f64(w["w2"])
    nt, ts = _i32(w.get("num_targets")), _i64(w.get("timestamps"))
    rp, rt = _f64(w.get("rab_pos")), _f64(w.get("rab_ts"))
    y = np.zeros((T, D)); attn = np.zeros((T, H * d))
    _load().hstu_ref_layer_fwd(B, H, d, D, _ptr(off), int(w["max_seqlen"]),
                               int(w.get("num_contexts", 0)), _ptr(nt), _ptr(ts), _ptr(rp),
                               _ptr(rt), float(w["alpha"]), _ptr(x), _ptr(w1), _ptr(w2), eps,
                               _ptr(y), _ptr(attn), nthreads)
    return y, attn


def layer_bwd(w: dict, dy=None, eps: float = 1e-5, nthreads: int = 0) -> dict:
    """Gradients of sum(dy * Y) for Y = layer_fwd(w): dx (T, D), dw1 (D, 4Hd), dw2 (Hd, D) and the
    bias-table gradients (H, 128) when the tables are present; fp64."""
    off = _i64(w["seq_offsets"])
    B, H, d, D = len(off) - 1, int(w["heads"]), int(w["d"]), int(w["layer_dim"])
    T = int(off[-1])
    x, w1, w2 = _f64(w["x"]), _f64(w["w1"]), _f64(w["w2"])
    g = _f64(w["dy"] if dy is None else dy)
    nt, ts = _i32(w.get("num_targets")), _i64(w.get("timestamps"))
    rp, rt = _f64(w.get("rab_pos")), _f64(w.get("rab_ts"))
    dx = np.zeros((T, D)); dw1 = np.zeros((D, 4 * H * d)); dw2 = np.zeros((H * d, D))
    drp = np.zeros((H, 128)) if rp is not None else None
    drt = np.zeros((H, 128)) if rt is not None else None
    _load().hstu_ref_layer_bwd(B, H, d, D, _ptr(off), int(w["max_seqlen"]),
                               int(w.get("num_contexts", 0)), _ptr(nt), _ptr(ts), _ptr(rp),
                               _ptr(rt), float(w["alpha"]), _ptr(x), _ptr(w1), _ptr(w2), _ptr(g),
                               eps, _ptr(dx), _ptr(dw1), _ptr(dw2), _ptr(drp), _ptr(drt), nthreads)
    return dict(dx=dx, dw1=dw1, dw2=dw2, drab_pos=drp, drab_ts=drt)
