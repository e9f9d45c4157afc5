"""Padded-dense numpy formulation of HSTU attention -- TEST INFRASTRUCTURE ONLY.

A second, independent way of writing the definitions in ``hstu_ref.c``, used only to pin the
loop oracle on tiny inputs.  It shares no code with the loops:

* the mask is assembled rule by rule from the token roles (context tokens are seen by every
  query; a history query sees its own past; a candidate sees every non-candidate token and
  itself; no candidate sees another candidate) -- page 1 section 2.1.2 ranking task and page 2
  section on the HSTU acceleration operator (composite causal + context/target mask);
* bucket ids come from a sorted list of bucket start points (every integer below 16, then the
  start of each quarter of each octave) and ``numpy.searchsorted``, not from bit arithmetic;
* the sequences are padded to N and handled as one dense (B, N, N) batch with ``einsum``.
"""
from __future__ import annotations

import numpy as np


def bucket_starts(max_exp: int = 62) -> np.ndarray:
    """Sorted first value of every bucket: 0..15, then 2^k * (1 + m/4) for k >= 4, m = 0..3."""
    starts = list(range(16))
    for k in range(4, max_exp + 1):
        for m in range(4):
            starts.append((1 << k) + m * (1 << (k - 2)))
    return np.asarray(starts, dtype=np.int64)


_STARTS = bucket_starts()


def bucket_table_lookup(x: np.ndarray) -> np.ndarray:
    """Bucket id of each non-negative int64 distance: index of the last start <= x, capped."""
    x = np.asarray(x, dtype=np.int64)
    idx = np.searchsorted(_STARTS, x, side="right") - 1
    return np.minimum(idx, 127)


def role_mask(n: int, num_contexts: int, num_targets: int, N: int) -> np.ndarray:
    """(N, N) boolean visibility for one sequence padded to N."""
    nc = max(0, min(num_contexts, n))
    nt = max(0, min(num_targets, n - nc))
    nh = n - nt
    m = np.zeros((N, N), dtype=bool)
    history_rows = range(0, nh)
    target_rows = range(nh, n)
    for i in history_rows:          # causal: a history token sees itself and everything before
        m[i, : i + 1] = True
    for i in target_rows:           # a candidate sees all non-candidates and itself only
        m[i, :nh] = True
        m[i, i] = True
    m[:n, :nc] = True               # context tokens are visible to every real query
    return m


def pad(x: np.ndarray, off: np.ndarray, N: int) -> np.ndarray:
    """(T, ...) jagged -> (B, N, ...) zero padded."""
    B = len(off) - 1
    out = np.zeros((B, N) + x.shape[1:], dtype=x.dtype)
    for b in range(B):
        n = off[b + 1] - off[b]
        out[b, :n] = x[off[b]: off[b + 1]]
    return out


def unpad(x: np.ndarray, off: np.ndarray) -> np.ndarray:
    B = len(off) - 1
    return np.concatenate([x[b, : off[b + 1] - off[b]] for b in range(B)], axis=0)


def dense_scores(w: dict, q=None, k=None):
    """Return (S, M, N): S (B, H, N, N) scores, M (B, 1, N, N) mask, N the padded length."""
    off = np.asarray(w["seq_offsets"], dtype=np.int64)
    B = len(off) - 1
    lengths = np.diff(off)
    N = int(w["max_seqlen"])
    H = int(w["heads"])
    q = np.asarray(w["q"] if q is None else q, np.float64)
    k = np.asarray(w["k"] if k is None else k, np.float64)
    qp, kp = pad(q, off, N), pad(k, off, N)                     # (B, N, H, d)
    S = float(w["alpha"]) * np.einsum("bihd,bjhd->bhij", qp, kp)
    pos = np.arange(N)
    if w.get("rab_pos") is not None:
        dist = np.abs(pos[:, None] - pos[None, :])
        S = S + np.asarray(w["rab_pos"], np.float64)[:, bucket_table_lookup(dist)][None]
    if w.get("rab_ts") is not None:
        ts = pad(np.asarray(w["timestamps"], np.int64), off, N)  # (B, N)
        dt = np.abs(ts[:, :, None] - ts[:, None, :])             # (B, N, N)
        tab = np.asarray(w["rab_ts"], np.float64)                # (H, 128)
        S = S + np.transpose(tab[:, bucket_table_lookup(dt)], (1, 0, 2, 3))
    nts = w.get("num_targets")
    M = np.stack([role_mask(int(lengths[b]), int(w.get("num_contexts", 0)),
                            int(nts[b]) if nts is not None else 0, N) for b in range(B)])
    return S, M[:, None], N


def attn_fwd(w: dict, q=None, k=None, v=None) -> np.ndarray:
    off = np.asarray(w["seq_offsets"], dtype=np.int64)
    S, M, N = dense_scores(w, q, k)
    silu = S / (1.0 + np.exp(-S))
    P = np.where(M, silu / float(N), 0.0)
    v = np.asarray(w["v"] if v is None else v, np.float64)
    vp = pad(v, off, N)
    O = np.einsum("bhij,bjhd->bihd", P, vp)
    return unpad(O, off)


def layer_fwd(w: dict, eps: float = 1e-5):
    """Full layer from library routines: matrix products, mean, var, and the dense attention."""
    x = np.asarray(w["x"], np.float64)
    H, d = int(w["heads"]), int(w["d"])
    Hd = H * d
    Z = x @ np.asarray(w["w1"], np.float64)
    Z = Z / (1.0 + np.exp(-Z))
    T = x.shape[0]
    U, V, Q, K = (Z[:, c * Hd:(c + 1) * Hd] for c in range(4))
    A = attn_fwd(w, Q.reshape(T, H, d), K.reshape(T, H, d), V.reshape(T, H, d)).reshape(T, Hd)
    G = (A - A.mean(axis=1, keepdims=True)) / np.sqrt(A.var(axis=1, keepdims=True) + eps) * U
    Y = G @ np.asarray(w["w2"], np.float64) + x
    return Y, A
