"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what pins which part:
  * bucket function: start points of each bucket built from the definition's intent (16 exact
    buckets, then quarter octaves) and closed-form values at powers of two;
  * mask: closed-form count of visible pairs, and a rule-by-rule padded mask (brute force);
  * scores and weights: identity-V read-out compared with scalar ``math`` evaluation;
  * aggregation: closed form with alpha = 0 and a constant bias (prefix sums), the worked
    KeyedJaggedTensor example printed on the pages, and the padded dense formulation;
  * invariants stated for the method: jagged == padded, future tokens never leak into earlier
    rows, candidates do not see each other, V = 0 gives 0, linearity in V;
  * backward: central finite differences and inner-product identities;
  * full layer: numpy matrix products, mean and var around the dense attention.
"""
import json
import math
import os

import numpy as np
import pytest

import hstu_synth as hs
import oracle
import oracle.brute as brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def silu(x):
    return x / (1.0 + math.exp(-x))


def small(lengths, H=2, d=8, seed=0, **kw):
    kw.setdefault("dtype", "fp32")
    return hs.make_inputs(lengths, H, d, seed=seed, **kw)


# ---- bucket function ------------------------------------------------------------------------

def test_bucket_identity_below_16():
    assert [oracle.bucket(x) for x in range(16)] == list(range(16))


def test_bucket_powers_of_two_and_quarters():
    # Each octave [2^k, 2^(k+1)) is split into four equal quarters, bucket 4k + m.
    for k in range(4, 31):
        for m in range(4):
            start = (1 << k) + m * (1 << (k - 2))
            assert oracle.bucket(start) == 4 * k + m
            assert oracle.bucket(start - 1) == 4 * k + m - 1
    assert oracle.bucket(1 << 31) == 124
    # saturation at the last bucket
    for x in [(1 << 32) - 1, 1 << 32, 1 << 40, (1 << 62) + 12345, (1 << 63) - 1]:
        assert oracle.bucket(x) == 127


def test_bucket_exhaustive_against_start_points():
    xs = np.arange(0, 1 << 17, dtype=np.int64)
    got = np.array([oracle.bucket(int(x)) for x in xs])
    np.testing.assert_array_equal(got, brute.bucket_table_lookup(xs))
    assert np.all(np.diff(got) >= 0)
    edges = []
    for k in range(1, 63):
        edges += [(1 << k) - 1, 1 << k, (1 << k) + 1, (1 << k) + (1 << max(k - 2, 0))]
    edges = np.array(edges, dtype=np.int64)
    got = np.array([oracle.bucket(int(x)) for x in edges])
    np.testing.assert_array_equal(got, brute.bucket_table_lookup(edges))


# ---- mask -----------------------------------------------------------------------------------

def closed_form_pairs(n, nc_arg, nt_arg):
    nc = min(nc_arg, n)
    nt = min(max(nt_arg, 0), n - nc)
    nh = n - nt
    return nc * nc + (nh * (nh + 1) - nc * (nc + 1)) // 2 + nt * (nh + 1)


def test_pair_count_closed_form():
    for n in range(0, 41):
        for nc in range(0, 7):
            for nt in range(0, 22, 3):
                off = np.array([0, n], np.int64)
                got = oracle.count_pairs(off, nc, np.array([nt], np.int32))
                assert got == closed_form_pairs(n, nc, nt), (n, nc, nt)


def test_mask_matches_role_rules():
    for n in [0, 1, 2, 5, 16, 23]:
        for nc in [0, 1, 3, 30]:
            for nt in [0, 1, 4, 30]:
                m = brute.role_mask(n, nc, nt, max(n, 1))
                for i in range(n):
                    for j in range(n):
                        assert oracle.visible(n, nc, nt, i, j) == m[i, j], (n, nc, nt, i, j)


def test_every_row_sees_its_diagonal():
    for n in range(1, 30):
        for nc in [0, 2, 40]:
            for nt in [0, 3, 40]:
                assert all(oracle.visible(n, nc, nt, i, i) for i in range(n))


# ---- forward --------------------------------------------------------------------------------

CASES = [
    dict(lengths=[5, 0, 17, 33, 1], rab=True, num_contexts=2, num_targets=4),
    dict(lengths=[9, 12], rab=False),
    dict(lengths=[40], rab=True, num_contexts=0, num_targets=39),
    dict(lengths=[3, 8], rab=True, num_contexts=10, num_targets=2),
    dict(lengths=[16, 15, 1], rab=True, num_contexts=4, num_targets=16),
    dict(lengths=[0, 0], rab=True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fwd_matches_padded_dense(case):
    w = small(**CASES[case], seed=case)
    a = oracle.attn_fwd(w)
    b = brute.attn_fwd(w) if w["total_tokens"] else np.zeros_like(a)
    assert a.shape == (w["total_tokens"], 2, 8)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_fwd_max_seqlen_larger_than_lengths():
    w = small([7, 4], rab=True, num_targets=2, max_seqlen=50)
    np.testing.assert_allclose(oracle.attn_fwd(w), brute.attn_fwd(w), rtol=0, atol=1e-12)


def test_closed_form_constant_bias():
    # alpha = 0 and a constant position bias c: every visible pair has weight SiLU(c)/N.
    c = 0.7
    for nc, nt in [(0, 0), (3, 0), (0, 5), (2, 4), (9, 9)]:
        w = small([11, 1, 20], H=1, d=3, seed=nc + nt, rab=False, num_contexts=nc,
                  num_targets=nt, alpha=0.0)
        w["rab_pos"] = np.full((1, 128), c, np.float64)
        out = oracle.attn_fwd(w)
        scale = silu(c) / w["max_seqlen"]
        v = w["v"].astype(np.float64)
        off = w["seq_offsets"]
        for b in range(len(off) - 1):
            s, n = off[b], off[b + 1] - off[b]
            vb = v[s:s + n, 0]
            ncb = min(nc, n); ntb = min(nt, n - ncb); nh = n - ntb
            pref = np.cumsum(vb, axis=0)
            for i in range(n):
                if i < ncb:
                    want = pref[ncb - 1]
                elif i < nh:
                    want = pref[i]
                else:
                    want = pref[nh - 1] + vb[i] if nh > 0 else vb[i]
                np.testing.assert_allclose(out[s + i, 0], scale * want, rtol=1e-13, atol=1e-15)


def test_kjt_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "kjt_example.json")))
    lengths = g["lengths"]
    off = hs.offsets_from_lengths(lengths)
    assert off.tolist() == g["offsets"]
    vals = np.asarray(g["values"], np.float64)
    assert [vals[off[b]:off[b + 1]].tolist() for b in range(len(lengths))] == g["groups"]
    c = 0.25
    N = max(lengths)
    T = len(vals)
    w = dict(seq_offsets=off, heads=1, max_seqlen=N, alpha=0.0, num_contexts=0,
             num_targets=np.zeros(len(lengths), np.int32), timestamps=None,
             rab_pos=np.full((1, 128), c), rab_ts=None,
             q=np.zeros((T, 1, 1)), k=np.zeros((T, 1, 1)), v=vals.reshape(T, 1, 1))
    out = oracle.attn_fwd(w)[:, 0, 0]
    want = silu(c) / N * np.asarray(g["causal_prefix_sums"], np.float64)
    np.testing.assert_allclose(out, want, rtol=1e-14)


def test_identity_v_reads_out_weights():
    # With v_j = e_j, row i of O is row i of P; check entries against scalar math.
    n = 21
    w = small([n], H=2, d=6, seed=7, rab=True, num_contexts=3, num_targets=5)
    H = 2
    eye = np.zeros((n, H, n))
    for j in range(n):
        eye[j, :, j] = 1.0
    O = oracle.attn_fwd(w, v=eye)
    ts = w["timestamps"]
    starts = brute.bucket_starts()
    nc, nt = 3, 5
    nh = n - nt
    for h in range(H):
        for i in range(n):
            for j in range(n):
                vis = (j < nc) or (i < nh and j <= i) or (i >= nh and (j < nh or j == i))
                if not vis:
                    assert O[i, h, j] == 0.0
                    continue
                dot = sum(float(w["q"][i, h, c]) * float(w["k"][j, h, c]) for c in range(6))
                bp = min(127, int(np.searchsorted(starts, abs(i - j), side="right")) - 1)
                bt = min(127, int(np.searchsorted(starts, abs(int(ts[i]) - int(ts[j])),
                                                  side="right")) - 1)
                s = w["alpha"] * dot + float(w["rab_pos"][h, bp]) + float(w["rab_ts"][h, bt])
                assert O[i, h, j] == pytest.approx(silu(s) / w["max_seqlen"], rel=1e-13, abs=1e-16)


def test_silu_special_values():
    # q.k = 0 and no bias: SiLU(0) = 0, so the output is exactly 0.
    w = small([6, 9], rab=False, num_targets=2)
    w["q"] = np.zeros_like(w["q"])
    assert np.all(oracle.attn_fwd(w) == 0.0)
    # alpha * q.k = 1 for a single pair (n = 1): weight is 1/(1 + e^-1) / N.
    w = dict(seq_offsets=np.array([0, 1]), heads=1, max_seqlen=4, alpha=0.5, num_contexts=0,
             num_targets=None, timestamps=None, rab_pos=None, rab_ts=None,
             q=np.array([[[2.0]]]), k=np.array([[[1.0]]]), v=np.array([[[3.0]]]))
    assert oracle.attn_fwd(w)[0, 0, 0] == pytest.approx(3.0 / (1.0 + math.exp(-1.0)) / 4, rel=1e-15)


# ---- invariants -----------------------------------------------------------------------------

def test_jagged_equals_each_sequence_alone():
    w = small([13, 2, 30, 7], seed=11, rab=True, num_contexts=2, num_targets=3, max_seqlen=40)
    full = oracle.attn_fwd(w)
    off = w["seq_offsets"]
    for b in range(4):
        s, e = off[b], off[b + 1]
        wb = dict(w)
        wb.update(seq_offsets=np.array([0, e - s]), num_targets=w["num_targets"][b:b + 1],
                  timestamps=w["timestamps"][s:e], q=w["q"][s:e], k=w["k"][s:e], v=w["v"][s:e])
        np.testing.assert_array_equal(oracle.attn_fwd(wb), full[s:e])


def test_future_tokens_do_not_leak():
    n, nc, nt = 30, 3, 6
    w = small([n], seed=5, rab=True, num_contexts=nc, num_targets=nt)
    base = oracle.attn_fwd(w)
    rng = np.random.default_rng(1)
    for j0 in [nc, 10, n - nt - 1, n - nt, n - 2, n - 1]:
        w2 = dict(w)
        for key in ("q", "k", "v"):
            a = w[key].copy()
            a[j0] = rng.normal(size=a[j0].shape)
            w2[key] = a
        ts = w["timestamps"].copy()
        ts[j0:] += 12345  # keep timestamps increasing while moving token j0 in time
        w2["timestamps"] = ts
        out = oracle.attn_fwd(w2)
        # rows before j0 are unchanged, except that a shifted timestamp of later tokens can
        # only matter to rows that see them: none of the rows i < j0 do
        np.testing.assert_array_equal(out[:j0], base[:j0])


def test_candidates_do_not_see_each_other():
    n, nt = 25, 7
    nh = n - nt
    w = small([n], seed=9, rab=True, num_targets=nt)
    base = oracle.attn_fwd(w)
    keep = nh + 2
    others = [t for t in range(nh, n) if t != keep]
    perm = list(np.random.default_rng(3).permutation(others))
    idx = list(range(n))
    for src, dst in zip(others, perm):
        idx[dst] = src
    w2 = dict(w)
    for key in ("q", "k", "v", "timestamps"):
        w2[key] = w[key][idx]
    out = oracle.attn_fwd(w2)
    np.testing.assert_array_equal(out[keep], base[keep])
    np.testing.assert_array_equal(out[:nh], base[:nh])


def test_zero_v_and_linearity():
    w = small([12, 19], seed=2, rab=True, num_contexts=1, num_targets=4)
    assert np.all(oracle.attn_fwd(w, v=np.zeros_like(w["v"])) == 0.0)
    v2 = np.random.default_rng(4).normal(size=w["v"].shape)
    lhs = oracle.attn_fwd(w, v=w["v"] + 2.0 * v2)
    rhs = oracle.attn_fwd(w) + 2.0 * oracle.attn_fwd(w, v=v2)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-14)


def test_rows_variant_matches_full():
    w = small([10, 33, 4], seed=8, rab=True, num_contexts=2, num_targets=5)
    full = oracle.attn_fwd(w)
    rt = np.array([0, 9, 10, 25, 42, 46, 45])
    rh = np.array([0, 1, 1, 0, 1, 0, 1])
    np.testing.assert_array_equal(oracle.attn_fwd_rows(w, rt, rh), full[rt, rh])


# ---- backward -------------------------------------------------------------------------------

def _loss(w, dout, **over):
    return float(np.sum(oracle.attn_fwd(w, **over) * dout))


def test_backward_finite_differences():
    w = small([6, 9], H=2, d=3, seed=21, rab=True, num_contexts=1, num_targets=3, max_seqlen=10)
    rng = np.random.default_rng(0)
    dout = rng.normal(size=(w["total_tokens"], 2, 3))
    g = oracle.attn_bwd(w, dout=dout)
    eps = 1e-6
    for name, key in (("dq", "q"), ("dk", "k"), ("dv", "v")):
        base = w[key].astype(np.float64)
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            p = base.copy(); p[idx] += eps
            m = base.copy(); m[idx] -= eps
            num[idx] = (_loss(w, dout, **{key: p}) - _loss(w, dout, **{key: m})) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-9)
    for name, key in (("drab_pos", "rab_pos"), ("drab_ts", "rab_ts")):
        base = w[key].astype(np.float64)
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            w2 = dict(w); p = base.copy(); p[idx] += eps; w2[key] = p
            w3 = dict(w); m = base.copy(); m[idx] -= eps; w3[key] = m
            num[idx] = (_loss(w2, dout) - _loss(w3, dout)) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-9)


def test_backward_identities():
    w = small([14, 3, 27], H=2, d=5, seed=4, rab=True, num_contexts=2, num_targets=4)
    dout = np.random.default_rng(1).normal(size=w["v"].shape)
    g = oracle.attn_bwd(w, dout=dout)
    O = oracle.attn_fwd(w)
    off = w["seq_offsets"]
    for b in range(3):
        s, e = off[b], off[b + 1]
        for h in range(2):
            assert np.sum(g["dv"][s:e, h] * w["v"][s:e, h]) == pytest.approx(
                np.sum(dout[s:e, h] * O[s:e, h]), rel=1e-12, abs=1e-15)
            assert np.sum(g["dq"][s:e, h] * w["q"][s:e, h]) == pytest.approx(
                np.sum(g["dk"][s:e, h] * w["k"][s:e, h]), rel=1e-12, abs=1e-15)
    np.testing.assert_allclose(g["drab_pos"].sum(axis=1), g["drab_ts"].sum(axis=1), rtol=1e-12)


def test_backward_constant_bias_reverse_cumsum():
    c, nt = -0.4, 3
    w = small([10], H=1, d=2, seed=6, rab=False, num_targets=nt, alpha=0.0)
    w["rab_pos"] = np.full((1, 128), c)
    dout = np.random.default_rng(2).normal(size=w["v"].shape)
    g = oracle.attn_bwd(w, dout=dout)
    n, nh = 10, 10 - nt
    scale = silu(c) / w["max_seqlen"]
    for j in range(n):
        if j < nh:   # seen by history rows i >= j and by every target row
            want = dout[j:nh, 0].sum(axis=0) + dout[nh:, 0].sum(axis=0)
        else:        # a target is seen only by itself
            want = dout[j, 0]
        np.testing.assert_allclose(g["dv"][j, 0], scale * want, rtol=1e-13)
    assert np.all(g["dq"] == 0.0) and np.all(g["dk"] == 0.0)


def test_backward_rows_variant_matches_full():
    w = small([10, 33, 4], seed=8, rab=True, num_contexts=2, num_targets=5, backward=True)
    g = oracle.attn_bwd(w)
    rt = np.array([0, 9, 10, 25, 42, 46, 45])
    rh = np.array([0, 1, 1, 0, 1, 0, 1])
    r = oracle.attn_bwd_rows(w, rt, rh)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(r[name], g[name][rt, rh], rtol=1e-13, atol=1e-16)


def test_backward_is_thread_count_independent():
    w = small([30, 17, 8, 25], seed=3, rab=True, num_targets=2, backward=True)
    a = oracle.attn_bwd(w, nthreads=1)
    b = oracle.attn_bwd(w, nthreads=4)
    for name in a:
        np.testing.assert_array_equal(a[name], b[name])


# ---- candidate scoring against cached history -----------------------------------------------

def _as_full_sequences(w, num_contexts=0, seed=0):
    """The same users as one jagged batch [history | candidates] with the candidates as targets;
    history queries (whose rows are not compared) are random."""
    rng = np.random.default_rng(seed)
    ho, co = w["cache_offsets"], w["cand_offsets"]
    H, d = w["heads"], w["d"]
    parts = {k: [] for k in ("q", "k", "v", "timestamps")}
    lengths, cand_rows = [], []
    pos = 0
    for b in range(w["batch"]):
        nh, m = ho[b + 1] - ho[b], co[b + 1] - co[b]
        parts["q"] += [rng.normal(size=(nh, H, d)), w["q"][co[b]:co[b + 1]]]
        parts["k"] += [w["k_cache"][ho[b]:ho[b + 1]], w["k"][co[b]:co[b + 1]]]
        parts["v"] += [w["v_cache"][ho[b]:ho[b + 1]], w["v"][co[b]:co[b + 1]]]
        if w["timestamps"] is not None:
            parts["timestamps"] += [w["cache_timestamps"][ho[b]:ho[b + 1]],
                                    w["timestamps"][co[b]:co[b + 1]]]
        cand_rows += list(range(pos + nh, pos + nh + m))
        lengths.append(nh + m)
        pos += nh + m
    full = dict(w, seq_offsets=hs.offsets_from_lengths(lengths), total_tokens=pos,
                num_contexts=num_contexts,
                num_targets=np.diff(co).astype(np.int32))
    for key, val in parts.items():
        full[key] = np.concatenate(val) if val else None
    if w["timestamps"] is None:
        full["timestamps"] = None
    return full, np.array(cand_rows, dtype=np.int64)


@pytest.mark.parametrize("rab", [True, False])
def test_cached_equals_target_rows_of_full_forward(rab):
    w = hs.make_cached_inputs([37, 1, 5, 130, 1], [4, 3, 0, 17, 1], 2, 8, seed=51, rab=rab)
    for key in ("q", "k", "v", "k_cache", "v_cache"):
        w[key] = w[key].astype(np.float64)
    got = oracle.attn_fwd_cached(w)
    # Leading contexts change nothing for candidates, who see the whole history anyway, as long
    # as the history is at least as long as the contexts (else candidates become contexts).
    for nc in (0, 1):
        full, rows = _as_full_sequences(w, num_contexts=nc)
        want = oracle.attn_fwd(full)[rows]
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)


def test_cached_closed_form_constant_bias():
    c = 0.3
    w = hs.make_cached_inputs([9, 0, 20], [3, 2, 5], 1, 4, seed=52, rab=False, alpha=0.0)
    # (a user without history: its candidates see only themselves)
    w["rab_pos"] = np.full((1, 128), c)
    got = oracle.attn_fwd_cached(w)
    scale = silu(c) / w["max_seqlen"]
    ho, co = w["cache_offsets"], w["cand_offsets"]
    for b in range(3):
        hist = w["v_cache"][ho[b]:ho[b + 1], 0].astype(np.float64).sum(axis=0)
        for r in range(co[b], co[b + 1]):
            np.testing.assert_allclose(got[r, 0], scale * (hist + w["v"][r, 0]), rtol=1e-12,
                                       atol=1e-15)


def test_cached_candidates_do_not_see_each_other():
    w = hs.make_cached_inputs([25, 40], [6, 5], 2, 8, seed=53)
    base = oracle.attn_fwd_cached(w)
    w2 = dict(w)
    for key in ("q", "k", "v"):
        w2[key] = w[key].copy()
    w2["timestamps"] = w["timestamps"].copy()
    # replace candidate 2 of user 0 entirely; the others must not change
    for key in ("q", "k", "v"):
        w2[key][2] = -w[key][2] + 0.5
    w2["timestamps"][2] += 1000
    got = oracle.attn_fwd_cached(w2)
    keep = [r for r in range(11) if r != 2]
    np.testing.assert_array_equal(got[keep], base[keep])
    assert not np.allclose(got[2], base[2])


# ---- Stochastic Length compaction -------------------------------------------------------------

def test_jagged_select_on_the_printed_example():
    # The KeyedJaggedTensor example printed on the pages, each sequence cut to its last
    # min(n, 2) tokens, then to one token at a chosen start; results written out by hand from
    # the printed grouping [[101, 102], [201, 202, 203], [1001], [1002, 1003]].
    with open(os.path.join(GOLDEN, "kjt_example.json")) as f:
        ex = json.load(f)
    vals = np.array(ex["values"], dtype=np.int64)[:, None]
    got = oracle.jagged_select(vals, ex["offsets"], [0, 2, 4, 5, 7])
    assert got[:, 0].tolist() == [101, 102, 202, 203, 1001, 1002, 1003]
    got = oracle.jagged_select(vals, ex["offsets"], [0, 1, 2, 3, 4], keep_start=[0, 1, 0, 1])
    assert got[:, 0].tolist() == [101, 202, 1001, 1003]
    got = oracle.jagged_select(vals, ex["offsets"], [0, 0, 0, 0, 0])
    assert got.shape == (0, 1)


def test_jagged_select_identity_and_rows():
    rng = np.random.default_rng(3)
    lengths = np.array([5, 0, 9, 1])
    off = hs.offsets_from_lengths(lengths)
    x = rng.normal(size=(int(off[-1]), 3, 4))
    np.testing.assert_array_equal(oracle.jagged_select(x, off, off), x)
    keep = np.minimum(lengths, 3)
    got = oracle.jagged_select(x, off, hs.offsets_from_lengths(keep))
    np.testing.assert_array_equal(got, np.concatenate([x[0:5][-3:], x[5:14][-3:], x[14:15]]))


# ---- full layer ----------------------------------------------------------------------------

def test_layer_matches_library_routines():
    w = hs.make_inputs([9, 1, 20], 2, 4, dtype="fp32", seed=12, rab=True, num_contexts=2,
                       num_targets=3, layer_dim=16)
    y, a = oracle.layer_fwd(w)
    yb, ab = brute.layer_fwd(w)
    np.testing.assert_allclose(a, ab, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y, yb, rtol=0, atol=1e-12)


def test_layer_backward_finite_differences():
    # Central differences of L = sum(dy * Y) through the (separately pinned) layer forward, for
    # every entry of x, w1, w2 and of both bias tables.  Weights are drawn large enough that the
    # attention, LayerNorm and gate terms all carry weight in the gradients.
    rng = np.random.default_rng(5)
    w = hs.make_inputs([5, 8], 2, 3, dtype="fp32", seed=31, rab=True, num_contexts=1,
                       num_targets=2, layer_dim=6, max_seqlen=9)
    w["w1"] = rng.normal(0.0, 0.6, w["w1"].shape)
    w["w2"] = rng.normal(0.0, 0.6, w["w2"].shape)
    w["rab_pos"] = rng.normal(0.0, 0.5, w["rab_pos"].shape)
    w["rab_ts"] = rng.normal(0.0, 0.5, w["rab_ts"].shape)
    dy = rng.normal(size=(w["total_tokens"], 6))
    g = oracle.layer_bwd(w, dy=dy)

    def loss(**over):
        return float(np.sum(oracle.layer_fwd(dict(w, **over))[0] * dy))

    eps = 1e-6
    for name, key in (("dx", "x"), ("dw1", "w1"), ("dw2", "w2"), ("drab_pos", "rab_pos"),
                      ("drab_ts", "rab_ts")):
        base = np.asarray(w[key], dtype=np.float64)
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            p = base.copy(); p[idx] += eps
            m = base.copy(); m[idx] -= eps
            num[idx] = (loss(**{key: p}) - loss(**{key: m})) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8, err_msg=name)
    assert np.all(g["drab_pos"][:, 16:] == 0.0)    # no position distance reaches 16 here
    assert np.abs(g["dw1"]).max() > 1e-2 and np.abs(g["drab_ts"]).max() > 1e-3


def test_layer_backward_linear_in_dy():
    w = hs.make_inputs([7, 12], 2, 4, dtype="fp32", seed=32, rab=True, num_targets=3,
                       layer_dim=8)
    rng = np.random.default_rng(6)
    d1 = rng.normal(size=(19, 8)); d2 = rng.normal(size=(19, 8))
    g1, g2 = oracle.layer_bwd(w, dy=d1), oracle.layer_bwd(w, dy=d2)
    g3 = oracle.layer_bwd(w, dy=2.0 * d1 - d2)
    for name in ("dx", "dw1", "dw2", "drab_pos", "drab_ts"):
        np.testing.assert_allclose(g3[name], 2.0 * g1[name] - g2[name], rtol=1e-9, atol=1e-13)


# ---- workload recipe --------------------------------------------------------------------------

def test_workload_shapes():
    w = hs.make_workload("tiny_fp32")
    assert w["lengths"].tolist() == [7, 16, 33, 64] and w["max_seqlen"] == 64
    assert w["q"].shape == (120, 2, 32) and w["rab_pos"] is None
    w = hs.make_workload("longtail_fwd")
    assert w["batch"] == 128 and w["lengths"].min() >= 8 and w["lengths"].max() <= 4096
    ts = w["timestamps"]
    off = w["seq_offsets"]
    for b in range(w["batch"]):
        assert np.all(np.diff(ts[off[b]:off[b + 1]]) >= 1)
    # bf16 rounding: every value is representable in bf16 (low 16 bits of float32 clear)
    assert np.all(w["q"].view(np.uint32) & 0xFFFF == 0)
