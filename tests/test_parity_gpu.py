"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.

Tolerances: fp32 inputs, max |gpu - oracle| <= 1e-5; bf16 inputs, max |gpu - oracle| <=
2e-2 * max |oracle| per output tensor.  Small cases are compared element by element; the
full-size long-sequence workload is compared on sampled rows the oracle computes one by one.
"""
import os
import sys

import numpy as np
import pytest

import hstu_synth as hs
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import hstu_jagged_pointwise_amd as hj  # noqa: E402
from hstu_jagged_pointwise_amd import runner  # noqa: E402

hj.load_library()  # fail loudly if the HIP library is missing

BF16_REL = 2e-2
F32_ABS = 1e-5


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, got, want, dtype):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.all(np.isfinite(got)), name
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    if dtype == "fp32":
        assert err <= F32_ABS, f"{name}: max abs err {err:.3e} > {F32_ABS}"
    else:
        scale = float(np.max(np.abs(want))) if want.size else 0.0
        assert err <= BF16_REL * scale + 1e-30, f"{name}: max err {err:.3e} vs {BF16_REL} * {scale:.3e}"
    return err


def run_fwd(w, **kw):
    dev = runner.to_device(w)
    out = runner.attn_fwd(w, dev, **kw)
    torch.cuda.synchronize()
    return host(out)


# ---- forward --------------------------------------------------------------------------------

def test_tiny_fp32_workload():
    w = hs.make_workload("tiny_fp32")
    say("tiny_fp32 forward")
    check("O", run_fwd(w), oracle.attn_fwd(w), "fp32")


EDGE_LENGTHS = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 257, 0, 15, 2]
MASKS = [(0, 0), (0, 16), (4, 16), (8, 64), (3, 300), (300, 0)]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mask", range(len(MASKS)))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fwd_edges(d, mask, dtype):
    nc, nt = MASKS[mask]
    w = hs.make_inputs(EDGE_LENGTHS, 2, d, dtype=dtype, seed=100 + d + mask, rab=True,
                       num_contexts=nc, num_targets=nt, max_seqlen=300)
    say(f"fwd edges d={d} nc={nc} nt={nt} {dtype}")
    check("O", run_fwd(w), oracle.attn_fwd(w), dtype)


@pytest.mark.parametrize("which", ["none", "pos", "ts"])
def test_fwd_bias_subsets(which):
    w = hs.make_inputs([70, 5, 190], 3, 64, dtype="bf16", seed=7, rab=True, num_targets=8)
    if which in ("none", "ts"):
        w["rab_pos"] = None
    if which in ("none", "pos"):
        w["rab_ts"] = None
    say(f"fwd bias subset {which}")
    check("O", run_fwd(w), oracle.attn_fwd(w), "bf16")


def test_fwd_strided_inputs():
    w = hs.make_inputs([50, 129, 3], 2, 64, dtype="bf16", seed=9, rab=True, num_contexts=2,
                       num_targets=5)
    dev = runner.to_device(w)
    T, H, d = w["total_tokens"], 2, 64
    big = torch.zeros((T, 3, H * d), dtype=torch.bfloat16, device="cuda:0")
    for s, key in enumerate(("q", "k", "v")):
        big[:, s] = dev[key].reshape(T, H * d)
        dev[key] = big[:, s]
    args = runner.args_for(w, dev, qkv_token_stride=3 * H * d)
    say("fwd strided q/k/v")
    out = runner.attn_fwd(w, dev, args=args)
    torch.cuda.synchronize()
    check("O", host(out), oracle.attn_fwd(w), "bf16")


def test_fwd_wide_timestamps_take_64bit_path():
    w = hs.make_inputs([100, 77, 300], 2, 128, dtype="bf16", seed=11, rab=True, num_targets=16)
    ts = w["timestamps"].copy()
    ts[100:177] = np.sort(np.random.default_rng(0).integers(-(1 << 40), 1 << 40, 77))
    ts[200] += 3 << 31          # one token far in the future inside the third sequence
    w["timestamps"] = ts
    say("fwd wide timestamps")
    check("O", run_fwd(w), oracle.attn_fwd(w), "bf16")


def test_bwd_wide_timestamps_take_64bit_path():
    w = hs.make_inputs([130, 77, 300], 2, 64, dtype="bf16", seed=12, rab=True, num_targets=16,
                       backward=True)
    ts = w["timestamps"].copy()
    ts[130:207] = np.sort(np.random.default_rng(1).integers(-(1 << 40), 1 << 40, 77))
    ts[230] += 3 << 31          # one token far in the future inside the third sequence
    w["timestamps"] = ts
    say("bwd wide timestamps")
    _bwd_check(w, "bf16")


def _one_hot_values(T, H, d):
    v = np.zeros((T, H, d), np.float32)
    v[np.arange(T), :, np.arange(T) % d] = 1.0
    return v


@pytest.mark.parametrize("gap", [1 << 12, 1 << 18, (1 << 24) // 48])
def test_fwd_bias_buckets_one_hot(gap):
    # Scores from the bias tables alone (alpha = 0), neighbouring buckets with far-apart biases,
    # and one-hot value rows, so that each output element holds the probabilities of two or three
    # keys: a key that took a wrong position or time bucket moves its output element by far more
    # than the tolerance.  Time gaps of up to 2^24 / 24 per token put the tiles near the diagonal
    # on both sides of the 2^24 limit of the float-class time bias (page 1, section 2.1.2:
    # rab^{p,t} of the bucketized |i - j| and |t_i - t_j|).
    lengths = [300, 129, 700, 64]
    w = hs.make_inputs(lengths, 2, 128, dtype="bf16", seed=31, rab=True, alpha=0.0)
    T = w["total_tokens"]
    w["v"] = _one_hot_values(T, 2, 128)
    rng = np.random.default_rng(gap)
    ts = np.empty(T, np.int64)
    off = w["seq_offsets"]
    for b in range(len(lengths)):
        ts[off[b]:off[b + 1]] = 1_700_000_000 + np.cumsum(rng.integers(1, 2 * gap, off[b + 1] - off[b]))
    w["timestamps"] = ts
    buckets = np.arange(128, dtype=np.float32)
    w["rab_ts"] = np.stack([(buckets % 7) * 0.8 - 2.4, 2.0 - (buckets % 5) * 0.9]).astype(np.float32)
    w["rab_pos"] = np.stack([1.5 * np.cos(buckets), 1.5 * np.sin(1.3 * buckets)]).astype(np.float32)
    say(f"fwd one-hot bias buckets gap={gap}")
    check("O", run_fwd(w), oracle.attn_fwd(w), "bf16")


def test_fwd_empty_and_single():
    w = hs.make_inputs([0, 1, 0, 0, 1], 2, 32, dtype="bf16", seed=3, rab=True, num_targets=1,
                       max_seqlen=8)
    say("fwd empty and single-token sequences")
    check("O", run_fwd(w), oracle.attn_fwd(w), "bf16")
    w = hs.make_inputs([0, 0], 2, 32, dtype="bf16", seed=3, rab=True, max_seqlen=8)
    say("fwd all-empty batch")
    assert run_fwd(w).shape == (0, 2, 32)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fwd_gated_by_u(dtype):
    w = hs.make_inputs([40, 130, 7], 4, 32, dtype=dtype, seed=5, rab=True, num_contexts=1,
                       num_targets=4)
    u = np.random.default_rng(1).normal(size=(w["total_tokens"], 4 * 32)).astype(np.float32)
    if dtype == "bf16":
        u = hs.round_bf16(u)
    dev = runner.to_device(w)
    ut = torch.from_numpy(u).to("cuda:0", torch.bfloat16 if dtype == "bf16" else torch.float32)
    say(f"fwd gated by u {dtype}")
    out = runner.attn_fwd(w, dev, u=ut, ln_eps=1e-5)
    torch.cuda.synchronize()
    A = oracle.attn_fwd(w).reshape(w["total_tokens"], -1)
    G = (A - A.mean(axis=1, keepdims=True)) / np.sqrt(A.var(axis=1, keepdims=True) + 1e-5) * u
    check("LN(O)*u", host(out).reshape(G.shape), G, dtype)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("short", [40, 300])
def test_fwd_split_row_blocks(gated, short):
    # one long sequence among short ones: its last row blocks run as several items whose fp32
    # partial outputs a fix-up pass sums (the plan reports them); with 40 short sequences the
    # items are 64-row blocks in the key-half layout, with 300 the 128-row blocks
    w = hs.make_inputs([3000] + [60] * short, 2, 64, dtype="bf16", seed=21, rab=True,
                       num_contexts=2, num_targets=8)
    dev = runner.to_device(w)
    a = runner.args_for(w, dev)
    plan = runner.plan_for(w, a)
    info = hj.hstu_plan_info(plan)
    assert info["fwd_split_blocks"] > 0
    assert info["fwd_item_rows"] == (64 if short == 40 else 128)
    plan.close()
    say(f"fwd split row blocks gated={gated} short={short}")
    A = oracle.attn_fwd(w)
    if not gated:
        check("O", run_fwd(w), A, "bf16")
        return
    u = hs.round_bf16(np.random.default_rng(2).normal(size=(w["total_tokens"], 2 * 64)).astype(np.float32))
    ut = torch.from_numpy(u).to("cuda:0", torch.bfloat16)
    out = runner.attn_fwd(w, dev, u=ut, ln_eps=1e-5)
    torch.cuda.synchronize()
    A = A.reshape(w["total_tokens"], -1)
    G = (A - A.mean(axis=1, keepdims=True)) / np.sqrt(A.var(axis=1, keepdims=True) + 1e-5) * u
    check("LN(O)*u", host(out).reshape(G.shape), G, "bf16")


def test_ranking_workload_full():
    w = hs.make_workload("ranking_fwd")
    say("ranking_fwd full size")
    check("O", run_fwd(w), oracle.attn_fwd(w), "bf16")


def test_longtail_workload_full():
    w = hs.make_workload("longtail_fwd")
    say("longtail_fwd full size")
    check("O", run_fwd(w), oracle.attn_fwd(w), "bf16")


def test_plan_built_while_kernels_run():
    # a plan created and used while another plan's launches are still queued: its upload does not
    # wait for them, and its lists are complete before its own kernels read them
    say("plan created behind queued long-tail forwards, then the ranking forward")
    w1, w2 = hs.make_workload("longtail_fwd"), hs.make_workload("ranking_fwd")
    dev1, dev2 = runner.to_device(w1), runner.to_device(w2)
    a1 = runner.args_for(w1, dev1)
    p1 = runner.plan_for(w1, a1)
    out1 = runner.empty_like_thd(w1, dev1)
    for _ in range(40):
        hj.hstu_attn_fwd(p1, a1, dev1["q"], dev1["k"], dev1["v"], out1)
    a2 = runner.args_for(w2, dev2)
    p2 = runner.plan_for(w2, a2)
    out2 = runner.empty_like_thd(w2, dev2)
    hj.hstu_attn_fwd(p2, a2, dev2["q"], dev2["k"], dev2["v"], out2)
    torch.cuda.synchronize()
    check("O ranking", host(out2), oracle.attn_fwd(w2), "bf16")
    check("O long-tail", host(out1), oracle.attn_fwd(w1), "bf16")
    p1.close()
    p2.close()


# ---- full layer -----------------------------------------------------------------------------

def _layer_check(w):
    dev = runner.to_device(w)
    y = runner.layer_fwd(w, dev)
    torch.cuda.synchronize()
    yo, _ = oracle.layer_fwd(w)
    got = host(y)
    check("Y", got, yo, "bf16")
    # The residual branch Y - X alone, so the attention path is not hidden behind X.  Y is stored
    # in bf16, so each element also carries Y's own rounding, at most half a bf16 ulp <= 2^-8 |Y|.
    branch = yo - w["x"]
    err = np.abs(got - yo)
    allowed = BF16_REL * np.max(np.abs(branch)) + 2.0 ** -8 * np.abs(yo)
    worst = int(np.argmax(err - allowed))
    assert np.all(err <= allowed), (f"Y - X: err {err.flat[worst]:.3e} > allowed "
                                    f"{allowed.flat[worst]:.3e}")


def test_layer_small():
    w = hs.make_inputs([17, 130, 1, 64], 4, 128, dtype="bf16", seed=21, rab=True,
                       num_contexts=4, num_targets=16, layer_dim=512)
    say("layer small")
    _layer_check(w)


def test_layer_branch_dominant():
    # W2 scaled up so that the attention / LayerNorm / gate branch dominates Y
    w = hs.make_inputs([40, 200, 3], 4, 128, dtype="bf16", seed=22, rab=True,
                       num_contexts=4, num_targets=16, layer_dim=512)
    w["w2"] = hs.round_bf16(w["w2"] * 256.0)
    say("layer with a dominant residual branch")
    dev = runner.to_device(w)
    y = runner.layer_fwd(w, dev)
    torch.cuda.synchronize()
    yo, _ = oracle.layer_fwd(w)
    got = host(y)
    assert np.max(np.abs(yo - w["x"])) > 4 * np.max(np.abs(w["x"]))
    check("Y", got, yo, "bf16")


def test_layer_workload_full():
    w = hs.make_workload("layer_fwd")
    say("layer_fwd full size")
    _layer_check(w)


# ---- candidate scoring against cached history ------------------------------------------------

def _cached_check(w):
    dev = runner.to_device(w)
    out = runner.attn_fwd_cached(w, dev)
    torch.cuda.synchronize()
    return check("O", host(out), oracle.attn_fwd_cached(w), "bf16")


@pytest.mark.parametrize("d", [32, 64, 128])
def test_cached_small(d):
    # users without history, without candidates, more than one row block of candidates, and a
    # cache that is not a whole number of key tiles
    w = hs.make_cached_inputs([37, 1, 5, 130, 0, 700], [4, 3, 0, 17, 2, 150], 2, d, seed=61 + d)
    say(f"cached scoring small d={d}")
    _cached_check(w)


@pytest.mark.parametrize("rab", ["none", "pos"])
def test_cached_bias_subsets(rab):
    w = hs.make_cached_inputs([64, 200, 3], [16, 9, 130], 4, 128, seed=62, rab=True)
    if rab == "none":
        w["rab_pos"] = w["rab_ts"] = w["timestamps"] = w["cache_timestamps"] = None
    else:
        w["rab_ts"] = None
    say(f"cached scoring bias {rab}")
    _cached_check(w)


def test_cached_long_cache_is_split():
    lengths = [8000] + [50] * 200
    w = hs.make_cached_inputs(lengths, [16] * len(lengths), 4, 128, seed=63)
    dev = runner.to_device(w)
    a = runner.args_for(w, dev)
    plan = hj.hstu_plan_create_cached(a, w["cand_offsets"], w["cache_offsets"])
    assert hj.hstu_plan_info(plan)["fwd_split_blocks"] > 0
    say("cached scoring with a split long cache")
    out = runner.attn_fwd_cached(w, dev, plan=plan, args=a)
    torch.cuda.synchronize()
    check("O", host(out), oracle.attn_fwd_cached(w), "bf16")


def test_cached_workload_full():
    w = hs.make_cached_workload()
    say(f"cached scoring workload, {w['total_tokens']} candidates, {w['cache_tokens']} cached")
    _cached_check(w)


def test_cached_rejects_regular_calls():
    w = hs.make_cached_inputs([10], [2], 2, 64, seed=64)
    dev = runner.to_device(w)
    a = runner.args_for(w, dev)
    plan = hj.hstu_plan_create_cached(a, w["cand_offsets"], w["cache_offsets"])
    out = runner.empty_like_thd(w, dev)
    with pytest.raises(hj.HstuError):
        hj.hstu_attn_fwd(plan, a, dev["q"], dev["k"], dev["v"], out)


# ---- Stochastic Length compaction -----------------------------------------------------------

def _select_case(lengths, keep, starts, row_shape, dtype, seed):
    rng = np.random.default_rng(seed)
    so = hs.offsets_from_lengths(lengths)
    do = hs.offsets_from_lengths(keep)
    src = rng.normal(size=(int(so[-1]),) + row_shape)
    if dtype == torch.int64:
        src = rng.integers(-2 ** 62, 2 ** 62, size=src.shape)
    want = oracle.jagged_select(src, so, do, starts)
    ts = torch.from_numpy(np.ascontiguousarray(src)).to(device="cuda", dtype=dtype)
    dst = torch.full((int(do[-1]),) + row_shape, 7, dtype=dtype, device="cuda")
    dev = lambda a: torch.from_numpy(np.asarray(a, np.int64)).cuda()
    hj.hstu_jagged_select(dev(so), dev(do), ts, dst,
                          keep_start=None if starts is None else dev(starts))
    torch.cuda.synchronize()
    exp = torch.from_numpy(np.ascontiguousarray(want)).to(dtype)  # same rounding as the source
    assert torch.equal(dst.cpu(), exp), "compaction is not bit-exact"


@pytest.mark.parametrize("row_shape,dtype", [((512,), torch.bfloat16), ((4, 128), torch.float32),
                                             ((), torch.int64), ((4,), torch.float16)])
def test_jagged_select_tail_and_windows(row_shape, dtype):
    lengths = np.array([40, 0, 7, 300, 1, 64])
    keep = np.array([10, 0, 7, 0, 1, 33])
    say(f"jagged select {row_shape} {dtype}")
    _select_case(lengths, keep, None, row_shape, dtype, 71)
    starts = np.array([30, 0, 0, 17, 0, 31])
    _select_case(lengths, keep, starts, row_shape, dtype, 72)


def test_jagged_select_workload_full():
    w = hs.make_workload("longtail_fwd")
    L = w["lengths"]
    keep = np.minimum(L, 256)   # every sequence cut to its 256 most recent tokens
    say("jagged select, long-tail lengths cut to 256")
    _select_case(L, keep, None, (4, 128), torch.bfloat16, 73)


# ---- full layer backward ---------------------------------------------------------------------

def _layer_bwd_check(w):
    dev = runner.to_device(w)
    g = runner.layer_bwd(w, dev)
    torch.cuda.synchronize()
    ref = oracle.layer_bwd(w)
    errs = {}
    for name in ("dx", "dw1", "dw2", "drab_pos", "drab_ts"):
        if ref[name] is not None:
            errs[name] = check(name, host(g[name]), ref[name], "bf16")
    # dx = dy + (branch through the layer): judge the branch on its own scale too; dx is stored
    # in bf16, so each element also carries half a bf16 ulp of |dx|.
    got = host(g["dx"])
    branch = ref["dx"] - w["dy"]
    err = np.abs(got - ref["dx"])
    allowed = BF16_REL * np.max(np.abs(branch)) + 2.0 ** -8 * np.abs(ref["dx"])
    worst = int(np.argmax(err - allowed))
    assert np.all(err <= allowed), (f"dx - dy: err {err.flat[worst]:.3e} > allowed "
                                    f"{allowed.flat[worst]:.3e}")
    say("  relative errors " + ", ".join(
        f"{k} {v / max(np.max(np.abs(ref[k])), 1e-30):.2e}" for k, v in errs.items()))
    return errs


def test_layer_bwd_small():
    w = hs.make_inputs([17, 130, 1, 64], 4, 128, dtype="bf16", seed=41, rab=True,
                       num_contexts=4, num_targets=16, layer_dim=512, backward=True)
    say("layer backward small")
    _layer_bwd_check(w)


def test_layer_bwd_without_bias_gradient_outputs():
    """Bias tables present but their gradients not asked for (NULL outputs): the dK/dV pass still
    sums them in LDS and writes nothing; dX, dW1, dW2 are unchanged."""
    w = hs.make_inputs([17, 130, 1, 64], 4, 128, dtype="bf16", seed=41, rab=True,
                       num_contexts=4, num_targets=16, layer_dim=512, backward=True)
    dev = runner.to_device(w)
    args = runner.args_for(w, dev)
    plan = runner.plan_for(w, args)
    T, D, Hd = w["total_tokens"], w["layer_dim"], w["heads"] * w["d"]
    dx = torch.empty((T, D), dtype=torch.bfloat16, device="cuda:0")
    dw1 = torch.empty((D, 4 * Hd), dtype=torch.float32, device="cuda:0")
    dw2 = torch.empty((Hd, D), dtype=torch.float32, device="cuda:0")
    say("layer backward without bias-gradient outputs")
    hj.hstu_layer_bwd(plan, args, D, dev["x"], dev["w1"], dev["w2"], dev["dy"], dx, dw1, dw2)
    torch.cuda.synchronize()
    ref = oracle.layer_bwd(w)
    for name, got in (("dx", dx), ("dw1", dw1), ("dw2", dw2)):
        check(name, host(got), ref[name], "bf16")
    plan.close()


@pytest.mark.parametrize("heads,d,D", [(2, 64, 128), (4, 32, 256), (1, 128, 384)])
def test_layer_bwd_shapes(heads, d, D):
    # weights scaled so that the attention, LayerNorm and gate terms carry the gradients
    w = hs.make_inputs([5, 70, 129, 2, 64], heads, d, dtype="bf16", seed=42 + d, rab=True,
                       num_contexts=2, num_targets=5, layer_dim=D, backward=True)
    w["w1"] = hs.round_bf16(w["w1"] * 8.0)
    w["w2"] = hs.round_bf16(w["w2"] * 16.0)
    say(f"layer backward H={heads} d={d} D={D}")
    _layer_bwd_check(w)


def test_layer_bwd_without_time_bias():
    w = hs.make_inputs([33, 250], 4, 128, dtype="bf16", seed=43, rab=True, num_targets=8,
                       layer_dim=512, backward=True)
    w["rab_ts"] = None
    say("layer backward, position bias only")
    _layer_bwd_check(w)


def test_layer_bwd_empty_batch_clears_gradients():
    w = hs.make_inputs([0, 0], 4, 128, dtype="bf16", seed=44, rab=True, layer_dim=512,
                       backward=True, max_seqlen=8)
    say("layer backward, no tokens")
    dev = runner.to_device(w)
    dev["x"] = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    dev["dy"] = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    g = runner.layer_bwd(w, dev)
    torch.cuda.synchronize()
    for name in ("dw1", "dw2", "drab_pos", "drab_ts"):
        assert torch.all(g[name] == 0), name


def test_layer_bwd_workload_full():
    w = hs.make_workload("layer_fwd")
    w["dy"] = hs.round_bf16(np.random.default_rng(7).normal(
        0.0, 1.0, (w["total_tokens"], w["layer_dim"])).astype(np.float32))
    say(f"layer backward full size, T={w['total_tokens']}")
    _layer_bwd_check(w)


# ---- backward -------------------------------------------------------------------------------

def _bwd_check(w, dtype):
    dev = runner.to_device(w)
    g = runner.attn_bwd(w, dev)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(w)
    for name in ("dq", "dk", "dv"):
        check(name, host(g[name]), ref[name], dtype)
    for name in ("drab_pos", "drab_ts"):
        if ref[name] is not None:
            # fp32 sums over many pairs: judge fp32 gradients relative to their scale as well
            check(name, host(g[name]), ref[name], "bf16" if dtype == "bf16" else "fp32")


@pytest.mark.parametrize("gap", [1 << 12, (1 << 24) // 48])
def test_bwd_bias_buckets_strong(gap):
    # Neighbouring buckets with far-apart biases (the scores depend strongly on which bucket each
    # pair takes) at time gaps on both sides of the float-class limit; contexts and candidates in
    # the mask, so the dK/dV pass meets its one-, two- and three-bucket and per-element modes
    # (page 1, section 2.1.2: rab^{p,t} and its gradients).
    lengths = [300, 129, 700]
    w = hs.make_inputs(lengths, 2, 64, dtype="bf16", seed=41, rab=True, alpha=0.3,
                       num_contexts=3, num_targets=9, backward=True)
    T = w["total_tokens"]
    rng = np.random.default_rng(gap + 1)
    ts = np.empty(T, np.int64)
    off = w["seq_offsets"]
    for b in range(len(lengths)):
        ts[off[b]:off[b + 1]] = 1_700_000_000 + np.cumsum(rng.integers(1, 2 * gap, off[b + 1] - off[b]))
    w["timestamps"] = ts
    buckets = np.arange(128, dtype=np.float32)
    w["rab_ts"] = np.stack([(buckets % 7) * 0.8 - 2.4, 2.0 - (buckets % 5) * 0.9]).astype(np.float32)
    w["rab_pos"] = np.stack([1.5 * np.cos(buckets), 1.5 * np.sin(1.3 * buckets)]).astype(np.float32)
    say(f"bwd strong bias buckets gap={gap}")
    _bwd_check(w, "bf16")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mask", [0, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bwd_edges(d, mask, dtype):
    nc, nt = MASKS[mask]
    w = hs.make_inputs(EDGE_LENGTHS, 2, d, dtype=dtype, seed=200 + d + mask, rab=True,
                       num_contexts=nc, num_targets=nt, max_seqlen=300, backward=True)
    say(f"bwd edges d={d} nc={nc} nt={nt} {dtype}")
    _bwd_check(w, dtype)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", [0, 2, 3, 4])
def test_bwd_recompute_path(d, mask):
    """hstu_attn_bwd_dkdv + hstu_attn_bwd_dq: the dQ pass recomputes S and dP (no stored dS)."""
    nc, nt = MASKS[mask]
    w = hs.make_inputs(EDGE_LENGTHS, 2, d, dtype="bf16", seed=200 + d + mask, rab=True,
                       num_contexts=nc, num_targets=nt, max_seqlen=300, backward=True)
    say(f"bwd recompute path d={d} nc={nc} nt={nt}")
    dev = runner.to_device(w)
    g = runner.attn_bwd(w, dev, split=True)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(w)
    for name in ("dq", "dk", "dv", "drab_pos", "drab_ts"):
        check(name, host(g[name]), ref[name], "bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("which", ["none", "pos", "ts"])
def test_bwd_bias_subsets_stored_ds(d, which):
    """Stored-dS backward with each subset of the bias tables: the dK/dV pass sums only the
    gradients of the tables present (position only, time only, none)."""
    w = hs.make_inputs([300, 64, 1, 129, 200], 3, d, dtype="bf16", seed=51 + d, rab=True,
                       num_contexts=2, num_targets=8, max_seqlen=300, backward=True)
    if which in ("none", "ts"):
        w["rab_pos"] = None
    if which in ("none", "pos"):
        w["rab_ts"] = None
    say(f"bwd stored dS bias subset {which} d={d}")
    _bwd_check(w, "bf16")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_split_calls_share_workspace(d):
    """hstu_attn_bwd_dkdv then hstu_attn_bwd_dq on one workspace (the bench's calls): the dK/dV
    pass leaves dS and the bias-table gradients there and the dQ pass hands the gradients out;
    a dQ call that asks for one table only gets that one."""
    w = hs.make_inputs([500, 64, 129, 200], 2, d, dtype="bf16", seed=61 + d, rab=True,
                       num_contexts=3, num_targets=9, max_seqlen=500, backward=True)
    dev = runner.to_device(w)
    args = runner.args_for(w, dev)
    plan = runner.plan_for(w, args)
    ws = torch.empty(hj.hstu_workspace_bytes(plan, hj.OP_BWD), dtype=torch.uint8, device="cuda:0")
    dq, dk, dv = (runner.empty_like_thd(w, dev) for _ in range(3))
    drp = torch.full((2, 128), float("nan"), dtype=torch.float32, device="cuda:0")
    drt = torch.full((2, 128), float("nan"), dtype=torch.float32, device="cuda:0")
    say(f"bwd split calls on one workspace d={d}")
    hj.hstu_attn_bwd_dkdv(plan, args, dev["q"], dev["k"], dev["v"], dev["dout"], dk, dv, ws=ws)
    hj.hstu_attn_bwd_dq(plan, args, dev["q"], dev["k"], dev["v"], dev["dout"], dq, drp, None,
                        ws=ws)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(w)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("drab_pos", drp)):
        check(name, host(got), ref[name], "bf16")
    assert torch.isnan(drt).all()  # not asked for: left alone
    plan.close()


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_stored_ds_ignores_stale_workspace(d):
    """The stored-dS path reads only the dS entries its own dK/dV pass wrote (or masks them):
    a workspace filled with NaN beforehand changes nothing."""
    w = hs.make_inputs([300, 64, 1, 129, 200], 2, d, dtype="bf16", seed=31 + d, rab=True,
                       num_contexts=3, num_targets=9, max_seqlen=300, backward=True)
    dev = runner.to_device(w)
    plan = runner.plan_for(w, runner.args_for(w, dev))
    need = hj.hstu_workspace_bytes(plan, hj.OP_BWD)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda:0")
    say(f"bwd stored dS over a NaN-filled workspace d={d}")
    g = runner.attn_bwd(w, dev, plan=plan, ws=ws)
    g2 = runner.attn_bwd(w, dev, plan=plan, split=True)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(w)
    for name in ("dq", "dk", "dv", "drab_pos", "drab_ts"):
        assert torch.isfinite(g[name]).all(), name
        check(name, host(g[name]), ref[name], "bf16")
    # dK and dV come from the same kernel code either way
    for name in ("dk", "dv"):
        assert torch.equal(g[name], g2[name]), name


def test_bwd_no_bias_and_determinism():
    w = hs.make_inputs([300, 64, 1], 2, 64, dtype="bf16", seed=4, rab=False, num_targets=7,
                       backward=True)
    dev = runner.to_device(w)
    say("bwd without bias, twice")
    g1 = runner.attn_bwd(w, dev)
    g2 = runner.attn_bwd(w, dev)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv"):
        assert torch.equal(g1[name], g2[name]), name
    ref = oracle.attn_bwd(w)
    for name in ("dq", "dk", "dv"):
        check(name, host(g1[name]), ref[name], "bf16")


def test_long_workload_reduced_full_compare():
    w = hs.make_workload("long_fwdbwd", batch=3, len_cap=1100)
    say("long_fwdbwd reduced: forward")
    check("O", run_fwd(w), oracle.attn_fwd(w), "bf16")
    say("long_fwdbwd reduced: backward")
    _bwd_check(w, "bf16")


def test_long_workload_full_sampled():
    w = hs.make_workload("long_fwdbwd")
    dev = runner.to_device(w)
    say("long_fwdbwd full size: forward + backward")
    out = runner.attn_fwd(w, dev)
    g = runner.attn_bwd(w, dev)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    T, H = w["total_tokens"], w["heads"]
    off = w["seq_offsets"]
    # rows from every sequence: first, last, candidates, contexts and random ones
    toks = []
    for b in range(w["batch"]):
        s, e = int(off[b]), int(off[b + 1])
        toks += [s, s + 3, e - 1, e - 40, e - 70] + list(rng.integers(s, e, 4))
    toks = np.array(toks, np.int64)
    heads = rng.integers(0, H, len(toks))
    ref_o = oracle.attn_fwd_rows(w, toks, heads)
    ref_g = oracle.attn_bwd_rows(w, toks, heads)
    o = host(out)
    # per-tensor scale from the sampled oracle rows
    check("O rows", o[toks, heads], ref_o, "bf16")
    for name in ("dq", "dk", "dv"):
        check(f"{name} rows", host(g[name])[toks, heads], ref_g[name], "bf16")
    # bias gradients: every bucket sum equals the total of dS, for both tables, per head
    dp, dt = host(g["drab_pos"]), host(g["drab_ts"])
    np.testing.assert_allclose(dp.sum(axis=1), dt.sum(axis=1),
                               rtol=2e-2, atol=2e-2 * np.abs(dp).max())


def _longest_sequence(w_full):
    """The longest sequence of a workload as a batch of its own (same max_seqlen, contexts,
    candidates, bias tables and inputs)."""
    off = w_full["seq_offsets"]
    b = int(np.argmax(np.diff(off)))
    s, e = int(off[b]), int(off[b + 1])
    w = dict(w_full)
    w.update(batch=1, seq_offsets=np.array([0, e - s], np.int64), lengths=np.array([e - s]),
             num_targets=w_full["num_targets"][b:b + 1].copy(), total_tokens=e - s,
             timestamps=w_full["timestamps"][s:e].copy())
    for key in ("q", "k", "v", "dout"):
        w[key] = np.ascontiguousarray(w_full[key][s:e])
    return w


def test_long_workload_longest_sequence_full_compare():
    """The long-sequence workload's longest sequence (7983 tokens, 8 contexts, 64 candidates, all
    8 heads) alone, forward and stored-dS backward, compared element by element with the oracle:
    O, dQ, dK, dV and both bias-table gradients.  Its position distances reach bucket 51 and its
    key blocks far from the diagonal take the one-, two- and three-bucket gradient sums over
    spans of thousands of tokens."""
    w = _longest_sequence(hs.make_workload("long_fwdbwd"))
    assert w["total_tokens"] == 7983 and w["heads"] == 8
    dev = runner.to_device(w)
    args = runner.args_for(w, dev)
    plan = runner.plan_for(w, args)
    info = hj.hstu_plan_info(plan)
    assert info["bwd_stored_ds"] == 1 and info["bwd_ds_bytes"] > 0
    say("long_fwdbwd longest sequence: forward + stored-dS backward, all heads")
    out = runner.attn_fwd(w, dev, plan=plan, args=args)
    g = runner.attn_bwd(w, dev, plan=plan, args=args)
    torch.cuda.synchronize()
    say("long_fwdbwd longest sequence: oracle")
    check("O", host(out), oracle.attn_fwd(w), "bf16")
    ref = oracle.attn_bwd(w)
    # the far position buckets are really exercised
    assert np.all(np.abs(ref["drab_pos"][:, 41:52]) > 0)
    for name in ("dq", "dk", "dv", "drab_pos", "drab_ts"):
        check(name, host(g[name]), ref[name], "bf16")
    plan.close()


def test_plan_freed_in_stream_order_while_kernels_queued():
    """A plan destroyed right after its launches (in the order of the launch stream) and a second
    plan created and launched at once, reusing the freed memory: both outputs are right.  Once
    on the default stream and once on a non-blocking stream."""
    wa = hs.make_inputs([900, 40, 333], 4, 128, dtype="bf16", seed=61, rab=True, num_targets=16)
    wb = hs.make_inputs([77, 1200, 5, 260], 4, 128, dtype="bf16", seed=62, rab=True,
                        num_contexts=3, num_targets=9)
    for label, stream in (("default", None), ("non-blocking", torch.cuda.Stream())):
        say(f"plan destroyed in {label} stream order, next plan launched at once")
        outs = []
        for w in (wa, wb):
            dev = runner.to_device(w)
            torch.cuda.synchronize()
            args = runner.args_for(w, dev)
            plan = runner.plan_for(w, args)
            out = runner.empty_like_thd(w, dev)
            hj.hstu_attn_fwd(plan, args, dev["q"], dev["k"], dev["v"], out, stream=stream)
            plan.close(stream if stream is not None else torch.cuda.current_stream())
            outs.append(out)
        torch.cuda.synchronize()
        for w, out in zip((wa, wb), outs):
            check("O", host(out), oracle.attn_fwd(w), "bf16")


def test_runner_temporary_plans_on_side_stream():
    """The convenience layer's per-call plans and workspaces on a non-blocking stream: freed in
    that stream's order, so back-to-back calls leave both results intact."""
    w1 = hs.make_inputs([500, 64, 129], 2, 64, dtype="bf16", seed=71, rab=True, num_targets=8,
                        backward=True)
    w2 = hs.make_inputs([300, 700], 2, 64, dtype="bf16", seed=72, rab=True, num_contexts=2,
                        num_targets=5, backward=True)
    side = torch.cuda.Stream()
    d1, d2 = runner.to_device(w1), runner.to_device(w2)
    torch.cuda.synchronize()
    say("runner calls with temporary plans on a side stream")
    with torch.cuda.stream(side):
        o1 = runner.attn_fwd(w1, d1, stream=side)
        g1 = runner.attn_bwd(w1, d1, stream=side)
        o2 = runner.attn_fwd(w2, d2, stream=side)
        g2 = runner.attn_bwd(w2, d2, stream=side)
    side.synchronize()
    for w, o, g in ((w1, o1, g1), (w2, o2, g2)):
        check("O", host(o), oracle.attn_fwd(w), "bf16")
        ref = oracle.attn_bwd(w)
        for name in ("dq", "dk", "dv", "drab_pos", "drab_ts"):
            check(name, host(g[name]), ref[name], "bf16")


def test_bwd_stored_ds_sequence_beyond_32k():
    """A 33000-token sequence takes the stored-dS path (chunked per key block, 64-bit chunk
    offsets): sampled rows of dQ, dK, dV from the oracle, the bias-table gradients' totals."""
    w = hs.make_inputs([33000, 70], 1, 64, dtype="bf16", seed=91, rab=True, num_contexts=2,
                       num_targets=16, backward=True)
    dev = runner.to_device(w)
    args = runner.args_for(w, dev)
    plan = runner.plan_for(w, args)
    assert hj.hstu_plan_info(plan)["bwd_stored_ds"] == 1
    say("bwd stored dS on a 33000-token sequence")
    g = runner.attn_bwd(w, dev, plan=plan, args=args)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    toks = np.concatenate([[0, 1, 2, 100, 32767, 32768, 32769, 32983, 32984, 32999, 33000, 33069],
                           rng.integers(0, 33070, 12)]).astype(np.int64)
    heads = np.zeros(len(toks), np.int64)
    ref = oracle.attn_bwd_rows(w, toks, heads)
    for name in ("dq", "dk", "dv"):
        check(f"{name} rows", host(g[name])[toks, 0], ref[name], "bf16")
    # every bucket's gradient is a sum of dS, so both tables share one total per head
    dp, dt = host(g["drab_pos"]), host(g["drab_ts"])
    np.testing.assert_allclose(dp.sum(), dt.sum(), rtol=1e-3, atol=1e-3 * np.abs(dp).max())
    plan.close()
