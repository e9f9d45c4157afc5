"""hstu_attn_fwd_noalloc, the forward entry point that allocates nothing, against hstu_attn_fwd.

Both are called through the C ABI on the same plan and inputs; the no-alloc call keeps its
scratch (partial sums of split row blocks, and the attention output before the LayerNorm of the
gated form) in the library's static per-device array.  Its outputs must equal the regular
call's bit for bit (the same kernels run in the same order) and match the oracle at the bf16
tolerance.  Two calls in a row, the second on a smaller batch, show that nothing left in the
array by a call leaks into the next; a plan that needs more than the array holds is refused on
the host before anything is launched.
"""
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

hj.load_library()

SCRATCH_LIMIT = 9


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def gated_ref(w, u):
    A = oracle.attn_fwd(w).reshape(w["total_tokens"], -1)
    return (A - A.mean(axis=1, keepdims=True)) / np.sqrt(A.var(axis=1, keepdims=True) + 1e-5) * u


def within(got, want):
    err = float(np.max(np.abs(got - want)))
    assert err <= 2e-2 * float(np.max(np.abs(want))), err


def run_pair(w, gated, seed):
    """The regular and the no-alloc forward on one plan; returns both outputs and the oracle's."""
    T, H, d = w["total_tokens"], w["heads"], w["d"]
    dev = runner.to_device(w)
    args = runner.args_for(w, dev)
    plan = runner.plan_for(w, args)
    info = hj.hstu_plan_info(plan)
    u = ut = None
    if gated:
        u = hs.round_bf16(np.random.default_rng(seed).normal(size=(T, H * d)).astype(np.float32))
        ut = torch.from_numpy(u).to("cuda:0", torch.bfloat16)
    ref_out = runner.empty_like_thd(w, dev)
    new_out = torch.full_like(ref_out, float("nan"))
    ws = torch.empty(max(hj.hstu_workspace_bytes(plan, hj.OP_FWD_GATED if gated else hj.OP_FWD), 16),
                     dtype=torch.uint8, device="cuda:0")
    hj.hstu_attn_fwd(plan, args, dev["q"], dev["k"], dev["v"], ref_out, u=ut, ws=ws)
    hj.hstu_attn_fwd_noalloc(plan, args, dev["q"], dev["k"], dev["v"], new_out, u=ut)
    torch.cuda.synchronize()
    want = gated_ref(w, u) if gated else oracle.attn_fwd(w)
    plan.close()
    return info, ref_out, new_out, want


@pytest.mark.parametrize("gated", [False, True])
def test_noalloc_matches_fwd_on_two_calls(gated):
    # first call: one long sequence among short ones (split row blocks use partial slots)
    big = hs.make_inputs([3000] + [60] * 40, 2, 64, dtype="bf16", seed=41, rab=True,
                         num_contexts=2, num_targets=8)
    # second call: a smaller batch with splits of its own
    small = hs.make_inputs([1500, 20, 9, 33], 2, 64, dtype="bf16", seed=42, rab=True,
                           num_contexts=1, num_targets=4)
    for label, w in (("first, larger", big), ("second, smaller", small)):
        say(f"noalloc forward gated={gated}: {label} call")
        info, ref_out, new_out, want = run_pair(w, gated, 7)
        assert info["fwd_split_blocks"] > 0
        assert torch.equal(ref_out, new_out), label
        within(new_out.float().cpu().numpy().reshape(want.shape), want)


def test_noalloc_without_scratch_and_empty_batch():
    # no split blocks and no gate: nothing needs scratch
    w = hs.make_inputs([100, 37, 250], 2, 128, dtype="bf16", seed=43, rab=True, num_targets=16)
    say("noalloc forward needing no scratch")
    info, ref_out, new_out, want = run_pair(w, False, 8)
    assert info["fwd_split_blocks"] == 0
    assert torch.equal(ref_out, new_out)
    within(new_out.float().cpu().numpy(), want)
    e = hs.make_inputs([0, 0], 2, 64, dtype="bf16", seed=44, rab=False, max_seqlen=4)
    args = hj.make_args(dtype=hj.HSTU_BF16, batch=2, num_heads=2, head_dim=64, total_tokens=0,
                        max_seqlen=4)
    plan = hj.hstu_plan_create(args, e["seq_offsets"])
    hj.hstu_attn_fwd_noalloc(plan, args, None, None, None, None)
    plan.close()


def test_noalloc_refuses_plans_beyond_the_scratch():
    # gated: the attention output alone needs T * H * d * 2 bytes > 64 MiB; refused on the host
    T, H, d = 70000, 4, 128
    args = hj.make_args(dtype=hj.HSTU_BF16, batch=1, num_heads=H, head_dim=d, total_tokens=T,
                        max_seqlen=T, alpha=0.1)
    plan = hj.hstu_plan_create(args, np.array([0, T]))
    assert hj.hstu_workspace_bytes(plan, hj.OP_FWD_GATED) > 64 << 20
    tiny = torch.zeros(64, dtype=torch.bfloat16, device="cuda:0")
    say("noalloc forward refusing a plan beyond the scratch")
    with pytest.raises(hj.HstuError) as e:
        hj.hstu_attn_fwd_noalloc(plan, args, tiny, tiny, tiny, tiny, u=tiny)
    assert e.value.status == SCRATCH_LIMIT
    plan.close()
