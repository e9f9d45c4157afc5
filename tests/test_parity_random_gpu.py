"""Randomized small shapes on the GPU against the oracle (derandomized, bounded, no shrinking).

Each example draws a jagged batch: 1 to 5 sequences of 0 to 300 tokens, a context count and a
candidate count that may exceed the sequence length, head dim 32, 64 or 128, 1 to 3 heads, one
of the four bias-table subsets, bf16 or fp32, and whether to run the backward too.  These are the
shapes where contexts and candidates collide with the 32-row, 64-key and 128-row tile edges
(page 1 section 2.1.2, ranking: candidates appended and isolated from each other; page 2, HSTU
acceleration operator: the composite mask).  The forward output, and for backward examples dQ,
dK, dV and the requested bias-table gradients, are compared with the oracle at the usual
tolerances.  Examples are generated deterministically; a failure is reported as drawn, not
shrunk, so that no extra GPU runs follow it.
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
hypothesis = pytest.importorskip("hypothesis")
from hypothesis import Phase, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import hstu_jagged_pointwise_amd as hj  # noqa: E402
from hstu_jagged_pointwise_amd import runner  # noqa: E402

hj.load_library()

BF16_REL = 2e-2
F32_ABS = 1e-5


def _check(name, got, want, dtype, case):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (case, name)
    assert np.all(np.isfinite(got)), (case, name)
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    bound = F32_ABS if dtype == "fp32" else BF16_REL * (float(np.max(np.abs(want))) if want.size else 0.0)
    assert err <= bound + 1e-30, f"{case}: {name} max err {err:.3e} > {bound:.3e}"


cases = st.fixed_dictionaries({
    "lengths": st.lists(st.integers(0, 300), min_size=1, max_size=5),
    "nc": st.sampled_from([0, 0, 1, 3, 8, 40, 400]),
    "nt": st.sampled_from([0, 0, 1, 5, 16, 64, 400]),
    "d": st.sampled_from([32, 64, 128]),
    "heads": st.integers(1, 3),
    "bias": st.sampled_from(["none", "pos", "ts", "both"]),
    "dtype": st.sampled_from(["bf16", "bf16", "bf16", "fp32"]),
    "backward": st.booleans(),
    "seed": st.integers(0, 2 ** 16),
})


@settings(max_examples=60, derandomize=True, deadline=None, database=None,
          phases=[Phase.explicit, Phase.generate], print_blob=False)
@given(case=cases)
def test_random_shapes_match_oracle(case):
    lengths = case["lengths"]
    if sum(lengths) == 0:
        lengths = lengths + [1]
    w = hs.make_inputs(lengths, case["heads"], case["d"], dtype=case["dtype"], seed=case["seed"],
                       rab=case["bias"] != "none", num_contexts=case["nc"],
                       num_targets=case["nt"], max_seqlen=max(lengths) + 3,
                       backward=case["backward"])
    if case["bias"] == "pos":
        w["rab_ts"] = None
    if case["bias"] == "ts":
        w["rab_pos"] = None
    label = {k: case[k] for k in ("lengths", "nc", "nt", "d", "heads", "bias", "dtype", "backward", "seed")}
    print(f"[gpu-case] random {label}", flush=True)
    sys.stdout.flush()
    dev = runner.to_device(w)
    out = runner.attn_fwd(w, dev)
    g = runner.attn_bwd(w, dev) if case["backward"] else None
    torch.cuda.synchronize()
    _check("O", out.float().cpu().numpy(), oracle.attn_fwd(w), case["dtype"], label)
    if g is not None:
        ref = oracle.attn_bwd(w)
        for name in ("dq", "dk", "dv"):
            _check(name, g[name].float().cpu().numpy(), ref[name], case["dtype"], label)
        for name in ("drab_pos", "drab_ts"):
            if ref[name] is not None:
                _check(name, g[name].float().cpu().numpy(), ref[name],
                       "bf16" if case["dtype"] == "bf16" else "fp32", label)
