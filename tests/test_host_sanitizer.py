"""The library's host code (argument checks, plan building, work-list readback) run under
AddressSanitizer and UndefinedBehaviorSanitizer on the CPU.

hstu_api.hip is compiled with both sanitizers on its host code (its device part, a static
scratch array, is built as usual) and linked into a small driver (sanitize_plan_driver.cpp) whose
kernel launchers are stubs that abort: host-only plans never launch.  The driver builds plans for
the five workload shapes, a ranking batch of thousands of users, and randomized jagged batches
with edge lengths, contexts and candidates beyond the sequence length, then reads back every
work list.  Any sanitizer report fails the test."""
import os
import subprocess

import numpy as np
import pytest

import hstu_synth as hs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hstu_jagged_pointwise_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Each -fsanitize= follows -Xarch_host: the sanitizers apply to host code only.
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
CFLAGS = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("san")
    objs = []
    for src in (os.path.join(CSRC, "hstu_api.hip"), os.path.join(ROOT, "tests", "sanitize_plan_driver.cpp")):
        obj = str(d / (os.path.basename(src) + ".o"))
        subprocess.run([HIPCC, *CFLAGS, "-c", src, "-o", obj], check=True, capture_output=True)
        objs.append(obj)
    exe = str(d / "drv")
    subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe], check=True,
                   capture_output=True)
    return exe


def _line(kind, dtype, H, d, nc, lengths, targets):
    vals = [kind, dtype, H, d, nc, len(lengths), *map(int, lengths), *map(int, targets)]
    return " ".join(map(str, vals))


def _problems():
    lines = []
    for name in hs.WORKLOAD_ORDER:
        spec = hs.WORKLOADS[name]
        L = hs.draw_lengths(np.random.default_rng(0), spec, spec.batch)
        dtype = 0 if spec.dtype == "fp32" else 1
        lines.append(_line(0, dtype, spec.heads, spec.d, spec.num_contexts, L,
                           [spec.num_targets] * len(L)))
    # a ranking batch of thousands of users
    rng = np.random.default_rng(5)
    L = rng.integers(100, 301, 4096)
    lines.append(_line(0, 1, 8, 64, 0, L, [16] * len(L)))
    # cached scoring: long-tail histories, some empty, 64 candidates (one user with none)
    L = np.clip(np.rint(rng.lognormal(5.0, 1.0, 64)), 0, 4096).astype(int)
    L[3] = 0
    cands = [64] * 64
    cands[7] = 0
    lines.append(_line(1, 1, 4, 128, 0, L, cands))
    edges = [0, 1, 2, 15, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000]
    for seed in range(40):
        r = np.random.default_rng(100 + seed)
        B = int(r.integers(0, 12))
        L = r.choice(edges, B) if seed % 2 else r.integers(0, 700, B)
        nt = r.integers(0, 300, B)
        nc = int(r.choice([0, 1, 4, 8, 200]))
        d = int(r.choice([32, 64, 128]))
        dtype = int(seed % 5 != 0)
        lines.append(_line(0, dtype, int(r.integers(1, 5)), d, nc, L, nt))
        if dtype == 1 and B > 0:
            lines.append(_line(1, 1, 2, d, 0, L, r.integers(0, 200, B)))
    # one very long sequence among short ones (split row blocks), and one beyond 32k tokens
    lines.append(_line(0, 1, 2, 128, 3, [40000, 5, 17, 300], [64, 0, 3, 16]))
    return lines


def test_plan_code_is_sanitizer_clean(driver):
    lines = _problems()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True,
                       env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.stdout.startswith(f"problems {len(lines)} "), r.stdout
