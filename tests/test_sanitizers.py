"""CPU sanitizer runs: the fp64 oracle and the library's host-only code
(configuration checks, blob sizes, weight repacks: csrc/host_pack.h) built
with AddressSanitizer + UndefinedBehaviorSanitizer (no recovery: the first
report ends the process) and run on small cases.

- tests/native/host_check.cpp fuzzes the configuration checks and checks the
  repacks against properties of the packed layouts;
- oracle/sanitize_driver.c runs the oracle's loop variants, the single
  velocity and the prefix pass from case files; its outputs must equal the
  ordinary build's (the same C code, so the same bits: neither build
  contracts or reorders floating point, and OpenMP only splits independent
  outputs).

Both are plain executables, so no sanitizer runtime is preloaded anywhere.
The guard canaries around every device buffer (pi0x_expert_check_guards) are
checked by the GPU tests, at every handle's close (tests/conftest.py)."""
from __future__ import annotations

import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

from oracle import oracle
from vla_flow_matching_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.fail(f"sanitizer build failed:\n{' '.join(cmd)}\n{res.stderr[-4000:]}")


@pytest.fixture(scope="module")
def tools(tmp_path_factory):
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc/g++ not available")
    d = tmp_path_factory.mktemp("san")
    host = str(d / "host_check")
    _build(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "vla_flow_matching_amd", "csrc"),
            os.path.join(ROOT, "tests", "native", "host_check.cpp"), "-o", host])
    drv = str(d / "oracle_driver")
    _build(["gcc", "-std=c11", "-D_GNU_SOURCE", *SAN, os.path.join(ROOT, "oracle", "sanitize_driver.c"),
            os.path.join(ROOT, "oracle", "pi0_oracle.c"), "-lm", "-o", drv])
    return {"dir": d, "host": host, "driver": drv}


def _run_clean(args):
    res = subprocess.run(args, capture_output=True, text=True, env=ENV, timeout=600)
    report = res.stderr[-6000:]
    assert "runtime error" not in res.stderr, f"UBSan report:\n{report}"
    assert "Sanitizer" not in res.stderr, f"sanitizer report:\n{report}"
    assert res.returncode == 0, f"exit {res.returncode}:\n{report}"
    return res


def test_host_code_under_asan_ubsan(tools):
    res = _run_clean([tools["host"]])
    assert "host checks passed" in res.stdout


def _case(path, mode, s, arrays, L, valid=0, steps=0, schedule=0, xpred=0, causal=0, blend=0, pos_shift=0.0, t=0.0):
    with open(path, "wb") as f:
        f.write(b"PI0OSAN1")
        f.write(struct.pack("<i", mode))
        f.write(struct.pack("<9i", s.width, s.depth, s.mlp_dim, s.num_heads, s.num_kv_heads, s.head_dim,
                            s.horizon, s.action_dim, s.state_dim))
        f.write(struct.pack("<4d", s.rms_eps, s.rope_theta, s.min_period, s.max_period))
        f.write(struct.pack("<7i", L, valid, steps, schedule, xpred, causal, blend))
        f.write(struct.pack("<2d", pos_shift, t))
        for a in arrays:
            f.write(np.ascontiguousarray(a, dtype="<f8").tobytes())


def _driver(tools, name, mode, s, arrays, n_out, **kw):
    case, out = str(tools["dir"] / f"{name}.case"), str(tools["dir"] / f"{name}.out")
    _case(case, mode, s, arrays, **kw)
    _run_clean([tools["driver"], case, out])
    got = np.fromfile(out, dtype="<f8")
    assert got.size == n_out
    return got


TINY = synth.TINY
LOOP_CASES = [
    # (L, valid, steps, schedule, x_prediction, causal, blend)
    (64, 64, 2, "pi0", False, False, False),
    (64, 37, 3, "pi0", False, False, False),
    (64, 1, 2, "zero_to_one", True, False, False),
    (64, 0, 2, "pi0", False, True, True),
    (0, 0, 2, "zero_to_one", False, False, False),
    (17, 17, 1, "pi0", True, True, True),
]


@pytest.mark.parametrize("L,valid,steps,schedule,xpred,causal,blend", LOOP_CASES)
def test_oracle_loop_under_asan_ubsan(tools, L, valid, steps, schedule, xpred, causal, blend):
    s = TINY
    w = synth.make_weights(s, seed=11, dtype="fp32", norm_std=0.1).astype(np.float64)
    rng = np.random.default_rng(L * 100 + valid)
    state = rng.standard_normal(s.state_dim)
    noise = rng.standard_normal((s.horizon, s.action_dim))
    kv = rng.standard_normal((s.depth, 2, L, s.num_kv_heads, s.head_dim))
    arrays = [w, state, noise, kv]
    mask = pad = None
    if blend:
        mask = (rng.random((s.horizon, s.action_dim)) < 0.5).astype(np.float64)
        pad = rng.standard_normal((s.horizon, s.action_dim))
        arrays += [mask, pad]
    got = _driver(tools, f"loop_{L}_{valid}_{steps}_{schedule}_{int(xpred)}{int(causal)}{int(blend)}", 0, s, arrays,
                  s.horizon * s.action_dim, L=L, valid=valid, steps=steps, schedule=oracle.SCHEDULES[schedule],
                  xpred=int(xpred), causal=int(causal), blend=int(blend))
    ref = oracle.Oracle(s, w).denoise_ex(state, noise, kv, L, valid, steps, schedule=schedule, x_prediction=xpred,
                                         causal=causal, dof_mask=mask, padding=pad)
    assert np.array_equal(got, ref.ravel())


def test_oracle_velocity_under_asan_ubsan(tools):
    s = TINY
    w = synth.make_weights(s, seed=12, dtype="fp32", norm_std=0.1).astype(np.float64)
    rng = np.random.default_rng(3)
    L, valid = 40, 29
    state = rng.standard_normal(s.state_dim)
    x = rng.standard_normal((s.horizon, s.action_dim))
    kv = rng.standard_normal((s.depth, 2, L, s.num_kv_heads, s.head_dim))
    got = _driver(tools, "velocity", 1, s, [w, state, x, kv], s.horizon * s.action_dim, L=L, valid=valid, t=0.3)
    ref = oracle.Oracle(s, w).velocity(state, x, 0.3, kv, L, valid)
    assert np.array_equal(got, ref.ravel())


@pytest.mark.parametrize("L,valid", [(24, 17), (8, 8), (5, 0)])
def test_oracle_prefill_under_asan_ubsan(tools, L, valid):
    s = synth.TINY_VLM
    w = synth.make_weights(s, seed=13, dtype="fp32", norm_std=0.1, layout=synth.layer_layout).astype(np.float64)
    emb = np.random.default_rng(L).standard_normal((L, s.width))
    n = s.depth * 2 * L * s.num_kv_heads * s.head_dim
    got = _driver(tools, f"prefill_{L}_{valid}", 2, s, [w, emb], n, L=L, valid=valid)
    ref = oracle.PrefillOracle(s, w).prefill(emb, valid)
    assert np.array_equal(got, ref.ravel())
