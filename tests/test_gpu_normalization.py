"""Boundary normalization (page 1, _build_norm_buffers / _apply_norm) through
the C ABI against the fp64 oracle: the state is normalized before state_proj,
the returned action chunk is unnormalized, features past `count` pass through.
float32 mode, bar max|diff| <= 1e-4 (the pages' parity bar)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import oracle
from vla_flow_matching_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TINY = synth.WORKLOADS["tiny_fp32_b1"]


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def _stats(seed: int, mode: str, count: int) -> dict:
    rng = np.random.default_rng(seed)
    if mode == "mean_std":
        return {"mode": mode, "mean": rng.standard_normal(count).astype(np.float32),
                "std": rng.uniform(0.5, 2.0, count).astype(np.float32)}
    return {"mode": mode, "min": rng.uniform(-2.0, -1.0, count).astype(np.float32),
            "max": rng.uniform(1.0, 2.0, count).astype(np.float32)}


@pytest.fixture(scope="module")
def case():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vla_flow_matching_amd import binding
    blob = synth.make_weights(TINY.shape, seed=TINY.seed, dtype=TINY.dtype, norm_std=0.1)
    inputs = synth.make_inputs(TINY)
    cfg = binding.make_config(TINY.shape, TINY.dtype, max_batch=1, max_prefix_len=64, max_steps=16)
    _say("create tiny fp32 handle for normalization")
    ex = binding.Expert(cfg, blob)
    dev = binding.device_inputs(inputs, TINY.dtype)
    orc = oracle.Oracle(TINY.shape, blob)
    yield ex, dev, inputs, orc
    ex.close()


def _run(ex, dev):
    out = ex.denoise(dev["prefix_kv"], dev["valid_len"], dev["state"], dev["noise"], TINY.num_steps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("smode,amode", [("mean_std", "min_max"), ("min_max", "mean_std")])
def test_normalized_denoise_matches_oracle(case, smode, amode):
    ex, dev, inputs, orc = case
    s = TINY.shape
    sn, an = _stats(11, smode, s.state_dim - 3), _stats(12, amode, s.action_dim - 5)
    ex.set_normalization(sn, an)
    try:
        _say(f"normalized denoise state={smode} action={amode}")
        gpu = _run(ex, dev)
    finally:
        ex.set_normalization(None, None)
    ref = orc.denoise_batch(inputs, TINY.num_steps, state_norm=sn, action_norm=an)
    err = float(np.max(np.abs(gpu - ref)))
    _say(f"normalized denoise: max|diff| {err:.3e}")
    assert err <= 1e-4
    # features past the action statistics are the loop's own (normalized-space) values
    plain = orc.denoise_batch(inputs, TINY.num_steps, state_norm=sn)
    assert np.max(np.abs(gpu[..., s.action_dim - 5:] - plain[..., s.action_dim - 5:])) <= 1e-4


def test_clearing_normalization_restores_bitwise_output(case):
    ex, dev, inputs, orc = case
    base = _run(ex, dev)
    ex.set_normalization(_stats(21, "mean_std", TINY.shape.state_dim), _stats(22, "min_max", TINY.shape.action_dim))
    changed = _run(ex, dev)
    ex.set_normalization(None, None)
    again = _run(ex, dev)
    assert not np.array_equal(base, changed)
    assert np.array_equal(base, again)


def test_denoise_step_normalizes_state_only(case):
    ex, dev, inputs, orc = case
    s = TINY.shape
    sn, an = _stats(31, "min_max", s.state_dim), _stats(32, "mean_std", s.action_dim)
    rng = np.random.default_rng(33)
    x = rng.standard_normal((1, s.horizon, s.action_dim)).astype(np.float32)
    ex.set_normalization(sn, an)
    try:
        _say("normalized denoise_step t=0.6")
        v = ex.denoise_step(dev["prefix_kv"], dev["valid_len"], dev["state"], torch.from_numpy(x).cuda(), 0.6)
        torch.cuda.synchronize()
    finally:
        ex.set_normalization(None, None)
    state = oracle.apply_norm(inputs["state"][0], sn, inverse=False)
    ref = orc.velocity(state, x[0], float(np.float32(0.6)), inputs["prefix_kv"][:, :, 0], TINY.prefix_len,
                       int(inputs["valid_len"][0]))
    err = float(np.max(np.abs(v.cpu().numpy()[0] - ref)))
    _say(f"normalized velocity: max|diff| {err:.3e}")
    assert err <= 1e-4


def test_set_normalization_rejects_bad_arguments(case):
    import ctypes
    from vla_flow_matching_amd import binding as b
    ex = case[0]
    s = TINY.shape
    a = np.zeros(64, np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    good = b.pi0x_norm(b.PI0X_NORM_MEAN_STD, 4, a.ctypes.data_as(fp), a.ctypes.data_as(fp))
    bad = [b.pi0x_norm(7, 4, a.ctypes.data_as(fp), a.ctypes.data_as(fp)),
           b.pi0x_norm(b.PI0X_NORM_MIN_MAX, 0, a.ctypes.data_as(fp), a.ctypes.data_as(fp)),
           b.pi0x_norm(b.PI0X_NORM_MIN_MAX, s.state_dim + 1, a.ctypes.data_as(fp), a.ctypes.data_as(fp)),
           b.pi0x_norm(b.PI0X_NORM_MEAN_STD, 4, None, a.ctypes.data_as(fp))]
    for n in bad:
        assert b.lib().pi0x_set_normalization(ex.h, ctypes.byref(n), None) == b.PI0X_ERR_INVALID_ARG
        assert b.lib().pi0x_set_normalization(ex.h, None, ctypes.byref(n)) == b.PI0X_ERR_INVALID_ARG
    assert b.lib().pi0x_set_normalization(ex.h, ctypes.byref(good), ctypes.byref(good)) == b.PI0X_OK
    assert b.lib().pi0x_set_normalization(ex.h, None, None) == b.PI0X_OK
