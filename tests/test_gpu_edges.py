"""Edge cases of the boundary against the fp64 oracle: valid lengths outside
[0, prefix_len] (clamped into it, as the header states), an empty prefix
(prefix_len 0, no cache at all), the step-count limits, and the longest
prefix at the largest batch of the benched configuration (batch 64, prefix
1024: 16 prefix key blocks of 64 plus the suffix block, 416 tiles per
residual GEMM)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import oracle
from vla_flow_matching_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TINY = synth.WORKLOADS["tiny_fp32_b1"].shape


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def check_close(gpu, ref, dtype, what):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = float(np.max(np.abs(gpu - ref)))
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30))
    _say(f"{what}: max|diff| {err:.3e} rel-L2 {rel:.3e}")
    if dtype == "fp32":
        assert err <= 1e-4, f"{what}: max|diff| {err}"
    else:
        assert err <= 3e-2 and rel <= 1e-2, f"{what}: max|diff| {err} rel-L2 {rel}"


def _handle(shape, dtype, batch, max_prefix_len, max_steps=16, seed=0, norm_std=0.1):
    from vla_flow_matching_amd import binding
    blob = synth.make_weights(shape, seed=seed, dtype=dtype, norm_std=norm_std)
    cfg = binding.make_config(shape, dtype, max_batch=batch, max_prefix_len=max_prefix_len, max_steps=max_steps)
    _say(f"create {dtype} B={batch} Lmax={max_prefix_len} Nmax={max_steps} seed={seed}")
    return binding.Expert(cfg, blob), blob


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_valid_lengths_outside_the_prefix_are_clamped(gpu, dtype):
    from vla_flow_matching_amd import binding
    w = synth.Workload("tiny_clamp", TINY, dtype, 3, 64, 2, seed=61)
    ex, blob = _handle(TINY, dtype, 3, 64, seed=61)
    try:
        inp = synth.make_inputs(w)
        inp["valid_len"][:] = [-7, 64 + 50, 20]
        d = binding.device_inputs(inp, dtype)
        _say(f"denoise {dtype} valid {list(inp['valid_len'])}")
        out = ex.denoise(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], 2).cpu().numpy()
        ref_inp = dict(inp)
        ref_inp["valid_len"] = np.clip(inp["valid_len"], 0, 64).astype(np.int32)
        check_close(out, oracle.Oracle(TINY, blob).denoise_batch(ref_inp, 2), dtype,
                    f"tiny {dtype} valid -7 / 114 / 20 clamped to 0 / 64 / 20")
    finally:
        ex.close()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_empty_prefix(gpu, dtype):
    # prefix_len 0 and no cache pointer: the suffix attends to itself only
    from vla_flow_matching_amd import binding
    w = synth.Workload("tiny_empty", TINY, dtype, 2, 0, 3, seed=62)
    ex, blob = _handle(TINY, dtype, 2, 64, seed=62)
    try:
        inp = synth.make_inputs(w)
        d = binding.device_inputs(inp, dtype)
        _say(f"denoise {dtype} prefix_len 0")
        out = ex.denoise(None, d["valid_len"], d["state"], d["noise"], 3).cpu().numpy()
        check_close(out, oracle.Oracle(TINY, blob).denoise_batch(inp, 3), dtype, f"tiny {dtype} empty prefix")
    finally:
        ex.close()


def test_step_count_limits(gpu):
    from vla_flow_matching_amd import binding
    w = synth.Workload("tiny_steps", TINY, "fp32", 1, 64, 16, seed=63)
    ex, blob = _handle(TINY, "fp32", 1, 64, max_steps=16, seed=63)
    try:
        inp = synth.make_inputs(w)
        d = binding.device_inputs(inp, "fp32")
        orc = oracle.Oracle(TINY, blob)
        for n in (1, 16):
            _say(f"denoise fp32 N={n}")
            out = ex.denoise(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], n).cpu().numpy()
            check_close(out, orc.denoise_batch(inp, n), "fp32", f"tiny fp32 N={n}")
        with pytest.raises(binding.Pi0xError) as e:
            ex.denoise(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], 17)
        assert e.value.status == binding.PI0X_ERR_CAPACITY
        with pytest.raises(binding.Pi0xError) as e:
            ex.denoise(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], 0)
        assert e.value.status == binding.PI0X_ERR_INVALID_ARG
    finally:
        ex.close()


def test_full_bf16_b64_longest_prefix(gpu):
    # the benched batch at the largest prefix of the default configuration,
    # with ragged valid lengths; samples spread over the row tiles
    from vla_flow_matching_amd import binding
    w = synth.WORKLOADS["pi0_bf16_b64"].replace(name="pi0_bf16_b64_l1024", prefix_len=1024, seed=64)
    ex, blob = _handle(w.shape, "bf16", 64, 1024, seed=64, norm_std=0.0)
    try:
        inp = synth.make_inputs(w)
        inp["valid_len"][:] = 1024 - (np.arange(64) * 37) % 300
        d = binding.device_inputs(inp, "bf16")
        _say("denoise pi0 bf16 B=64 L=1024 N=10")
        out = ex.denoise(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], 10).cpu().numpy()
        samples = [0, 2, 37, 63]
        ref = oracle.Oracle(w.shape, blob).denoise_batch(inp, 10, samples=samples)
        for i, b in enumerate(samples):
            check_close(out[b], ref[i], "bf16", f"pi0 bf16 B=64 L=1024 valid {int(inp['valid_len'][b])} sample {b}")
    finally:
        ex.close()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_growing_key_scores_move_the_softmax_reference(gpu, dtype):
    # prefix key rows scaled by 1, 7, 13, 19 per group of 16 keys.  In float32
    # (32-key blocks) the second block's scores pass the first block's
    # maximum by more than the softmax's 2^8 slack, so the reference moves
    # mid-sequence; bf16 stages all 64 keys as one block.  End to end against
    # the oracle at each dtype's bar (float32: 1e-4)
    from vla_flow_matching_amd import binding
    w = synth.Workload("tiny_moving", TINY, dtype, 2, 64, 2, seed=65)
    ex, blob = _handle(TINY, dtype, 2, 64, seed=65)
    try:
        inp = synth.make_inputs(w)
        scale = (1.0 + 6.0 * (np.arange(64) // 16)).astype(np.float32)
        kv = inp["prefix_kv"]
        kv[:, 0] = kv[:, 0] * scale[None, None, :, None, None]
        if dtype == "bf16":
            kv[:, 0] = synth.round_bf16(kv[:, 0]).reshape(kv[:, 0].shape)
        d = binding.device_inputs(inp, dtype)
        _say(f"denoise {dtype} growing key scale")
        out = ex.denoise(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], 2).cpu().numpy()
        check_close(out, oracle.Oracle(TINY, blob).denoise_batch(inp, 2), dtype, f"tiny {dtype} growing key scores")
    finally:
        ex.close()
