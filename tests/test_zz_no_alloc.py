"""pi0x_denoise_noalloc, the call variant that allocates nothing (its working
buffers live in a static per-GPU device array), against pi0x_denoise on the
same handle and inputs: the pi0 expert in bf16 at batch 1, two calls in a
row, the second with a shorter prefix, fewer valid keys and fewer steps.

Both entry points run the same kernels with the same launch shapes in the
same order, so the chunks must agree bit for bit (which is inside the loop's
bf16 bar of max|diff| <= 3e-2 and relative L2 <= 1e-2 against each other)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from vla_flow_matching_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

W1 = synth.WORKLOADS["pi0_bf16_b1"]


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def b1():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vla_flow_matching_amd import binding
    blob = synth.make_weights(W1.shape, seed=W1.seed, dtype="bf16")
    cfg = binding.make_config(W1.shape, "bf16", max_batch=2, max_prefix_len=1024, max_steps=16)
    _say("create pi0 bf16 handle, max_batch 2, max_prefix_len 1024")
    ex = binding.Expert(cfg, blob)
    dev = binding.device_inputs(synth.make_inputs(W1), "bf16")
    yield ex, dev
    ex.close()


def _inputs(dev, prefix_len, valid):
    kv = dev["prefix_kv"][:, :, :, :prefix_len].contiguous()
    v = torch.full((1,), valid, dtype=torch.int32, device="cuda")
    return kv, v


def _both(ex, kv, valid, state, noise, n):
    _say(f"pi0x_denoise B=1 L={kv.shape[3]} valid={int(valid[0])} N={n}")
    ref = ex.denoise(kv, valid, state, noise, n)
    torch.cuda.synchronize()
    out = torch.full_like(noise, float("nan"))
    _say(f"pi0x_denoise_noalloc B=1 L={kv.shape[3]} valid={int(valid[0])} N={n}")
    ex.denoise_noalloc(kv, valid, state, noise, out, n)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


def test_noalloc_equals_denoise_on_two_calls_in_a_row(b1):
    ex, dev = b1
    state, noise = dev["state"], dev["noise"]
    cases = [(816, 816, 10), (640, 600, 5)]  # the second call is smaller on every axis
    for L, valid, n in cases:
        kv, v = _inputs(dev, L, valid)
        ref, out = _both(ex, kv, v, state, noise, n)
        assert np.all(np.isfinite(out)), f"L={L}: non-finite output"
        diff = np.abs(out.astype(np.float64) - ref)
        rel = float(np.linalg.norm(out.astype(np.float64) - ref) / np.linalg.norm(ref))
        _say(f"L={L} valid={valid} N={n}: max|diff| {diff.max():.3e} rel-L2 {rel:.3e}")
        assert diff.max() <= 3e-2 and rel <= 1e-2
        assert np.array_equal(out, ref), f"L={L}: the no-alloc call differs from pi0x_denoise"


def test_noalloc_leaves_the_handle_path_unchanged(b1):
    ex, dev = b1
    kv, v = _inputs(dev, 816, 700)
    before = ex.denoise(kv, v, dev["state"], dev["noise"], 3).cpu().numpy()
    out = torch.empty_like(dev["noise"])
    ex.denoise_noalloc(kv, v, dev["state"], dev["noise"], out, 3)
    after = ex.denoise(kv, v, dev["state"], dev["noise"], 3).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(before, after)
    assert np.array_equal(out.cpu().numpy(), before)


def test_noalloc_rejects_more_than_64_rows(b1):
    from vla_flow_matching_amd import binding
    ex, dev = b1
    B = 2
    kv = dev["prefix_kv"].expand(-1, -1, B, -1, -1).contiguous()
    v = torch.full((B,), 816, dtype=torch.int32, device="cuda")
    state = dev["state"].expand(B, -1).contiguous()
    noise = dev["noise"].expand(B, -1, -1).contiguous()
    out = torch.empty_like(noise)
    with pytest.raises(binding.Pi0xError) as e:
        ex.denoise_noalloc(kv, v, state, noise, out, 2)
    assert e.value.status == binding.PI0X_ERR_CAPACITY and "suffix rows" in str(e.value)


def test_noalloc_rejects_a_call_beyond_the_scratch_array():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vla_flow_matching_amd import binding
    # 40 layers of head_dim 256: the V^T copies of a 2048-key prefix alone
    # take 40 x 256 x 2048 x 2 bytes, more than the 32 MiB array
    shape = synth.ExpertShape(width=256, depth=40, mlp_dim=512, num_heads=1, num_kv_heads=1, head_dim=256,
                              horizon=15, action_dim=32, state_dim=32)
    w = synth.Workload("deep_thin_bf16_b1", shape, "bf16", 1, 2048, 2)
    cfg = binding.make_config(shape, "bf16", max_batch=1, max_prefix_len=2048, max_steps=4)
    _say("create deep thin bf16 handle, max_prefix_len 2048")
    ex = binding.Expert(cfg, synth.make_weights(shape, seed=3, dtype="bf16"))
    try:
        d = binding.device_inputs(synth.make_inputs(w), "bf16")
        out = torch.empty_like(d["noise"])
        with pytest.raises(binding.Pi0xError) as e:
            ex.denoise_noalloc(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], out, 2)
        assert e.value.status == binding.PI0X_ERR_CAPACITY and "bytes of scratch" in str(e.value)
        # a prefix that fits runs
        kv = d["prefix_kv"][:, :, :, :256].contiguous()
        v = torch.full((1,), 256, dtype=torch.int32, device="cuda")
        ref = ex.denoise(kv, v, d["state"], d["noise"], 2)
        ex.denoise_noalloc(kv, v, d["state"], d["noise"], out, 2)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy())
    finally:
        ex.close()


def test_noalloc_rejects_float32_handles():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vla_flow_matching_amd import binding
    w = synth.WORKLOADS["tiny_fp32_b1"]
    cfg = binding.make_config(w.shape, "fp32", max_batch=1, max_prefix_len=64, max_steps=4)
    ex = binding.Expert(cfg, synth.make_weights(w.shape, seed=0, dtype="fp32"))
    try:
        d = binding.device_inputs(synth.make_inputs(w), "fp32")
        out = torch.empty_like(d["noise"])
        with pytest.raises(binding.Pi0xError) as e:
            ex.denoise_noalloc(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], out, 2)
        assert e.value.status == binding.PI0X_ERR_DTYPE
    finally:
        ex.close()


def test_noalloc_under_stream_capture(b1):
    # the use it exists for: captured into the caller's own graph (every node
    # a kernel: no memset or copy nodes), replayed several times with other
    # eager work and synchronizations between the replays
    ex, dev = b1
    kv, v = _inputs(dev, 816, 750)
    state, noise = dev["state"], dev["noise"]
    eager = torch.empty_like(noise)
    _say("pi0x_denoise_noalloc eager reference")
    ex.denoise_noalloc(kv, v, state, noise, eager, 4)
    torch.cuda.synchronize()
    ref = eager.cpu().numpy()
    out = torch.full_like(noise, float("nan"))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    _say("capture pi0x_denoise_noalloc")
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ex.denoise_noalloc(kv, v, state, noise, out, 4)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        _say(f"replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref), f"replay {r} differs from the eager call"
        # other work between replays, on the same handle and array
        ex.denoise(kv, v, state, noise, 2)
        torch.cuda.synchronize()
