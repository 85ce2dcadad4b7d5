"""The batch-1 path (bf16, the pi0 expert shape: the one-kernel wide GEMMs, the
stream + reduce residual producers and the key-split attention) against the
fp64 oracle, on the edge cases of its 64-key blocks and on its determinism.

Bar: the loop's bf16 bar, max|diff| <= 3e-2 and relative L2 <= 1e-2."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import oracle
from vla_flow_matching_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

W1 = synth.WORKLOADS["pi0_bf16_b1"]


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def check_close(gpu, ref, what, max_abs=3e-2, max_rel=1e-2):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = float(np.max(np.abs(gpu - ref)))
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30))
    _say(f"{what}: max|diff| {err:.3e} rel-L2 {rel:.3e}")
    assert err <= max_abs and rel <= max_rel, f"{what}: max|diff| {err} rel-L2 {rel}"


# A single velocity is a bare head output: no noise term dilutes the bf16
# activation roundings, whose floor at the full expert shape is rel-L2
# 1.4e-2 - 1.6e-2 (a float32 emulation of the bf16 rounding points against the
# fp64 oracle; the rounding of the residual stream's bf16 copy alone gives
# 1.06e-2).  Velocities are held to twice the loop's bar.
HEAD_BAR = dict(max_abs=6e-2, max_rel=2e-2)


class B1:
    def __init__(self, seed=41, use_graphs=True, prefix_len=816):
        from vla_flow_matching_amd import binding
        self.w = W1.replace(name=f"pi0_bf16_b1_s{seed}", seed=seed, prefix_len=prefix_len)
        self.blob = synth.make_weights(self.w.shape, seed=seed, dtype="bf16")
        self.inputs = synth.make_inputs(self.w)
        cfg = binding.make_config(self.w.shape, "bf16", max_batch=1, max_prefix_len=1024, max_steps=16,
                                  use_graphs=use_graphs)
        _say(f"create pi0 bf16 B=1 seed={seed} graphs={use_graphs}")
        self.ex = binding.Expert(cfg, self.blob)
        self.dev = binding.device_inputs(self.inputs, "bf16")
        self.orc = oracle.Oracle(self.w.shape, self.blob)

    def run(self, n, dev=None):
        d = dev or self.dev
        _say(f"denoise B=1 valid={int(d['valid_len'][0])} N={n}")
        out = self.ex.denoise(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], n)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def ref(self, n, valid=None):
        inp = dict(self.inputs)
        if valid is not None:
            inp["valid_len"] = np.array([valid], np.int32)
        return self.orc.denoise_batch(inp, n)

    def with_valid(self, v, nan_pad=False):
        d = dict(self.dev)
        d["valid_len"] = torch.full((1,), v, dtype=torch.int32, device="cuda")
        if nan_pad:
            kv = d["prefix_kv"].clone()
            kv[:, :, 0, v:] = float("nan")
            d["prefix_kv"] = kv
        return d

    def close(self):
        self.ex.close()


@pytest.fixture(scope="module")
def b1():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = B1()
    yield c
    c.close()


@pytest.mark.parametrize("valid", [816, 700, 65, 64, 1, 0])
def test_valid_lengths_against_oracle(b1, valid):
    # whole key blocks, a partial last block, exactly one block, one key, and
    # no prefix at all (the state token then attends only to itself); the
    # 10-step loop the bf16 bar is stated for (with 2 steps each velocity's
    # bf16 error enters with weight 1/2 and the floor sits at the bar)
    out = b1.run(10, b1.with_valid(valid))
    check_close(out, b1.ref(10, valid), f"pi0 bf16 B=1 valid {valid} N=10")


def test_padded_keys_are_never_read(b1):
    a = b1.run(2, b1.with_valid(700))
    b = b1.run(2, b1.with_valid(700, nan_pad=True))
    assert np.array_equal(a, b), "NaN in the padded keys must not reach the output"


def test_repeated_calls_are_bitwise_stable(b1):
    a = b1.run(3)
    for _ in range(3):
        assert np.array_equal(b1.run(3), a)


def test_graph_replay_equals_eager(b1):
    eager = B1(use_graphs=False)
    try:
        assert np.array_equal(eager.run(3), b1.run(3))
    finally:
        eager.close()


def test_velocity_matches_oracle(b1):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, W1.shape.horizon, W1.shape.action_dim)).astype(np.float32)
    d = b1.dev
    for t in (1.0, 0.3):
        _say(f"denoise_step B=1 t={t}")
        v = b1.ex.denoise_step(d["prefix_kv"], d["valid_len"], d["state"], torch.from_numpy(x).cuda(), t)
        torch.cuda.synchronize()
        ref = b1.orc.velocity(b1.inputs["state"][0], x[0], float(np.float32(t)), b1.inputs["prefix_kv"][:, :, 0],
                              W1.prefix_len, W1.prefix_len)
        check_close(v.cpu().numpy()[0], ref, f"pi0 bf16 B=1 velocity t={t}", **HEAD_BAR)


def test_longest_prefix_seventeen_key_blocks():
    c = B1(seed=43, prefix_len=1024)
    try:
        check_close(c.run(10), c.ref(10), "pi0 bf16 B=1 L=1024 N=10")
    finally:
        c.close()
