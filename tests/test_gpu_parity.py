"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Bars (fixed for the pi0 denoise loop): float32 mode max|diff| <= 1e-4 (the
pages' own parity bar); bfloat16 mode max|diff| <= 3e-2 and relative L2
<= 1e-2.  Inputs are the seeded synthetic workloads; bfloat16 cases feed the
oracle the same bf16-rounded weights and prefix K/V the GPU reads.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import oracle
from vla_flow_matching_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from vla_flow_matching_amd import binding
    binding.lib()  # fails loudly when the HIP library is missing
    yield


def check_close(gpu, ref, dtype, what=""):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = float(np.max(np.abs(gpu - ref)))
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30))
    _say(f"{what}: max|diff| {err:.3e} rel-L2 {rel:.3e}")
    if dtype == "fp32":
        assert err <= 1e-4, f"{what}: max|diff| {err}"
    else:
        assert err <= 3e-2 and rel <= 1e-2, f"{what}: max|diff| {err} rel-L2 {rel}"
    return err, rel


class Case:
    """A workload, its weights, the GPU handle and device inputs."""

    def __init__(self, w: synth.Workload, use_graphs=True, norm_std=0.0, max_batch=None):
        from vla_flow_matching_amd import binding
        self.w = w
        self.blob = synth.make_weights(w.shape, seed=w.seed, dtype=w.dtype, norm_std=norm_std)
        self.inputs = synth.make_inputs(w)
        cfg = binding.make_config(w.shape, w.dtype, max_batch=max_batch or w.batch,
                                  max_prefix_len=max(w.prefix_len, 64), max_steps=16, use_graphs=use_graphs)
        _say(f"create {w.name} dtype={w.dtype} B={w.batch} L={w.prefix_len} N={w.num_steps} graphs={use_graphs}")
        self.ex = binding.Expert(cfg, self.blob)
        self.dev = binding.device_inputs(self.inputs, w.dtype)
        self._oracle = None

    @property
    def oracle(self):
        if self._oracle is None:
            self._oracle = oracle.Oracle(self.w.shape, self.blob)
        return self._oracle

    def run(self, num_steps=None, dev=None, out=None):
        d = dev or self.dev
        _say(f"denoise {self.w.name} N={num_steps or self.w.num_steps}")
        r = self.ex.denoise(d["prefix_kv"], d["valid_len"], d["state"], d["noise"],
                            num_steps or self.w.num_steps, out=out)
        torch.cuda.synchronize()
        return r.cpu().numpy()

    def ref(self, samples=None, num_steps=None):
        return self.oracle.denoise_batch(self.inputs, num_steps or self.w.num_steps, samples=samples)


TINY = synth.WORKLOADS["tiny_fp32_b1"]


@pytest.fixture(scope="module")
def tiny():
    c = Case(TINY, norm_std=0.1)
    yield c
    c.ex.close()


def test_tiny_fp32_parity(tiny):
    check_close(tiny.run(), tiny.ref(), "fp32", "tiny fp32")


def test_tiny_graph_replay_bitwise_stable_and_equal_to_eager(tiny):
    a = tiny.run()
    b = tiny.run()
    assert np.array_equal(a, b)
    eager = Case(TINY, use_graphs=False, norm_std=0.1)
    try:
        assert np.array_equal(eager.run(), a)
    finally:
        eager.ex.close()


def test_tiny_velocity_matches_oracle(tiny):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, TINY.shape.horizon, TINY.shape.action_dim)).astype(np.float32)
    xt = torch.from_numpy(x).cuda()
    d = tiny.dev
    for t in (1.0, 0.37):
        _say(f"denoise_step tiny t={t}")
        v = tiny.ex.denoise_step(d["prefix_kv"], d["valid_len"], d["state"], xt, t)
        torch.cuda.synchronize()
        ref = tiny.oracle.velocity(tiny.inputs["state"][0], x[0], float(np.float32(t)),
                                   tiny.inputs["prefix_kv"][:, :, 0], TINY.prefix_len, TINY.prefix_len)
        check_close(v.cpu().numpy()[0], ref, "fp32", f"velocity t={t}")


def test_tiny_single_step_is_noise_minus_velocity(tiny):
    d = tiny.dev
    x1 = tiny.run(num_steps=1)
    v = tiny.ex.denoise_step(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], 1.0)
    torch.cuda.synchronize()
    assert np.array_equal(x1, (d["noise"] - v).cpu().numpy())


def test_tiny_output_may_alias_noise(tiny):
    ref = tiny.run()
    noise = tiny.dev["noise"].clone()
    d = dict(tiny.dev)
    d["noise"] = noise
    tiny.ex.denoise(d["prefix_kv"], d["valid_len"], d["state"], noise, TINY.num_steps, out=noise)
    torch.cuda.synchronize()
    assert np.array_equal(noise.cpu().numpy(), ref)


def test_tiny_new_buffers_replay_same_graph(tiny):
    ref = tiny.run()
    d2 = {k: v.clone() for k, v in tiny.dev.items()}
    assert np.array_equal(tiny.run(dev=d2), ref)


def test_tiny_ragged_valid_lengths_and_nan_padding():
    w = TINY.replace(name="tiny_ragged", batch=4, seed=5)
    c = Case(w, norm_std=0.1)
    try:
        c.inputs["valid_len"][:] = [64, 23, 1, 0]
        c.dev = __import__("vla_flow_matching_amd.binding", fromlist=["x"]).device_inputs(c.inputs, w.dtype)
        out = c.run()
        check_close(out, c.ref(), "fp32", "tiny ragged")
        kv = c.dev["prefix_kv"].clone()
        for b, v in enumerate(c.inputs["valid_len"]):
            kv[:, :, b, v:] = float("nan")
        d2 = dict(c.dev)
        d2["prefix_kv"] = kv
        assert np.array_equal(c.run(dev=d2), out), "padded prefix keys must never be read"
    finally:
        c.ex.close()


def test_tiny_batch_independence():
    w = TINY.replace(name="tiny_b3", batch=3, seed=7)
    c = Case(w, max_batch=3)
    try:
        out = c.run()
        from vla_flow_matching_amd import binding
        for b in range(3):
            single = {k: (v[b:b + 1] if k != "prefix_kv" else v[:, :, b:b + 1]) for k, v in c.inputs.items()}
            d = binding.device_inputs(single, w.dtype)
            r = c.ex.denoise(d["prefix_kv"], d["valid_len"], d["state"], d["noise"], w.num_steps)
            torch.cuda.synchronize()
            assert np.max(np.abs(r.cpu().numpy()[0] - out[b])) <= 1e-5
    finally:
        c.ex.close()


def test_tiny_bf16_parity():
    w = TINY.replace(name="tiny_bf16", dtype="bf16", seed=2)
    c = Case(w, norm_std=0.1)
    try:
        check_close(c.run(), c.ref(), "bf16", "tiny bf16")
    finally:
        c.ex.close()


def test_tiny_bf16_batch8_tile_gemm_path():
    # 8 x 9 = 72 suffix rows: the GEMMs take the tile kernel (more than 64 rows);
    # the tiny q/k/v projection has 320 outputs, the 128x64 tile variant
    w = TINY.replace(name="tiny_bf16_b8", dtype="bf16", batch=8, seed=11)
    c = Case(w, norm_std=0.1)
    try:
        out = c.run()
        ref = c.ref()
        for b in range(w.batch):
            check_close(out[b], ref[b], "bf16", f"tiny bf16 B=8 sample {b}")
    finally:
        c.ex.close()


def test_tiny_fp32_batch8_split_k_path():
    # 72 suffix rows in float32: the 128x64 float32 tiles with split K
    w = TINY.replace(name="tiny_fp32_b8", batch=8, seed=13)
    c = Case(w, norm_std=0.1)
    try:
        out = c.run()
        check_close(out, c.ref(), "fp32", "tiny fp32 B=8")
    finally:
        c.ex.close()


def test_tiny_bf16_zero_and_one_valid_prefix():
    # valid lengths 0 and 1: an empty prefix (the state token attends to itself
    # only) and a single key, through the bf16 batch-1-style kernels (18 rows)
    w = TINY.replace(name="tiny_bf16_v01", dtype="bf16", batch=2, seed=17)
    c = Case(w, norm_std=0.1)
    try:
        c.inputs["valid_len"][:] = [0, 1]
        from vla_flow_matching_amd import binding
        c.dev = binding.device_inputs(c.inputs, w.dtype)
        out = c.run()
        check_close(out, c.ref(), "bf16", "tiny bf16 valid 0 and 1")
        kv = c.dev["prefix_kv"].clone()
        kv[:, :, 0, 0:] = float("nan")
        kv[:, :, 1, 1:] = float("nan")
        d2 = dict(c.dev)
        d2["prefix_kv"] = kv
        assert np.array_equal(c.run(dev=d2), out), "padded prefix keys must never be read"
    finally:
        c.ex.close()


def test_graph_cache_eviction_records_again(tiny):
    """More distinct (prefix length, steps) keys than the handle keeps graphs
    for: the oldest graphs are destroyed and recorded again when their key
    comes back, with bitwise the same result."""
    d = tiny.dev
    keys = [(L, N) for L in (64, 40) for N in range(1, 17)] + [(24, 1), (24, 2), (24, 3)]
    assert len(keys) > 32
    first = {}
    for L, N in keys:
        kv = d["prefix_kv"][:, :, :, :L].contiguous()
        valid = torch.clamp(d["valid_len"], max=L)
        first[(L, N)] = tiny.ex.denoise(kv, valid, d["state"], d["noise"], N).cpu().numpy()
    _say(f"{len(keys)} graph keys recorded; replaying the evicted ones")
    for L, N in keys[:4]:
        kv = d["prefix_kv"][:, :, :, :L].contiguous()
        valid = torch.clamp(d["valid_len"], max=L)
        again = tiny.ex.denoise(kv, valid, d["state"], d["noise"], N).cpu().numpy()
        assert np.array_equal(again, first[(L, N)]), (L, N)
    check_close(first[(TINY.prefix_len, 1)], tiny.ref(num_steps=1), "fp32", "tiny fp32 N=1 after eviction")


def test_call_argument_errors(tiny):
    from vla_flow_matching_amd import binding as b
    d = tiny.dev
    args = lambda B, N: (tiny.ex.h, B, TINY.prefix_len, d["prefix_kv"].data_ptr(), d["valid_len"].data_ptr(),
                         d["state"].data_ptr(), d["noise"].data_ptr(), N, d["noise"].data_ptr(), None)
    assert b.pi0x_denoise(*args(1, 0)) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_denoise(*args(1, 17)) == b.PI0X_ERR_CAPACITY
    assert b.pi0x_denoise(*args(2, 2)) == b.PI0X_ERR_CAPACITY
    assert b.pi0x_denoise(*args(0, 2)) == b.PI0X_ERR_INVALID_ARG
    bad = list(args(1, 2))
    bad[3] += 4  # a misaligned prefix cache is rejected before anything is enqueued
    assert b.pi0x_denoise(*bad) == b.PI0X_ERR_INVALID_ARG
    assert "aligned" in b.pi0x_last_error()


# ---------------------------------------------------------------------------
# Full pi0 expert shapes
# ---------------------------------------------------------------------------
def test_full_fp32_b1_parity():
    c = Case(synth.WORKLOADS["pi0_fp32_b1"])
    try:
        out = c.run()
        check_close(out, c.ref(), "fp32", "pi0 fp32 B=1 L=816 N=10")
    finally:
        c.ex.close()


def test_full_bf16_b1_parity():
    c = Case(synth.WORKLOADS["pi0_bf16_b1"])
    try:
        out = c.run()
        check_close(out, c.ref(), "bf16", "pi0 bf16 B=1 L=816 N=10")
    finally:
        c.ex.close()


def test_full_bf16_b2_partial_row_tile_and_key_splits():
    # 102 suffix rows (one partial 128-row GEMM tile); 2 x 4 query tiles, so the
    # attention splits every sample's keys and merges the splits
    w = synth.WORKLOADS["pi0_bf16_b1"].replace(name="pi0_bf16_b2", batch=2, num_steps=2, seed=3)
    c = Case(w)
    try:
        out = c.run()
        ref = c.ref()
        for b in range(2):
            check_close(out[b], ref[b], "bf16", f"pi0 bf16 B=2 N=2 sample {b}")
    finally:
        c.ex.close()


def test_full_bf16_b1_longest_prefix():
    # prefix_len 1024 (the default max_prefix_len): 16 prefix key blocks + 1
    # suffix block, so attention splits the keys 17 ways and the combine
    # merges them in two batches of loads, carrying the running maximum over
    w = synth.WORKLOADS["pi0_bf16_b1"].replace(name="pi0_bf16_b1_l1024", prefix_len=1024, seed=4)
    c = Case(w)
    try:
        out = c.run()
        check_close(out, c.ref(), "bf16", "pi0 bf16 B=1 L=1024 N=10")
    finally:
        c.ex.close()


def test_full_bf16_b64_every_sample():
    """All 64 samples against the stored oracle results (tests/golden/
    make_oracle_golden.py, written by the fp64 oracle alone), and two samples
    recomputed live -- 2 straddles the first 128-row GEMM tile boundary, 37
    another -- so a stale stored file fails here."""
    import os
    gold = np.load(os.path.join(os.path.dirname(__file__), "golden", "pi0_bf16_b64_oracle.npz"))
    c = Case(synth.WORKLOADS["pi0_bf16_b64"])
    try:
        out = c.run()
        assert np.all(np.isfinite(out))
        ref_all = gold["actions"].astype(np.float64)
        live = [2, 37]
        ref_live = c.ref(samples=live)
        for i, b in enumerate(live):
            d = float(np.max(np.abs(ref_live[i] - ref_all[b])))
            _say(f"stored vs live oracle, sample {b}: max|diff| {d:.2e}")
            assert d <= 1e-5, f"the stored oracle result of sample {b} is stale ({d})"
        worst = (0.0, 0.0)
        for b in range(64):
            e, r = check_close(out[b], ref_all[b], "bf16", f"pi0 bf16 B=64 sample {b} (rows {51 * b}..{51 * b + 50})")
            worst = (max(worst[0], e), max(worst[1], r))
        _say(f"B=64 worst over samples: max|diff| {worst[0]:.3e} rel-L2 {worst[1]:.3e}")
        check_close(out, ref_all, "bf16", "pi0 bf16 B=64 whole batch")
    finally:
        c.ex.close()


def test_fp32_action_rows_gemm_uses_the_path_tile():
    # batch 120 of the tiny shape: 960 action rows (<= 1024) but 1080 suffix
    # rows (> 1024).  The action-row MLP output must write its sum-of-squares
    # partials in the column groups the first layer's norm reads for 1080 rows.
    w = TINY.replace(name="tiny_fp32_b120", batch=120, seed=19)
    c = Case(w, norm_std=0.1)
    try:
        out = c.run()
        ref = c.ref()
        for b in range(w.batch):
            err = float(np.max(np.abs(out[b] - ref[b])))
            assert err <= 1e-4, f"sample {b}: max|diff| {err}"
        check_close(out, ref, "fp32", "tiny fp32 B=120 (960 action rows, 1080 suffix rows)")
    finally:
        c.ex.close()


def test_ragged_bf16_b16_parity_and_padding():
    w = synth.WORKLOADS["pi0_bf16_b16_ragged"]
    c = Case(w)
    try:
        out = c.run()
        v = c.inputs["valid_len"]
        ref = c.ref()  # every sample against its own oracle run
        for b in range(w.batch):
            check_close(out[b], ref[b], "bf16", f"ragged B=16 sample {b} valid {v[b]}")
        check_close(out, ref, "bf16", "ragged B=16 whole batch")
        kv = c.dev["prefix_kv"].clone()
        for b in range(w.batch):
            kv[:, :, b, int(v[b]):] = float("nan")
        d2 = dict(c.dev)
        d2["prefix_kv"] = kv
        assert np.array_equal(c.run(dev=d2), out)
    finally:
        c.ex.close()
