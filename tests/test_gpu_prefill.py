"""The prefix pass (page 1, _compute_layer_prefix_only and the prefix-only
branch of PaliGemmaWithExpertModel.forward) through pi0x_prefill against the
fp64 oracle, on the real rows of every layer's K/V cache.

Bars: float32 max|diff| <= 1e-4.  bfloat16: relative L2 <= 1e-2 and
max |diff| / max(1, |ref|) <= 3e-2 -- the loop's bf16 bar with the absolute
part scaled by the entry's magnitude: the cache is stored in bfloat16 and its
keys reach |k| ~ 7, where one bfloat16 step is 2^-5, so rounding the stored
value alone can cost up to 0.016 in absolute terms.  Through all 18 layers of
the 2B stack the bfloat16 activation roundings accumulate (relative L2 grows
about as sqrt(layer), to ~1e-2 at the last layer); there the elementwise bar
follows from the L2 bar: the largest of N ~ 4e5 errors of RMS e is about
e * sqrt(2 ln N) ~ 5 e, so max |diff| / max(1, |ref|) <= 5e-2.  The action
chunk computed from that cache is held to the loop's own bar."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest

from oracle import oracle
from vla_flow_matching_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def check_close(gpu, ref, dtype, what="", max_scaled=3e-2):
    """gpu, ref: [depth][2][rows][dh] caches (per-layer errors are printed)."""
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    d = np.abs(gpu - ref)
    err = float(np.max(d))
    scaled = float(np.max(d / np.maximum(1.0, np.abs(ref))))
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30))
    _say(f"{what}: max|diff| {err:.3e} scaled {scaled:.3e} rel-L2 {rel:.3e}")
    if gpu.ndim == 4:
        per = [np.linalg.norm(gpu[l] - ref[l]) / max(np.linalg.norm(ref[l]), 1e-30) for l in range(gpu.shape[0])]
        _say(f"{what}: rel-L2 per layer " + " ".join(f"{x:.1e}" for x in per))
    if dtype == "fp32":
        assert err <= 1e-4, f"{what}: max|diff| {err}"
    else:
        assert scaled <= max_scaled and rel <= 1e-2, f"{what}: scaled max|diff| {scaled} rel-L2 {rel}"


def real_rows(cache, valid):
    """Concatenate the real rows of every sample: [depth][2][sum v][dh]."""
    parts = [cache[:, :, b, :v].reshape(cache.shape[0], 2, v, cache.shape[-1]) for b, v in enumerate(valid)]
    return np.concatenate(parts, axis=2)


class Case:
    def __init__(self, w: synth.PrefillWorkload, norm_std=0.1, valid=None, use_graphs=True):
        from vla_flow_matching_amd import binding
        self.w = w
        self.blob = synth.make_prefill_weights(w.shape, seed=w.seed, dtype=w.dtype, norm_std=norm_std)
        self.inputs = synth.make_prefill_inputs(w)
        if valid is not None:
            self.inputs["valid_len"][:] = valid
        cfg = binding.make_config(w.shape, w.dtype, max_batch=w.batch, max_prefix_len=w.prefix_len,
                                  use_graphs=use_graphs)
        _say(f"create prefix model {w.name} dtype={w.dtype} B={w.batch} L={w.prefix_len} graphs={use_graphs}")
        self.pm = binding.PrefixModel(cfg, self.blob)
        self.dev = binding.prefill_device_inputs(self.inputs, w.dtype)

    def run(self, dev=None):
        d = dev or self.dev
        _say(f"prefill {self.w.name} valid={list(self.inputs['valid_len'])}")
        out = self.pm.prefill(d["embeddings"], d["valid_len"])
        torch.cuda.synchronize()
        return out.float().cpu().numpy()

    def ref(self, samples=None):
        """[depth][2][B][L][head_dim] (the single kv head), as the boundary lays it out."""
        r = oracle.PrefillOracle(self.w.shape, self.blob).prefill_batch(self.inputs, samples=samples)
        return r.reshape(r.shape[:4] + (-1,))

    def close(self):
        self.pm.close()


TINY = synth.PREFILL_WORKLOADS["tiny_prefill_fp32"]


@pytest.fixture(scope="module")
def tiny():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = Case(TINY)
    yield c
    c.close()


def test_tiny_fp32_prefill_parity(tiny):
    out = tiny.run()
    check_close(real_rows(out, [96]), real_rows(tiny.ref(), [96]), "fp32", "tiny prefill fp32 B=1 L=96")


def test_tiny_graph_replay_bitwise_and_equal_to_eager(tiny):
    a = tiny.run()
    assert np.array_equal(tiny.run(), a)
    eager = Case(TINY, use_graphs=False)
    try:
        assert np.array_equal(eager.run(), a)
    finally:
        eager.close()


def test_tiny_fp32_ragged_and_nan_padding():
    # 4 x 96 rows (the float32 tile GEMMs); valid lengths down to 1 and 0
    w = TINY.replace(name="tiny_prefill_ragged", batch=4, seed=3)
    valid = [96, 41, 1, 0]
    c = Case(w, valid=valid)
    try:
        out = c.run()
        check_close(real_rows(out, valid), real_rows(c.ref(), valid), "fp32", "tiny prefill fp32 ragged")
        emb = c.dev["embeddings"].clone()
        for b, v in enumerate(valid):
            emb[b, v:] = float("nan")
        d2 = dict(c.dev)
        d2["embeddings"] = emb
        assert np.array_equal(real_rows(c.run(dev=d2), valid), real_rows(out, valid)), \
            "padded embeddings must never reach a real row"
    finally:
        c.close()


def test_tiny_bf16_small_rows_path():
    # 40 rows: the batch-1 bf16 kernels (one-kernel wide GEMMs, K-split residual producers)
    w = TINY.replace(name="tiny_prefill_bf16_b1", dtype="bf16", prefix_len=40, seed=5)
    c = Case(w, valid=[33])
    try:
        out = c.run()
        check_close(real_rows(out, [33]), real_rows(c.ref(), [33]), "bf16", "tiny prefill bf16 40 rows")
    finally:
        c.close()


def test_tiny_bf16_tile_path_ragged():
    w = TINY.replace(name="tiny_prefill_bf16_b3", dtype="bf16", batch=3, seed=7)
    valid = [96, 50, 0]
    c = Case(w, valid=valid)
    try:
        out = c.run()
        check_close(real_rows(out, valid), real_rows(c.ref(), valid), "bf16", "tiny prefill bf16 B=3 ragged")
    finally:
        c.close()


def test_prefill_feeds_denoise():
    # the cache the prefix pass writes is the denoise loop's prefix_kv: prefill
    # then denoise on the GPU against the oracle's prefill then denoise
    from vla_flow_matching_amd import binding
    vlm = synth.ExpertShape(width=512, depth=2, mlp_dim=1536, num_heads=8, num_kv_heads=1, head_dim=32)
    pw = synth.PrefillWorkload("tiny_prefill_e2e", vlm, "fp32", 2, 64, seed=9)
    c = Case(pw, valid=[64, 37])
    ew = synth.WORKLOADS["tiny_fp32_b1"].replace(batch=2, seed=10)
    eblob = synth.make_weights(ew.shape, seed=ew.seed, norm_std=0.1)
    einp = synth.make_inputs(ew)
    ex = binding.Expert(binding.make_config(ew.shape, "fp32", max_batch=2, max_prefix_len=64), eblob)
    try:
        kv = c.pm.prefill(c.dev["embeddings"], c.dev["valid_len"])
        d = binding.device_inputs(einp, "fp32")
        _say("denoise on the prefilled cache")
        out = ex.denoise(kv, c.dev["valid_len"], d["state"], d["noise"], 2)
        torch.cuda.synchronize()
        einp = dict(einp)
        einp["prefix_kv"] = c.ref()
        einp["valid_len"] = c.inputs["valid_len"]
        ref = oracle.Oracle(ew.shape, eblob).denoise_batch(einp, 2)
        check_close(out.cpu().numpy(), ref, "fp32", "prefill -> denoise end to end")
    finally:
        ex.close()
        c.close()


def test_prefill_argument_errors(tiny):
    from vla_flow_matching_amd import binding as b
    d = tiny.dev
    kv = torch.empty((TINY.shape.depth, 2, 1, TINY.prefix_len, TINY.shape.head_dim), device="cuda")
    e, v = d["embeddings"].data_ptr(), d["valid_len"].data_ptr()
    assert b.pi0x_prefill(tiny.pm.h, 2, TINY.prefix_len, e, v, kv.data_ptr(), None) == b.PI0X_ERR_CAPACITY
    assert b.pi0x_prefill(tiny.pm.h, 1, TINY.prefix_len + 1, e, v, kv.data_ptr(), None) == b.PI0X_ERR_CAPACITY
    assert b.pi0x_prefill(tiny.pm.h, 0, TINY.prefix_len, e, v, kv.data_ptr(), None) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_prefill(tiny.pm.h, 1, TINY.prefix_len, e, v, kv.data_ptr() + 4, None) == b.PI0X_ERR_INVALID_ARG
    assert "aligned" in b.pi0x_last_error()
    assert b.pi0x_prefill(tiny.pm.h, 1, TINY.prefix_len, None, v, kv.data_ptr(), None) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_prefill(tiny.pm.h, 1, 0, e, v, kv.data_ptr(), None) == b.PI0X_OK


# ---------------------------------------------------------------------------
# The Gemma-2B prefix stack
# ---------------------------------------------------------------------------
def test_gemma_2b_two_layers_full_prefix_bf16():
    # full width (2048, mlp 16384) and the full 816-token prefix, two layers
    # (layer 0 complete, layer 1 up to its K/V): every row is real
    s = dataclasses.replace(synth.GEMMA_2B, depth=2)
    w = synth.PrefillWorkload("gemma2b_d2_bf16_b1", s, "bf16", 1, 816, seed=11)
    c = Case(w, norm_std=0.0)
    try:
        out = c.run()
        check_close(real_rows(out, [816]), real_rows(c.ref(), [816]), "bf16", "gemma-2b depth 2, 816 real tokens")
    finally:
        c.close()


def test_gemma_2b_two_layers_batched_ragged_bf16():
    # full width, batch 4 of a 256-token padded prefix with ragged real lengths:
    # 1024 GEMM rows (the K-split down projection over 8 row tiles), 4 samples
    # of attention, NaN in every padded embedding
    s = dataclasses.replace(synth.GEMMA_2B, depth=2)
    w = synth.PrefillWorkload("gemma2b_d2_bf16_b4", s, "bf16", 4, 256, seed=17)
    valid = [256, 200, 131, 40]
    c = Case(w, norm_std=0.0, valid=valid)
    try:
        emb = c.dev["embeddings"].clone()
        for b, v in enumerate(valid):
            emb[b, v:] = float("nan")
        d2 = dict(c.dev)
        d2["embeddings"] = emb
        out = c.run(dev=d2)
        check_close(real_rows(out, valid), real_rows(c.ref(), valid), "bf16", "gemma-2b depth 2, B=4 ragged")
    finally:
        c.close()


def test_gemma_2b_full_depth_short_prefix_bf16():
    # all 18 layers at full width over an 816-row padded prefix with 48 real
    # tokens (the padded rows run through the same kernels and are never read)
    w = synth.PREFILL_WORKLOADS["paligemma_bf16_b1"].replace(name="gemma2b_bf16_v48", seed=13)
    c = Case(w, norm_std=0.0, valid=[48])
    try:
        out = c.run()
        check_close(real_rows(out, [48]), real_rows(c.ref(), [48]), "bf16", "gemma-2b 18 layers, 48 real of 816",
                    max_scaled=5e-2)
    finally:
        c.close()


def test_gemma_2b_prefill_then_pi0_denoise_bf16():
    # the whole observation -> action path at full size: the 18-layer 2B prefix
    # pass (64 real tokens of 816) writes the cache, the 300M expert denoises
    # 10 steps from it; the action chunk against the oracle's prefill + denoise
    # under the loop's bf16 bar
    from vla_flow_matching_amd import binding
    pw = synth.PREFILL_WORKLOADS["paligemma_bf16_b1"].replace(name="gemma2b_bf16_v64_e2e", seed=15)
    c = Case(pw, norm_std=0.0, valid=[64])
    ew = synth.WORKLOADS["pi0_bf16_b1"].replace(seed=16)
    eblob = synth.make_weights(ew.shape, seed=ew.seed, dtype="bf16")
    einp = synth.make_inputs(ew)
    ex = binding.Expert(binding.make_config(ew.shape, "bf16", max_batch=1, max_prefix_len=816), eblob)
    try:
        kv = c.pm.prefill(c.dev["embeddings"], c.dev["valid_len"])
        d = binding.device_inputs(einp, "bf16")
        _say("pi0 denoise on the gemma-2b cache")
        out = ex.denoise(kv, c.dev["valid_len"], d["state"], d["noise"], ew.num_steps)
        torch.cuda.synchronize()
        einp = dict(einp)
        einp["prefix_kv"] = c.ref()
        einp["valid_len"] = c.inputs["valid_len"]
        ref = oracle.Oracle(ew.shape, eblob).denoise_batch(einp, ew.num_steps)
        check_close(out.cpu().numpy(), ref, "bf16", "gemma-2b prefill -> pi0 denoise, actions")
    finally:
        ex.close()
        c.close()


def test_gemma_2b_benched_shape_816_real_tokens_bf16():
    """The prefix pass at the shape bench.py times: all 18 Gemma-2B layers over
    816 real tokens.  The fp64 oracle needs minutes for it, so its results were
    stored by tests/golden/make_oracle_golden.py (the oracle alone): the cache
    at 32 rows of every layer, and the action chunk the 10-step expert denoise
    computes from the oracle's cache.  Layer 0's rows are recomputed live, so a
    stale stored file fails here.  The GPU's own cache then feeds the GPU
    denoise, whose chunk is held to the loop's bf16 bar."""
    import os
    from vla_flow_matching_amd import binding
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    import make_oracle_golden as mg
    gold = np.load(mg.PREFILL_FILE)
    pw, ew = mg.prefill_workloads()
    rows = gold["rows"]
    assert np.array_equal(rows, mg.prefill_rows(pw.prefix_len))
    c = Case(pw, norm_std=0.0)
    try:
        _say("prefill gemma-2b, 18 layers, 816 real tokens")
        kv = c.pm.prefill(c.dev["embeddings"], c.dev["valid_len"])
        torch.cuda.synchronize()
        got = kv.float().cpu().numpy()[:, :, 0]  # [depth][2][L][dh]
        ref = gold["cache_rows"].astype(np.float64)  # [depth][2][rows][dh]
        # the stored layer-0 rows against a live oracle layer 0 (the embeddings are the layer's input)
        po = oracle.PrefillOracle(pw.shape, c.blob)
        emb = c.inputs["embeddings"][0].astype(np.float64)
        _, k0, v0 = po.layer(0, emb, np.arange(pw.prefix_len, dtype=np.float64))
        live0 = np.stack([k0[rows], v0[rows]])
        d = float(np.max(np.abs(live0 - ref[0])))
        _say(f"stored vs live oracle, layer 0: max|diff| {d:.2e}")
        assert d <= 1e-5, "the stored prefix-pass oracle result is stale"
        check_close(got[:, :, rows], ref, "bf16", "gemma-2b 18 layers, 816 real tokens (32 stored rows per layer)",
                    max_scaled=5e-2)
        # the cache feeds the expert: GPU prefill -> GPU denoise vs oracle prefill -> oracle denoise
        eblob = synth.make_weights(ew.shape, seed=ew.seed, dtype="bf16")
        einp = synth.make_inputs(ew)
        ex = binding.Expert(binding.make_config(ew.shape, "bf16", max_batch=1, max_prefix_len=816), eblob)
        try:
            d = binding.device_inputs(einp, "bf16")
            _say("pi0 denoise on the 816-token gemma-2b cache")
            out = ex.denoise(kv, c.dev["valid_len"], d["state"], d["noise"], ew.num_steps)
            torch.cuda.synchronize()
        finally:
            ex.close()
        got_a = out.cpu().numpy().astype(np.float64)
        ref_a = gold["actions"].astype(np.float64)
        err = float(np.max(np.abs(got_a - ref_a)))
        rel = float(np.linalg.norm(got_a - ref_a) / np.linalg.norm(ref_a))
        _say(f"gemma-2b 816-token prefill -> pi0 denoise, actions: max|diff| {err:.3e} rel-L2 {rel:.3e}")
        assert np.all(np.isfinite(got_a)) and err <= 3e-2 and rel <= 1e-2, (err, rel)
    finally:
        c.close()
