"""Pins of the prefix-pass oracle (page 1, _compute_layer_prefix_only and the
prefix-only branch of PaliGemmaWithExpertModel.forward as sample_actions
calls it) to things other than itself: the second torch formulation built
from the Hugging Face Gemma modules with the page's additive mask, a
uniform-attention closed form, padding invariance, rotary shift invariance
and truncation to the real rows."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import oracle
from vla_flow_matching_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")

S = synth.TINY_VLM
LL = synth.layer_layout


def _blob(seed=0, shape=S, **kw):
    return synth.make_prefill_weights(shape, seed=seed, **kw).astype(np.float64)


def _inputs(seed=0, batch=1, L=40, valid=None, shape=S):
    w = synth.PrefillWorkload("t", shape, "fp32", batch, L, seed=seed)
    inp = synth.make_prefill_inputs(w)
    if valid is not None:
        inp["valid_len"][:] = valid
    return inp


@pytest.mark.parametrize("valid", [[40, 17], [40, 40], [1, 0]])
def test_prefill_matches_page_formulation(valid):
    from tests.page_formulation import PrefixFormulation
    blob = synth.make_prefill_weights(S, seed=3, norm_std=0.2)
    inp = _inputs(seed=4, batch=2, valid=valid)
    ref = PrefixFormulation(S, blob).prefill(inp)
    ours = oracle.PrefillOracle(S, blob).prefill_batch(inp)
    for b, v in enumerate(valid):
        assert np.max(np.abs(ours[:, :, b, :v] - ref[:, :, b, :v]), initial=0.0) < 1e-11
        assert not np.any(ours[:, :, b, v:])


def test_prefill_gqa_two_kv_heads_matches_page_formulation():
    from tests.page_formulation import PrefixFormulation
    s = synth.ExpertShape(width=128, depth=2, mlp_dim=256, num_heads=4, num_kv_heads=2, head_dim=32)
    blob = synth.make_prefill_weights(s, seed=5, norm_std=0.1)
    inp = _inputs(seed=6, batch=2, L=12, valid=[12, 7], shape=s)
    ref = PrefixFormulation(s, blob).prefill(inp)
    ours = oracle.PrefillOracle(s, blob).prefill_batch(inp)
    assert np.max(np.abs(ours[:, :, 0] - ref[:, :, 0])) < 1e-11
    assert np.max(np.abs(ours[:, :, 1, :7] - ref[:, :, 1, :7])) < 1e-11


def test_layer0_cache_is_projection_of_normalized_embeddings():
    # layer 0's cache does not depend on attention: k = RoPE_r(W_k rmsnorm(e_r)),
    # v = W_v rmsnorm(e_r); with norm weights 0 the norm is e / rms(e).
    blob = _blob(seed=7)
    inp = _inputs(seed=8, L=16)
    kv = oracle.PrefillOracle(S, blob).prefill(inp["embeddings"][0], 16)
    e = inp["embeddings"][0].astype(np.float64)
    y = e / np.sqrt(np.mean(e * e, axis=1, keepdims=True) + S.rms_eps)
    k = y @ synth.view(blob, S, "layers.0.k_proj", LL).T
    v = y @ synth.view(blob, S, "layers.0.v_proj", LL).T
    assert np.allclose(kv[0, 1, :, 0], v, atol=1e-13)
    for r in range(16):
        assert np.allclose(kv[0, 0, r, 0], oracle.rope(k[r], r, S.rope_theta), atol=1e-13)


def test_uniform_attention_closed_form():
    # W_q = 0 in layer 0 => every score is 0 => each real row's attention output
    # is the plain mean of the real rows' values (bidirectional, padding
    # excluded).  With layer 0's MLP zeroed, h1_r = e_r + W_o mean_j(v_j) for
    # every real row, and layer 1's values are W_v1 rmsnorm(h1_r).
    blob = _blob(seed=9)
    for name in ("q_proj", "gate_proj", "up_proj", "down_proj"):
        synth.view(blob, S, f"layers.0.{name}", LL)[...] = 0.0
    valid = 13
    inp = _inputs(seed=10, L=20, valid=valid)
    kv = oracle.PrefillOracle(S, blob).prefill(inp["embeddings"][0], valid)
    v0 = kv[0, 1, :valid, 0]
    mean = v0.mean(axis=0)
    o = np.tile(mean, S.num_heads)  # every head attends with the same weights to the one kv head
    e = inp["embeddings"][0, :valid].astype(np.float64)
    h1 = e + (synth.view(blob, S, "layers.0.o_proj", LL) @ o)[None]
    y = h1 / np.sqrt(np.mean(h1 * h1, axis=1, keepdims=True) + S.rms_eps)
    v1 = y @ synth.view(blob, S, "layers.1.v_proj", LL).T
    assert np.allclose(kv[1, 1, :valid, 0], v1, atol=1e-12)


def test_padded_rows_never_reach_real_rows():
    blob = _blob(seed=11, norm_std=0.1)
    inp = _inputs(seed=12, L=24, valid=15)
    o = oracle.PrefillOracle(S, blob)
    ref = o.prefill(inp["embeddings"][0], 15)
    e = inp["embeddings"][0].copy()
    e[15:] = np.nan
    assert np.array_equal(o.prefill(e, 15), ref)


def test_truncation_to_real_rows():
    # the real rows' cache does not depend on how much padding follows
    blob = _blob(seed=13, norm_std=0.1)
    inp = _inputs(seed=14, L=30, valid=21)
    o = oracle.PrefillOracle(S, blob)
    full = o.prefill(inp["embeddings"][0], 21)
    short = o.prefill(inp["embeddings"][0, :21], 21)
    assert np.array_equal(full[:, :, :21], short)


def test_rotary_shift_rotates_keys_only():
    # shifting every position by c leaves all scores unchanged (relative
    # rotary invariance), so hidden states and values are unchanged and each
    # cached key is the unshifted one rotated by c more.
    blob = _blob(seed=15, norm_std=0.1)
    inp = _inputs(seed=16, L=18, valid=18)
    o = oracle.PrefillOracle(S, blob)
    ref = o.prefill(inp["embeddings"][0], 18)
    for c in (3.0, 250.0):
        sh = o.prefill(inp["embeddings"][0], 18, pos_shift=c)
        assert np.allclose(sh[:, 1], ref[:, 1], atol=1e-11)
        for l in range(S.depth):
            for r in range(18):
                assert np.allclose(sh[l, 0, r, 0], oracle.rope(ref[l, 0, r, 0], c, S.rope_theta), atol=1e-11)


def test_layer_function_matches_prefill_steps():
    # prefill = the layer function applied depth times at positions 0..n-1
    blob = _blob(seed=17, norm_std=0.1)
    inp = _inputs(seed=18, L=10, valid=10)
    o = oracle.PrefillOracle(S, blob)
    kv = o.prefill(inp["embeddings"][0], 10)
    h = inp["embeddings"][0].astype(np.float64)
    for l in range(S.depth):
        h, k, v = o.layer(l, h, np.arange(10.0))
        assert np.array_equal(kv[l, 0, :, 0], k) and np.array_equal(kv[l, 1, :, 0], v)
