"""The configuration constants the page prints (tests/golden/pi0_page_constants.json,
each entry naming the part of page 1 that fixes it) against the synthetic
workloads, the C ABI defaults and the oracle."""
from __future__ import annotations

import json
import os

import numpy as np

from oracle import oracle
from vla_flow_matching_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
C = {k: v["value"] for k, v in json.load(open(os.path.join(HERE, "golden", "pi0_page_constants.json")))["constants"].items()}


def test_expert_shape_is_gemma_300m():
    s = synth.GEMMA_300M
    assert [s.width, s.depth, s.mlp_dim, s.num_heads, s.num_kv_heads, s.head_dim] == C["gemma_300m"]
    assert s.horizon == C["action_horizon"] and s.action_dim == C["action_dim"]
    assert (s.min_period, s.max_period) == (C["time_min_period"], C["time_max_period"])


def test_workload_prefix_is_three_cameras_plus_text():
    L = 3 * C["image_tokens_per_camera"] + C["max_text_tokens"]
    assert L == 816
    for name in ("pi0_fp32_b1", "pi0_bf16_b1", "pi0_bf16_b64"):
        w = synth.WORKLOADS[name]
        assert w.prefix_len == L and w.num_steps == C["num_inference_steps"]
    r = synth.WORKLOADS["pi0_bf16_b16_ragged"]
    assert r.prefix_len == 2 * C["image_tokens_per_camera"] + C["max_text_tokens"]


def test_abi_defaults_match_page():
    from vla_flow_matching_amd import binding
    cfg = binding.pi0x_config()
    binding.lib().pi0x_config_default(cfg)
    assert [cfg.width, cfg.depth, cfg.mlp_dim, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim] == C["gemma_300m"]
    assert cfg.action_horizon == C["action_horizon"] and cfg.action_dim == C["action_dim"]
    assert np.float32(cfg.time_min_period) == np.float32(C["time_min_period"])
    assert cfg.time_max_period == C["time_max_period"]


def test_sinusoid_uses_page_periods():
    # the lowest frequency 2 pi / max_period and the highest 2 pi / min_period
    W = 1024
    for t in (0.25, 0.7):
        tau = oracle.sinusoid(t, W, C["time_min_period"], C["time_max_period"])
        assert abs(tau[0] - np.sin(2 * np.pi * t / C["time_min_period"])) < 1e-12
        assert abs(tau[W // 2 - 1] - np.sin(2 * np.pi * t / C["time_max_period"])) < 1e-12


def test_masked_scores_underflow_to_exact_zero():
    # skipping masked keys (instead of adding the page's fill value) is exact:
    # the filled score's exponential is exactly 0 in float32 and float64
    m = C["attention_mask_value"]
    for dt in (np.float32, np.float64):
        for s in (-50.0, 0.0, 80.0):
            x = dt(m) + dt(s)
            assert np.exp(x - dt(s)) == 0.0 and np.exp(x - dt(-50.0)) == 0.0


def test_suffix_mask_flags_give_the_block_causal_rule():
    # cumulative-sum rule of make_att_2d_masks with flags [1, 1, 0, ...]: key j is
    # visible to query i iff cumsum[j] <= cumsum[i]
    H = 5
    flags = C["suffix_ar_flags_head"][:2] + [0] * (H - 1)
    cs = np.cumsum(flags)
    vis = cs[None, :] <= cs[:, None]
    assert vis[0].tolist() == [True] + [False] * H          # the state token sees itself only
    assert all(vis[i].all() for i in range(1, H + 1))        # every action token sees the whole suffix
