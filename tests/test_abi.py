"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/pi0x.h declares, and rejects bad arguments before it
touches the device."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from vla_flow_matching_amd import binding as b
from vla_flow_matching_amd import synth


def test_library_exports_every_declared_function():
    names = b.declared_functions()
    assert set(names) == {"pi0x_config_default", "pi0x_weight_count", "pi0x_expert_create", "pi0x_denoise",
                          "pi0x_denoise_noalloc", "pi0x_denoise_step", "pi0x_expert_destroy", "pi0x_last_error", "pi0x_set_timing",
                          "pi0x_read_timing", "pi0x_set_normalization", "pi0x_denoise_ex",
                          "pi0x_prefix_config_default", "pi0x_prefix_weight_count", "pi0x_prefix_create",
                          "pi0x_prefill", "pi0x_prefix_destroy", "pi0x_prefix_set_timing",
                          "pi0x_prefix_read_timing", "pi0x_expert_check_guards", "pi0x_prefix_check_guards",
                          "pi0x_debug_velocity_until"}
    lib = b.lib()
    for n in names:
        assert getattr(lib, n) is not None


def test_config_default_is_pi0_expert():
    c = b.pi0x_config_default()
    s = synth.GEMMA_300M
    assert (c.width, c.depth, c.mlp_dim, c.num_heads, c.num_kv_heads, c.head_dim) == (1024, 18, 4096, 8, 1, 256)
    assert (c.action_horizon, c.action_dim, c.state_dim) == (s.horizon, s.action_dim, s.state_dim)
    assert c.rms_eps == pytest.approx(1e-6) and c.rope_theta == 10000.0
    assert c.time_min_period == pytest.approx(4e-3) and c.time_max_period == 4.0
    assert c.dtype == b.PI0X_BF16 and c.use_graphs == 1


@pytest.mark.parametrize("shape", [synth.GEMMA_300M, synth.TINY])
def test_weight_count_matches_blob_layout(shape):
    assert b.pi0x_weight_count(b.make_config(shape)) == synth.weight_count(shape)


def test_weight_count_full_expert():
    # 18 layers x 17,303,552 + final norm 1024 + head 3,248,160
    assert synth.weight_count(synth.GEMMA_300M) == 314_713_120


def _create(cfg, nvals=None):
    n = b.pi0x_weight_count(cfg) if nvals is None else nvals
    w = np.zeros(max(n, 1), np.float32)
    return b.pi0x_expert_create(cfg, w.ctypes.data, 4 * n)


@pytest.mark.parametrize("field,value,status", [
    ("num_kv_heads", 2, b.PI0X_ERR_SHAPE),
    ("head_dim", 48, b.PI0X_ERR_SHAPE),
    ("width", 320, b.PI0X_ERR_SHAPE),
    ("action_dim", 65, b.PI0X_ERR_SHAPE),
    ("dtype", 7, b.PI0X_ERR_DTYPE),
    ("depth", 0, b.PI0X_ERR_INVALID_ARG),
    ("max_batch", 0, b.PI0X_ERR_INVALID_ARG),
    ("max_steps", -1, b.PI0X_ERR_INVALID_ARG),
])
def test_create_rejects_bad_config(field, value, status):
    cfg = b.make_config(synth.TINY)
    setattr(cfg, field, value)
    st, h = _create(cfg, nvals=16)
    assert st == status and h == 0
    assert b.pi0x_last_error() != ""


def test_create_rejects_wrong_blob_size():
    cfg = b.make_config(synth.TINY)
    st, h = _create(cfg, nvals=b.pi0x_weight_count(cfg) - 1)
    assert st == b.PI0X_ERR_SHAPE and h == 0
    assert "weights_bytes" in b.pi0x_last_error()


def test_create_rejects_null_pointers():
    cfg = b.make_config(synth.TINY)
    h = ctypes.c_void_p()
    assert b.lib().pi0x_expert_create(ctypes.byref(cfg), None, 0, ctypes.byref(h)) == b.PI0X_ERR_INVALID_ARG
    assert b.lib().pi0x_expert_create(None, None, 0, ctypes.byref(h)) == b.PI0X_ERR_INVALID_ARG


def test_calls_reject_null_handle():
    assert b.pi0x_denoise(None, 1, 8, 1, 1, 1, 1, 2, 1, None) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_denoise_step(None, 1, 8, 1, 1, 1, 1, 0.5, 1, None) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_denoise_noalloc(None, 1, 8, 1, 1, 1, 1, 2, 1, None) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_denoise_ex(None, 1, 8, 1, 1, 1, 1, 2, None, 1, None) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_denoise_ex(None, 1, 8, 1, 1, 1, 1, 2, b.pi0x_loop_options(), 1, None) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_set_timing(None, 1) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_read_timing(None)[0] == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_expert_check_guards(None)[0] == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_debug_velocity_until(None, 1, 8, 1, 1, 1, 1, 0.5, 1, 0, 0, 1, 64, None) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_prefix_check_guards(None)[0] == b.PI0X_ERR_INVALID_ARG
    b.pi0x_expert_destroy(None)  # ignored


def test_set_normalization_null_handle():
    assert b.lib().pi0x_set_normalization(None, None, None) == b.PI0X_ERR_INVALID_ARG


def test_loop_options_layout_matches_header():
    # int32 schedule, x_prediction, causal_actions, then two pointers
    o = b.pi0x_loop_options
    assert o.schedule.offset == 0 and o.x_prediction.offset == 4 and o.causal_actions.offset == 8
    assert o.dof_mask.offset == 16 and o.padding_action.offset == 24 and ctypes.sizeof(o) == 32
    assert (b.PI0X_SCHEDULE_PI0, b.PI0X_SCHEDULE_ZERO_TO_ONE) == (0, 1)


def test_prefix_config_default_is_gemma_2b():
    c = b.pi0x_prefix_config_default()
    assert (c.width, c.depth, c.mlp_dim, c.num_heads, c.num_kv_heads, c.head_dim) == (2048, 18, 16384, 8, 1, 256)
    assert c.dtype == b.PI0X_BF16 and c.max_batch == 1 and c.max_prefix_len == 1024


@pytest.mark.parametrize("shape", [synth.GEMMA_2B, synth.TINY_VLM])
def test_prefix_weight_count_matches_layer_layout(shape):
    assert b.pi0x_prefix_weight_count(b.make_config(shape)) == synth.prefill_weight_count(shape)


def test_prefix_weight_count_gemma_2b():
    # 18 layers x (2 norms of 2048 + q/o 2 x 2048^2 + k/v 2 x 256 x 2048 + 3 x 16384 x 2048)
    assert synth.prefill_weight_count(synth.GEMMA_2B) == 18 * (2 * 2048 + 2 * 2048 * 2048 + 2 * 256 * 2048
                                                               + 3 * 16384 * 2048)


def test_prefix_create_rejects_bad_config_and_blob():
    cfg = b.make_config(synth.TINY_VLM, "fp32", max_batch=2, max_prefix_len=64)
    w = np.zeros(16, np.float32)
    st, h = b.pi0x_prefix_create(cfg, w.ctypes.data, w.nbytes)
    assert st == b.PI0X_ERR_SHAPE and h == 0 and "weights_bytes" in b.pi0x_last_error()
    big = b.make_config(synth.TINY_VLM, "fp32", max_batch=128, max_prefix_len=1024)
    st, h = b.pi0x_prefix_create(big, w.ctypes.data, w.nbytes)
    assert st == b.PI0X_ERR_CAPACITY and h == 0
    bad = b.make_config(synth.TINY_VLM, "fp32")
    bad.head_dim = 48
    assert b.pi0x_prefix_create(bad, w.ctypes.data, w.nbytes)[0] == b.PI0X_ERR_SHAPE
    h = ctypes.c_void_p()
    assert b.lib().pi0x_prefix_create(None, None, 0, ctypes.byref(h)) == b.PI0X_ERR_INVALID_ARG


def test_prefix_calls_reject_null_handle():
    assert b.pi0x_prefill(None, 1, 8, 1, 1, 16, None) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_prefix_set_timing(None, 1) == b.PI0X_ERR_INVALID_ARG
    assert b.pi0x_prefix_read_timing(None)[0] == b.PI0X_ERR_INVALID_ARG
    b.pi0x_prefix_destroy(None)  # ignored
