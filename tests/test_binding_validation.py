"""The Python binding rejects tensors whose dtype, shape, contiguity, device or
overlap does not match what the C entry points assume, before any pointer
reaches the library (CPU only: a handle-less Expert on the CPU device; a
call that passes validation reaches the C ABI, which rejects the NULL handle)."""
from __future__ import annotations

import pytest

torch = pytest.importorskip("torch")

from vla_flow_matching_amd import binding, synth  # noqa: E402

S = synth.TINY


def _expert(dtype="fp32", device="cpu"):
    ex = binding.Expert.__new__(binding.Expert)
    ex.cfg = binding.make_config(S, dtype, max_batch=4, max_prefix_len=64)
    ex.device = torch.device(device)
    ex.h = 0
    ex._stream = lambda stream: None  # the null stream; no HIP call is made on the CPU
    return ex


def _args(B=2, L=16, kv_dtype=torch.float32):
    return dict(prefix_kv=torch.zeros((S.depth, 2, B, L, S.head_dim), dtype=kv_dtype),
                valid_len=torch.full((B,), L, dtype=torch.int32),
                state=torch.zeros((B, S.state_dim)),
                noise=torch.zeros((B, S.horizon, S.action_dim)))


def _call(ex, a, **kw):
    return ex.denoise(a["prefix_kv"], a["valid_len"], a["state"], a["noise"], 2, **kw)


def test_valid_arguments_reach_the_library():
    binding.lib()
    with pytest.raises(binding.Pi0xError) as e:
        _call(_expert(), _args())
    assert e.value.status == binding.PI0X_ERR_INVALID_ARG  # the NULL handle, past validation


@pytest.mark.parametrize("field,bad", [
    ("noise", lambda a: a["noise"].to(torch.bfloat16)),                 # half the bytes the Euler store writes
    ("valid_len", lambda a: a["valid_len"].to(torch.int64)),            # wrong element size
    ("state", lambda a: a["state"].double()),
    ("prefix_kv", lambda a: a["prefix_kv"].to(torch.bfloat16)),         # fp32 handle
    ("prefix_kv", lambda a: a["prefix_kv"][:, :, :1].clone()),          # batch 1 cache for batch 2
    ("prefix_kv", lambda a: a["prefix_kv"].transpose(3, 4).contiguous()),
    ("prefix_kv", lambda a: torch.zeros((S.depth, 2, 2, 16, 8, S.head_dim))[..., 0, :]),  # a strided view
    ("noise", lambda a: a["noise"][:, :4]),
    ("valid_len", lambda a: a["valid_len"][:1]),
])
def test_bad_tensor_is_rejected(field, bad):
    a = _args()
    a[field] = bad(a)
    with pytest.raises(ValueError):
        _call(_expert(), a)


def test_bf16_handle_requires_bf16_cache():
    ex = _expert("bf16")
    with pytest.raises(ValueError, match="prefix_kv"):
        _call(ex, _args())
    with pytest.raises(binding.Pi0xError):
        _call(ex, _args(kv_dtype=torch.bfloat16))


def test_wrong_device_is_rejected():
    ex = _expert(device="cuda:0")
    with pytest.raises(ValueError, match="must be on"):
        _call(ex, _args())


def test_out_overlap_rules():
    ex = _expert()
    a = _args()
    with pytest.raises(binding.Pi0xError):  # out may be the noise itself
        _call(ex, a, out=a["noise"])
    big = torch.zeros((2 * 2 * S.horizon * S.action_dim,))
    a["noise"] = big[:2 * S.horizon * S.action_dim].view(2, S.horizon, S.action_dim)
    with pytest.raises(ValueError, match="overlap"):  # a shifted window of the noise is not
        _call(ex, a, out=big[S.action_dim:S.action_dim + 2 * S.horizon * S.action_dim].view(2, S.horizon, S.action_dim))
    with pytest.raises(ValueError, match="overlap"):
        _call(ex, a, out=a["state"].new_zeros(0).set_(a["prefix_kv"].untyped_storage(), 0,
                                                        (2, S.horizon, S.action_dim)))


def test_step_and_variant_arguments():
    ex = _expert()
    a = _args()
    with pytest.raises(ValueError):
        ex.denoise_step(a["prefix_kv"], a["valid_len"], a["state"], a["noise"].half(), 0.5)
    with pytest.raises(ValueError, match="go together"):
        ex.denoise_ex(a["prefix_kv"], a["valid_len"], a["state"], a["noise"], 2, dof_mask=torch.ones_like(a["noise"]))
    with pytest.raises(ValueError):
        ex.denoise_ex(a["prefix_kv"], a["valid_len"], a["state"], a["noise"], 2,
                      dof_mask=torch.ones((2, S.horizon, 1)), padding_action=torch.ones((2, S.horizon, 1)))
    with pytest.raises(ValueError, match="schedule"):
        ex.denoise_ex(a["prefix_kv"], a["valid_len"], a["state"], a["noise"], 2, schedule="linear")


def test_prefill_arguments():
    pm = binding.PrefixModel.__new__(binding.PrefixModel)
    vlm = synth.TINY_VLM
    pm.cfg = binding.make_config(vlm, "bf16", max_batch=2, max_prefix_len=32)
    pm.device = torch.device("cpu")
    pm.h = 0
    pm._stream = lambda stream: None
    emb = torch.zeros((2, 32, vlm.width), dtype=torch.bfloat16)
    valid = torch.full((2,), 32, dtype=torch.int32)
    with pytest.raises(binding.Pi0xError):
        pm.prefill(emb, valid)
    with pytest.raises(ValueError):
        pm.prefill(emb.float(), valid)
    with pytest.raises(ValueError):
        pm.prefill(emb, valid.long())
    with pytest.raises(ValueError):
        pm.prefill(emb, valid, out=torch.zeros((vlm.depth, 2, 2, 32, vlm.head_dim)))
