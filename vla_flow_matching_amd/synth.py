"""Seeded synthetic inputs for the pi0 action-expert denoise loop.

This module only draws numbers and lays them out; it holds none of the
method's arithmetic.  Both the HIP path (through the C-ABI) and the fp64 CPU
oracle consume exactly the arrays it returns.

Every tensor comes from its own numpy PCG64 stream seeded with
``SeedSequence([seed, tensor_id])``, so the order in which tensors are drawn
does not matter.  Weights are N(0, 0.02) (head biases too), RMSNorm weights
are 0 unless a test asks otherwise, prefix K/V, state and noise are N(0, 1).
For bfloat16 workloads every weight and prefix K/V value is rounded to the
nearest bfloat16 (ties to even) before either side sees it, so the two sides
read identical values; state and noise stay float32 (the boundary takes them
as float32).

Shapes follow the pi0 defaults (page 1: action horizon 50, action dim 32,
48 text tokens, 224x224 images = 256 tokens per camera; get_gemma_config
"gemma_300m" = width 1024, depth 18, mlp 4096, 8 query heads, 1 kv head,
head_dim 256; "gemma_2b" = width 2048, depth 18, mlp 16384, same heads for
the prefix pass).  Prefix embeddings for the prefix pass are N(0, 1) like
the prefix K/V.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class ExpertShape:
    width: int = 1024
    depth: int = 18
    mlp_dim: int = 4096
    num_heads: int = 8
    num_kv_heads: int = 1
    head_dim: int = 256
    horizon: int = 50
    action_dim: int = 32
    state_dim: int = 32
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    min_period: float = 4e-3
    max_period: float = 4.0

    @property
    def suffix_len(self) -> int:
        return 1 + self.horizon


GEMMA_300M = ExpertShape()
TINY = ExpertShape(width=256, depth=2, mlp_dim=1024, num_heads=8, num_kv_heads=1, head_dim=32,
                   horizon=8, action_dim=32, state_dim=32)
# the prefix pass (PaliGemma language model); only the layer fields matter
GEMMA_2B = ExpertShape(width=2048, depth=18, mlp_dim=16384, num_heads=8, num_kv_heads=1, head_dim=256)
TINY_VLM = ExpertShape(width=512, depth=3, mlp_dim=1536, num_heads=8, num_kv_heads=1, head_dim=64)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ExpertShape
    dtype: str            # "fp32" or "bf16"
    batch: int
    prefix_len: int       # padded prefix length L
    num_steps: int
    ragged: bool = False  # per-sample valid length 512 + U{8..48}, else all valid
    seed: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_fp32_b1": Workload("tiny_fp32_b1", TINY, "fp32", 1, 64, 2),
    "pi0_fp32_b1": Workload("pi0_fp32_b1", GEMMA_300M, "fp32", 1, 816, 10),
    "pi0_bf16_b1": Workload("pi0_bf16_b1", GEMMA_300M, "bf16", 1, 816, 10),
    "pi0_bf16_b64": Workload("pi0_bf16_b64", GEMMA_300M, "bf16", 64, 816, 10),
    "pi0_bf16_b16_ragged": Workload("pi0_bf16_b16_ragged", GEMMA_300M, "bf16", 16, 560, 5, ragged=True),
}


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    shape: ExpertShape
    dtype: str
    batch: int
    prefix_len: int
    ragged: bool = False  # per-sample valid length 512 + U{8..48}, else all valid
    seed: int = 0

    def replace(self, **kw) -> "PrefillWorkload":
        return dataclasses.replace(self, **kw)


PREFILL_WORKLOADS = {
    "tiny_prefill_fp32": PrefillWorkload("tiny_prefill_fp32", TINY_VLM, "fp32", 1, 96),
    "paligemma_bf16_b1": PrefillWorkload("paligemma_bf16_b1", GEMMA_2B, "bf16", 1, 816),
}


def layer_layout(s: ExpertShape) -> list[tuple[str, tuple[int, ...]]]:
    """Per-layer tensors of a Gemma decoder stack in blob order: input norm, q,
    k, v, o, post-attention norm, gate, up, down ([out][in] matrices)."""
    W, M = s.width, s.mlp_dim
    qd, kd = s.num_heads * s.head_dim, s.num_kv_heads * s.head_dim
    out = []
    for l in range(s.depth):
        out += [
            (f"layers.{l}.input_norm", (W,)),
            (f"layers.{l}.q_proj", (qd, W)),
            (f"layers.{l}.k_proj", (kd, W)),
            (f"layers.{l}.v_proj", (kd, W)),
            (f"layers.{l}.o_proj", (W, qd)),
            (f"layers.{l}.post_norm", (W,)),
            (f"layers.{l}.gate_proj", (M, W)),
            (f"layers.{l}.up_proj", (M, W)),
            (f"layers.{l}.down_proj", (W, M)),
        ]
    return out


def blob_layout(s: ExpertShape) -> list[tuple[str, tuple[int, ...]]]:
    """Tensor names and shapes of the flat weight blob, in blob order.

    Matrices are [out_features][in_features] like nn.Linear weights.  Per layer:
    input norm, q, k, v, o, post-attention norm, gate, up, down; then the final
    norm; then state_proj, action_in_proj, action_time_mlp_in,
    action_time_mlp_out, action_out_proj (weight, bias each)."""
    W = s.width
    out = layer_layout(s)
    out += [
        ("final_norm", (W,)),
        ("state_proj.weight", (W, s.state_dim)),
        ("state_proj.bias", (W,)),
        ("action_in_proj.weight", (W, s.action_dim)),
        ("action_in_proj.bias", (W,)),
        ("action_time_mlp_in.weight", (W, 2 * W)),
        ("action_time_mlp_in.bias", (W,)),
        ("action_time_mlp_out.weight", (W, W)),
        ("action_time_mlp_out.bias", (W,)),
        ("action_out_proj.weight", (s.action_dim, W)),
        ("action_out_proj.bias", (s.action_dim,)),
    ]
    return out


def blob_offsets(s: ExpertShape, layout=blob_layout) -> dict[str, tuple[int, tuple[int, ...]]]:
    offs, p = {}, 0
    for name, shp in layout(s):
        offs[name] = (p, shp)
        p += int(np.prod(shp))
    return offs


def weight_count(s: ExpertShape) -> int:
    return sum(int(np.prod(shp)) for _, shp in blob_layout(s))


def prefill_weight_count(s: ExpertShape) -> int:
    return sum(int(np.prod(shp)) for _, shp in layer_layout(s))


def view(blob: np.ndarray, s: ExpertShape, name: str, layout=blob_layout) -> np.ndarray:
    off, shp = blob_offsets(s, layout)[name]
    return blob[off:off + int(np.prod(shp))].reshape(shp)


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(x)
    out = r.astype(np.uint32).view(np.float32)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bfloat16-representable."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


# tensor ids of the inputs (weights use their blob index)
_ID_PREFIX_KV, _ID_STATE, _ID_NOISE, _ID_VALID, _ID_EMB = 100_001, 100_002, 100_003, 100_004, 100_005


def make_weights(s: ExpertShape, seed: int = 0, dtype: str = "fp32", std: float = 0.02,
                 norm_std: float = 0.0, layout=blob_layout) -> np.ndarray:
    """Flat float32 weight blob.  Norm weights are N(0, norm_std) (0 by default).
    layout=layer_layout gives the prefix-pass blob (decoder layers only)."""
    entries = layout(s)
    blob = np.empty(sum(int(np.prod(shp)) for _, shp in entries), dtype=np.float32)
    p = 0
    for tid, (name, shp) in enumerate(entries):
        n = int(np.prod(shp))
        if name.endswith("norm"):
            if norm_std == 0.0:
                blob[p:p + n] = 0.0
            else:
                blob[p:p + n] = _rng(seed, tid).standard_normal(n, dtype=np.float32) * np.float32(norm_std)
        else:
            blob[p:p + n] = _rng(seed, tid).standard_normal(n, dtype=np.float32) * np.float32(std)
        p += n
    if dtype == "bf16":
        blob = round_bf16(blob)
    return blob


def make_prefill_weights(s: ExpertShape, seed: int = 0, dtype: str = "fp32", std: float = 0.02,
                         norm_std: float = 0.0) -> np.ndarray:
    return make_weights(s, seed, dtype, std, norm_std, layout=layer_layout)


def make_valid_len(w) -> np.ndarray:
    if not w.ragged:
        return np.full(w.batch, w.prefix_len, dtype=np.int32)
    # 2 cameras (2 x 256 image tokens) + text of valid length U{8..48}
    txt = _rng(w.seed, _ID_VALID).integers(8, 49, size=w.batch)
    return (512 + txt).astype(np.int32)


def make_inputs(w: Workload) -> dict[str, np.ndarray]:
    """prefix_kv [depth][2][B][L][n_kv][head_dim] float32, valid_len [B] int32,
    state [B][state_dim] float32, noise [B][horizon][action_dim] float32."""
    s = w.shape
    kv_shape = (s.depth, 2, w.batch, w.prefix_len, s.num_kv_heads, s.head_dim)
    kv = _rng(w.seed, _ID_PREFIX_KV).standard_normal(int(np.prod(kv_shape)), dtype=np.float32).reshape(kv_shape)
    if w.dtype == "bf16":
        kv = round_bf16(kv).reshape(kv_shape)
    state = _rng(w.seed, _ID_STATE).standard_normal((w.batch, s.state_dim), dtype=np.float32)
    noise = _rng(w.seed, _ID_NOISE).standard_normal((w.batch, s.horizon, s.action_dim), dtype=np.float32)
    return {"prefix_kv": kv, "valid_len": make_valid_len(w), "state": state, "noise": noise}


def make_prefill_inputs(w: PrefillWorkload) -> dict[str, np.ndarray]:
    """embeddings [B][L][width] float32 (bf16-rounded for bf16), valid_len [B] int32."""
    s = w.shape
    shp = (w.batch, w.prefix_len, s.width)
    emb = _rng(w.seed, _ID_EMB).standard_normal(int(np.prod(shp)), dtype=np.float32).reshape(shp)
    if w.dtype == "bf16":
        emb = round_bf16(emb).reshape(shp)
    return {"embeddings": emb, "valid_len": make_valid_len(w)}
