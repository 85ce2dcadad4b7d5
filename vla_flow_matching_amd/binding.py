"""ctypes binding of libpi0x.so (include/pi0x.h).

Argument marshalling only: every step of the denoise loop runs in the
library's HIP kernels.  The module-level functions carry the C names and
take raw integers for device pointers and streams; ``Expert`` wraps them for
torch device tensors.  Loading fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpi0x.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "pi0x.h")

PI0X_OK = 0
PI0X_ERR_INVALID_ARG = -1
PI0X_ERR_SHAPE = -2
PI0X_ERR_DTYPE = -3
PI0X_ERR_OOM = -4
PI0X_ERR_HIP = -5
PI0X_ERR_CAPACITY = -6
PI0X_FP32 = 0
PI0X_BF16 = 1


class pi0x_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "width", "depth", "mlp_dim", "num_heads", "num_kv_heads", "head_dim",
        "action_horizon", "action_dim", "state_dim", "max_batch", "max_prefix_len", "max_steps")] + \
        [(n, ctypes.c_float) for n in ("rms_eps", "rope_theta", "time_min_period", "time_max_period")] + \
        [("dtype", ctypes.c_int32), ("use_graphs", ctypes.c_int32)]


PI0X_NORM_NONE = 0
PI0X_NORM_MEAN_STD = 1
PI0X_NORM_MIN_MAX = 2


class pi0x_norm(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("count", ctypes.c_int32),
                ("a", ctypes.POINTER(ctypes.c_float)), ("b", ctypes.POINTER(ctypes.c_float))]


PI0X_SCHEDULE_PI0 = 0
PI0X_SCHEDULE_ZERO_TO_ONE = 1
SCHEDULES = {"pi0": PI0X_SCHEDULE_PI0, "zero_to_one": PI0X_SCHEDULE_ZERO_TO_ONE}


class pi0x_loop_options(ctypes.Structure):
    _fields_ = [("schedule", ctypes.c_int32), ("x_prediction", ctypes.c_int32), ("causal_actions", ctypes.c_int32),
                ("dof_mask", ctypes.c_void_p), ("padding_action", ctypes.c_void_p)]


class Pi0xError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"pi0x status {status}: {msg}")
        self.status = status


_lib = None


def declared_functions() -> list[str]:
    """Names of the functions include/pi0x.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"\b(pi0x_[a-z_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(the HIP library is required, there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(pi0x_config)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.pi0x_config_default.argtypes = [P]
        L.pi0x_config_default.restype = None
        L.pi0x_weight_count.argtypes = [P]
        L.pi0x_weight_count.restype = sz
        L.pi0x_expert_create.argtypes = [P, vp, sz, ctypes.POINTER(vp)]
        L.pi0x_expert_create.restype = i32
        L.pi0x_denoise.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, vp, vp]
        L.pi0x_denoise.restype = i32
        L.pi0x_denoise_noalloc.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, vp, vp]
        L.pi0x_denoise_noalloc.restype = i32
        L.pi0x_denoise_ex.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, ctypes.POINTER(pi0x_loop_options), vp, vp]
        L.pi0x_denoise_ex.restype = i32
        L.pi0x_denoise_step.argtypes = [vp, i32, i32, vp, vp, vp, vp, ctypes.c_float, vp, vp]
        L.pi0x_denoise_step.restype = i32
        L.pi0x_expert_destroy.argtypes = [vp]
        L.pi0x_expert_destroy.restype = None
        L.pi0x_last_error.argtypes = []
        L.pi0x_last_error.restype = ctypes.c_char_p
        L.pi0x_set_normalization.restype = i32
        L.pi0x_set_normalization.argtypes = [vp, ctypes.POINTER(pi0x_norm), ctypes.POINTER(pi0x_norm)]
        L.pi0x_set_timing.argtypes = [vp, i32]
        L.pi0x_set_timing.restype = i32
        L.pi0x_read_timing.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        L.pi0x_read_timing.restype = i32
        L.pi0x_prefix_config_default.argtypes = [P]
        L.pi0x_prefix_config_default.restype = None
        L.pi0x_prefix_weight_count.argtypes = [P]
        L.pi0x_prefix_weight_count.restype = sz
        L.pi0x_prefix_create.argtypes = [P, vp, sz, ctypes.POINTER(vp)]
        L.pi0x_prefix_create.restype = i32
        L.pi0x_prefill.argtypes = [vp, i32, i32, vp, vp, vp, vp]
        L.pi0x_prefill.restype = i32
        L.pi0x_prefix_destroy.argtypes = [vp]
        L.pi0x_prefix_destroy.restype = None
        L.pi0x_prefix_set_timing.argtypes = [vp, i32]
        L.pi0x_prefix_set_timing.restype = i32
        L.pi0x_prefix_read_timing.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        L.pi0x_prefix_read_timing.restype = i32
        L.pi0x_debug_velocity_until.argtypes = [vp, i32, i32, vp, vp, vp, vp, ctypes.c_float, i32, i32, i32, vp, sz,
                                                 vp]
        L.pi0x_debug_velocity_until.restype = i32
        L.pi0x_expert_check_guards.argtypes = [vp, ctypes.POINTER(i32)]
        L.pi0x_expert_check_guards.restype = i32
        L.pi0x_prefix_check_guards.argtypes = [vp, ctypes.POINTER(i32)]
        L.pi0x_prefix_check_guards.restype = i32
        _lib = L
    return _lib


# --- the C entry points, same names -----------------------------------------
def pi0x_config_default() -> pi0x_config:
    c = pi0x_config()
    lib().pi0x_config_default(ctypes.byref(c))
    return c


def pi0x_weight_count(cfg: pi0x_config) -> int:
    return lib().pi0x_weight_count(ctypes.byref(cfg))


def pi0x_last_error() -> str:
    return lib().pi0x_last_error().decode()


def pi0x_expert_create(cfg: pi0x_config, weights_ptr: int, weights_bytes: int) -> tuple[int, int]:
    h = ctypes.c_void_p()
    st = lib().pi0x_expert_create(ctypes.byref(cfg), weights_ptr, weights_bytes, ctypes.byref(h))
    return st, (h.value or 0)


def pi0x_denoise(h, batch, prefix_len, prefix_kv, valid, state, noise, num_steps, out, stream) -> int:
    return lib().pi0x_denoise(h, batch, prefix_len, prefix_kv, valid, state, noise, num_steps, out, stream)


def pi0x_denoise_noalloc(h, batch, prefix_len, prefix_kv, valid, state, noise, num_steps, out, stream) -> int:
    return lib().pi0x_denoise_noalloc(h, batch, prefix_len, prefix_kv, valid, state, noise, num_steps, out, stream)


def pi0x_denoise_ex(h, batch, prefix_len, prefix_kv, valid, state, noise, num_steps, options, out, stream) -> int:
    """options: a pi0x_loop_options or None."""
    opt = ctypes.byref(options) if options is not None else None
    return lib().pi0x_denoise_ex(h, batch, prefix_len, prefix_kv, valid, state, noise, num_steps, opt, out, stream)


def pi0x_denoise_step(h, batch, prefix_len, prefix_kv, valid, state, x_t, t, v_out, stream) -> int:
    return lib().pi0x_denoise_step(h, batch, prefix_len, prefix_kv, valid, state, x_t, float(t), v_out, stream)


def pi0x_expert_destroy(h) -> None:
    lib().pi0x_expert_destroy(h)


def pi0x_prefix_config_default() -> pi0x_config:
    c = pi0x_config()
    lib().pi0x_prefix_config_default(ctypes.byref(c))
    return c


def pi0x_prefix_weight_count(cfg: pi0x_config) -> int:
    return lib().pi0x_prefix_weight_count(ctypes.byref(cfg))


def pi0x_prefix_create(cfg: pi0x_config, weights_ptr: int, weights_bytes: int) -> tuple[int, int]:
    h = ctypes.c_void_p()
    st = lib().pi0x_prefix_create(ctypes.byref(cfg), weights_ptr, weights_bytes, ctypes.byref(h))
    return st, (h.value or 0)


def pi0x_prefill(p, batch, prefix_len, embeddings, valid, kv_out, stream) -> int:
    return lib().pi0x_prefill(p, batch, prefix_len, embeddings, valid, kv_out, stream)


def pi0x_prefix_destroy(p) -> None:
    lib().pi0x_prefix_destroy(p)


def pi0x_prefix_set_timing(p, enable: bool) -> int:
    return lib().pi0x_prefix_set_timing(p, int(bool(enable)))


def pi0x_prefix_read_timing(p) -> tuple[int, dict]:
    tot = (ctypes.c_double * len(KERNEL_CLASSES))()
    cnt = (ctypes.c_int64 * len(KERNEL_CLASSES))()
    st = lib().pi0x_prefix_read_timing(p, tot, cnt)
    return st, {k: (tot[i], int(cnt[i])) for i, k in enumerate(KERNEL_CLASSES)}


KERNEL_CLASSES = ["suffix_embed", "rmsnorm", "qkv_rope", "attention", "o_proj", "gate_up", "down", "final"]


def norm_struct(stats: dict | None):
    """pi0x_norm for {"mode": "mean_std", "mean": [...], "std": [...]} or
    {"mode": "min_max", "min": [...], "max": [...]} (None: off).  Returns the
    struct and the float32 arrays it points into (keep them alive for the call)."""
    if not stats:
        return None, ()
    mode = str(stats.get("mode", "mean_std")).lower()
    if mode == "mean_std":
        a, b, m = stats["mean"], stats["std"], PI0X_NORM_MEAN_STD
    elif mode == "min_max":
        a, b, m = stats["min"], stats["max"], PI0X_NORM_MIN_MAX
    else:
        raise ValueError(f"unknown normalization mode {mode!r}")
    a = np.ascontiguousarray(a, dtype=np.float32).ravel()
    b = np.ascontiguousarray(b, dtype=np.float32).ravel()
    fp = ctypes.POINTER(ctypes.c_float)
    return pi0x_norm(m, a.size, a.ctypes.data_as(fp), b.ctypes.data_as(fp)), (a, b)


def pi0x_set_normalization(h, state: dict | None, action: dict | None) -> int:
    ns, keep_s = norm_struct(state)
    na, keep_a = norm_struct(action)
    return lib().pi0x_set_normalization(h, ctypes.byref(ns) if ns is not None else None,
                                        ctypes.byref(na) if na is not None else None)


def pi0x_set_timing(h, enable: bool) -> int:
    return lib().pi0x_set_timing(h, 1 if enable else 0)


def pi0x_read_timing(h) -> tuple[int, dict]:
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    st = lib().pi0x_read_timing(h, ms, cnt)
    return st, {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_CLASSES)}


DEBUG_STAGES = {"embed": 0, "qkv": 1, "attention": 2, "o_proj": 3, "gate_up": 4, "down": 5}
DEBUG_BUFFERS = {"residual": 0, "qk": 1, "vt": 2, "attn_out": 3, "geglu": 4}


def pi0x_debug_velocity_until(h, batch, prefix_len, prefix_kv, valid, state, x_t, t, stage, layer, buffer, dst,
                              dst_bytes, stream) -> int:
    return lib().pi0x_debug_velocity_until(h, batch, prefix_len, prefix_kv, valid, state, x_t, float(t), stage, layer,
                                           buffer, dst, dst_bytes, stream)


def pi0x_expert_check_guards(h) -> tuple[int, int]:
    n = ctypes.c_int32(0)
    st = lib().pi0x_expert_check_guards(h, ctypes.byref(n))
    return st, n.value


def pi0x_prefix_check_guards(p) -> tuple[int, int]:
    n = ctypes.c_int32(0)
    st = lib().pi0x_prefix_check_guards(p, ctypes.byref(n))
    return st, n.value


def check(status: int) -> None:
    if status != PI0X_OK:
        raise Pi0xError(status, pi0x_last_error())


def make_config(shape, dtype: str = "bf16", max_batch: int = 64, max_prefix_len: int = 1024,
                max_steps: int = 64, use_graphs: bool = True) -> pi0x_config:
    c = pi0x_config()
    c.width, c.depth, c.mlp_dim = shape.width, shape.depth, shape.mlp_dim
    c.num_heads, c.num_kv_heads, c.head_dim = shape.num_heads, shape.num_kv_heads, shape.head_dim
    c.action_horizon, c.action_dim, c.state_dim = shape.horizon, shape.action_dim, shape.state_dim
    c.max_batch, c.max_prefix_len, c.max_steps = max_batch, max_prefix_len, max_steps
    c.rms_eps, c.rope_theta = shape.rms_eps, shape.rope_theta
    c.time_min_period, c.time_max_period = shape.min_period, shape.max_period
    c.dtype = PI0X_BF16 if dtype == "bf16" else PI0X_FP32
    c.use_graphs = 1 if use_graphs else 0
    return c


def check_tensor(name: str, t, dtype, shape: tuple, device) -> None:
    """Raises ValueError unless t is a contiguous torch tensor of dtype and shape
    on device (the layout the C entry points assume for a raw pointer)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _overlaps(a, b) -> bool:
    if a is None or b is None:
        return False
    a0, b0 = a.data_ptr(), b.data_ptr()
    return a0 < b0 + b.numel() * b.element_size() and b0 < a0 + a.numel() * a.element_size()


def model_dtype(cfg: pi0x_config):
    import torch
    return torch.bfloat16 if cfg.dtype == PI0X_BF16 else torch.float32


class Expert:
    """Owns a pi0x handle; calls take torch device tensors (validated here:
    dtype, shape, contiguity and device, before any pointer reaches the C ABI)."""

    def __init__(self, cfg: pi0x_config, weights: np.ndarray):
        import torch  # (device memory and streams come from torch)
        w = np.ascontiguousarray(weights, dtype=np.float32)
        self.cfg = cfg
        self.device = torch.device("cuda", torch.cuda.current_device())
        st, self.h = pi0x_expert_create(cfg, w.ctypes.data, w.nbytes)
        check(st)

    def _stream(self, stream):
        import torch
        return (stream or torch.cuda.current_stream()).cuda_stream

    @staticmethod
    def _ptr(t):
        return t.data_ptr() if t is not None else None

    def _validate(self, prefix_kv, valid_len, state, x, out, extra=(), alias_ok=None):
        """Shapes from state: B = state.shape[0]; the prefix length from
        prefix_kv [depth][2][B][L][head_dim] (None: an empty prefix).  Returns (B, L)."""
        import torch
        c, dev = self.cfg, self.device
        if not isinstance(state, torch.Tensor) or state.dim() != 2:
            raise ValueError("state must be a 2-D torch tensor [batch][state_dim]")
        B = int(state.shape[0])
        check_tensor("state", state, torch.float32, (B, c.state_dim), dev)
        check_tensor("valid_len", valid_len, torch.int32, (B,), dev)
        L = 0
        if prefix_kv is not None:
            if not isinstance(prefix_kv, torch.Tensor) or prefix_kv.dim() != 5:
                raise ValueError("prefix_kv must be a 5-D torch tensor [depth][2][batch][prefix_len][head_dim]")
            L = int(prefix_kv.shape[3])
            check_tensor("prefix_kv", prefix_kv, model_dtype(c), (c.depth, 2, B, L, c.head_dim), dev)
        chunk = (B, c.action_horizon, c.action_dim)
        check_tensor("x", x, torch.float32, chunk, dev)
        check_tensor("out", out, torch.float32, chunk, dev)
        for name, t in extra:
            check_tensor(name, t, torch.float32, chunk, dev)
        for name, t in [("prefix_kv", prefix_kv), ("valid_len", valid_len), ("state", state), ("x", x)] + list(extra):
            if t is alias_ok and t is not None and t.data_ptr() == out.data_ptr():
                continue
            if _overlaps(out, t):
                raise ValueError(f"out must not overlap {name}")
        return B, L

    def denoise(self, prefix_kv, valid_len, state, noise, num_steps: int, out=None, stream=None):
        """out may be noise itself (the loop copies x first); no other overlap."""
        import torch
        if out is None and isinstance(noise, torch.Tensor):
            out = torch.empty_like(noise)
        B, L = self._validate(prefix_kv, valid_len, state, noise, out, alias_ok=noise)
        check(pi0x_denoise(self.h, B, L, self._ptr(prefix_kv), self._ptr(valid_len), self._ptr(state),
                           self._ptr(noise), int(num_steps), self._ptr(out), self._stream(stream)))
        return out

    def denoise_noalloc(self, prefix_kv, valid_len, state, noise, out, num_steps: int, stream=None):
        """pi0x_denoise_noalloc: the caller passes the output buffer too; the
        call itself allocates nothing."""
        B, L = self._validate(prefix_kv, valid_len, state, noise, out, alias_ok=noise)
        check(pi0x_denoise_noalloc(self.h, B, L, self._ptr(prefix_kv), self._ptr(valid_len), self._ptr(state),
                                   self._ptr(noise), int(num_steps), self._ptr(out), self._stream(stream)))
        return out

    def denoise_ex(self, prefix_kv, valid_len, state, noise, num_steps: int, schedule: str = "pi0",
                   x_prediction: bool = False, causal_actions: bool = False, dof_mask=None, padding_action=None,
                   out=None, stream=None):
        """The loop variants of pi0x_denoise_ex; dof_mask / padding_action: float32
        device tensors [B][H][A] (both or neither)."""
        import torch
        if out is None and isinstance(noise, torch.Tensor):
            out = torch.empty_like(noise)
        if (dof_mask is None) != (padding_action is None):
            raise ValueError("dof_mask and padding_action go together")
        extra = [] if dof_mask is None else [("dof_mask", dof_mask), ("padding_action", padding_action)]
        B, L = self._validate(prefix_kv, valid_len, state, noise, out, extra=extra, alias_ok=noise)
        if schedule not in SCHEDULES:
            raise ValueError(f"unknown schedule {schedule!r}")
        opts = pi0x_loop_options(SCHEDULES[schedule], int(bool(x_prediction)), int(bool(causal_actions)),
                                 self._ptr(dof_mask), self._ptr(padding_action))
        check(pi0x_denoise_ex(self.h, B, L, self._ptr(prefix_kv), self._ptr(valid_len), self._ptr(state),
                              self._ptr(noise), int(num_steps), opts, self._ptr(out), self._stream(stream)))
        return out

    def denoise_step(self, prefix_kv, valid_len, state, x_t, t: float, out=None, stream=None):
        import torch
        if out is None and isinstance(x_t, torch.Tensor):
            out = torch.empty_like(x_t)
        B, L = self._validate(prefix_kv, valid_len, state, x_t, out)
        check(pi0x_denoise_step(self.h, B, L, self._ptr(prefix_kv), self._ptr(valid_len), self._ptr(state),
                                self._ptr(x_t), float(t), self._ptr(out), self._stream(stream)))
        return out

    def debug_until(self, prefix_kv, valid_len, state, x_t, t: float, stage: str, layer: int, buffer: str,
                    stream=None):
        """pi0x_debug_velocity_until: one working buffer after `stage` of
        `layer` of a single velocity evaluation, as a new device tensor
        (float32 for "residual", the model dtype otherwise, flat)."""
        import torch
        c = self.cfg
        B, L = self._validate(prefix_kv, valid_len, state, x_t, x_t, alias_ok=x_t)
        R, S = B * (c.action_horizon + 1), c.action_horizon + 1
        Sp = (S + 63) // 64 * 64
        qd = c.num_heads * c.head_dim
        n = {"residual": R * c.width, "qk": R * (qd + c.head_dim), "vt": B * c.head_dim * Sp,
             "attn_out": R * qd, "geglu": R * c.mlp_dim}[buffer]
        dt = torch.float32 if buffer == "residual" else model_dtype(c)
        dst = torch.empty(n, dtype=dt, device=self.device)
        check(pi0x_debug_velocity_until(self.h, B, L, self._ptr(prefix_kv), self._ptr(valid_len), self._ptr(state),
                                        self._ptr(x_t), t, DEBUG_STAGES[stage], int(layer), DEBUG_BUFFERS[buffer],
                                        dst.data_ptr(), dst.numel() * dst.element_size(), self._stream(stream)))
        return dst

    def guard_violations(self) -> int:
        """Buffers of the handle that a kernel wrote past (0 is correct)."""
        st, n = pi0x_expert_check_guards(self.h)
        check(st)
        return n

    def set_normalization(self, state: dict | None = None, action: dict | None = None):
        """State / action statistics in the page's format (see norm_struct); None turns a side off."""
        check(pi0x_set_normalization(self.h, state, action))

    def set_timing(self, enable: bool):
        check(pi0x_set_timing(self.h, enable))

    def read_timing(self) -> dict:
        st, t = pi0x_read_timing(self.h)
        check(st)
        return t

    def close(self):
        if getattr(self, "h", 0):
            pi0x_expert_destroy(self.h)
            self.h = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def device_inputs(inputs: dict, dtype: str, device: str = "cuda"):
    """Copy host inputs (synth.make_inputs) to device tensors in the boundary's layout:
    prefix_kv [depth][2][B][L][head_dim] in the model dtype, the rest as given."""
    import torch
    kv = inputs["prefix_kv"]
    kv = kv.reshape(kv.shape[0], kv.shape[1], kv.shape[2], kv.shape[3], int(np.prod(kv.shape[4:])))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {
        "prefix_kv": torch.from_numpy(np.ascontiguousarray(kv)).to(device=device, dtype=tdt),
        "valid_len": torch.from_numpy(np.ascontiguousarray(inputs["valid_len"], dtype=np.int32)).to(device),
        "state": torch.from_numpy(np.ascontiguousarray(inputs["state"], dtype=np.float32)).to(device),
        "noise": torch.from_numpy(np.ascontiguousarray(inputs["noise"], dtype=np.float32)).to(device),
    }


class PrefixModel:
    """Owns a pi0x prefix-pass handle; calls take torch device tensors."""

    def __init__(self, cfg: pi0x_config, weights: np.ndarray):
        import torch
        w = np.ascontiguousarray(weights, dtype=np.float32)
        self.cfg = cfg
        self.device = torch.device("cuda", torch.cuda.current_device())
        st, self.h = pi0x_prefix_create(cfg, w.ctypes.data, w.nbytes)
        check(st)

    def prefill(self, embeddings, valid_len, out=None, stream=None):
        """embeddings [B][L][width] (model dtype) -> cache [depth][2][B][L][head_dim]."""
        import torch
        c, dev, dt = self.cfg, self.device, model_dtype(self.cfg)
        if not isinstance(embeddings, torch.Tensor) or embeddings.dim() != 3:
            raise ValueError("embeddings must be a 3-D torch tensor [batch][prefix_len][width]")
        B, L = int(embeddings.shape[0]), int(embeddings.shape[1])
        check_tensor("embeddings", embeddings, dt, (B, L, c.width), dev)
        check_tensor("valid_len", valid_len, torch.int32, (B,), dev)
        if out is None:
            out = torch.empty((c.depth, 2, B, L, c.head_dim), dtype=dt, device=dev)
        check_tensor("out", out, dt, (c.depth, 2, B, L, c.head_dim), dev)
        if _overlaps(out, embeddings) or _overlaps(out, valid_len):
            raise ValueError("out must not overlap the inputs")
        check(pi0x_prefill(self.h, B, L, embeddings.data_ptr(), valid_len.data_ptr(), out.data_ptr(),
                           self._stream(stream)))
        return out

    def _stream(self, stream):
        import torch
        return (stream or torch.cuda.current_stream()).cuda_stream

    def guard_violations(self) -> int:
        """Buffers of the handle that a kernel wrote past (0 is correct)."""
        st, n = pi0x_prefix_check_guards(self.h)
        check(st)
        return n

    def set_timing(self, enable: bool):
        check(pi0x_prefix_set_timing(self.h, enable))

    def read_timing(self) -> dict:
        st, t = pi0x_prefix_read_timing(self.h)
        check(st)
        return t

    def close(self):
        if getattr(self, "h", 0):
            pi0x_prefix_destroy(self.h)
            self.h = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def prefill_device_inputs(inputs: dict, dtype: str, device: str = "cuda"):
    """Host prefix-pass inputs (synth.make_prefill_inputs) as device tensors."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {
        "embeddings": torch.from_numpy(np.ascontiguousarray(inputs["embeddings"])).to(device=device, dtype=tdt),
        "valid_len": torch.from_numpy(np.ascontiguousarray(inputs["valid_len"], dtype=np.int32)).to(device),
    }
