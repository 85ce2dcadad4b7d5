"""ctypes wrapper of the fp64 CPU oracle (pi0_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark.  Nothing in the product package imports it.

All arrays are converted to contiguous float64 before the call; the oracle
computes in double precision throughout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pi0_oracle.c")
_LIB = os.path.join(_HERE, "libpi0_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-D_GNU_SOURCE", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("width", "depth", "mlp_dim", "num_heads", "num_kv_heads",
                                             "head_dim", "horizon", "action_dim", "state_dim")] + \
               [(n, ctypes.c_double) for n in ("rms_eps", "rope_theta", "min_period", "max_period")]


_lib = None
_D = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER(_Cfg)
        lib.pi0o_weight_count.argtypes = [P]
        lib.pi0o_weight_count.restype = ctypes.c_size_t
        lib.pi0o_set_threads.argtypes = [ctypes.c_int]
        lib.pi0o_set_threads.restype = ctypes.c_int
        lib.pi0o_sinusoid.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_double, ctypes.c_double, _D]
        lib.pi0o_rmsnorm.argtypes = [_D, _D, ctypes.c_int, ctypes.c_double, _D]
        lib.pi0o_rope.argtypes = [_D, ctypes.c_int, ctypes.c_double, ctypes.c_double]
        lib.pi0o_gelu_tanh.argtypes = [ctypes.c_double]
        lib.pi0o_gelu_tanh.restype = ctypes.c_double
        lib.pi0o_silu.argtypes = [ctypes.c_double]
        lib.pi0o_silu.restype = ctypes.c_double
        lib.pi0o_attend_one.argtypes = [_D, ctypes.c_int, ctypes.c_double, _D, _D, ctypes.c_int, _D, _D,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t, _D]
        lib.pi0o_expert_layer.argtypes = [P, _D, _D, ctypes.c_int, _D, _D, ctypes.c_int, _D, ctypes.c_int]
        lib.pi0o_embed_suffix.argtypes = [P, _D, _D, _D, ctypes.c_double, _D]
        lib.pi0o_expert_forward.argtypes = [P, _D, _D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                            ctypes.c_int]
        lib.pi0o_velocity.argtypes = [P, _D, _D, _D, ctypes.c_double, _D, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_double, ctypes.c_int, _D]
        lib.pi0o_denoise.argtypes = [P, _D, _D, _D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_double, _D]
        lib.pi0o_denoise_ex.argtypes = [P, _D, _D, _D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int, _D, _D, _D]
        lib.pi0o_step_schedule.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _D, _D]
        lib.pi0o_step_schedule.restype = None
        lib.pi0o_prefill_weight_count.argtypes = [P]
        lib.pi0o_prefill_weight_count.restype = ctypes.c_size_t
        lib.pi0o_prefix_layer.argtypes = [P, _D, _D, ctypes.c_int, _D, _D, _D]
        lib.pi0o_prefix_layer.restype = None
        lib.pi0o_prefill.argtypes = [P, _D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_double, _D]
        lib.pi0o_prefill.restype = None
        lib.pi0o_step_time.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.pi0o_step_time.restype = ctypes.c_double
        lib.pi0o_apply_norm.argtypes = [_D, ctypes.c_int, ctypes.c_int, _D, _D, ctypes.c_int, ctypes.c_int]
        lib.pi0o_apply_norm.restype = None
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(_D)


def set_threads(n: int = 0) -> int:
    """Set the OpenMP thread count (0 keeps the default); returns the count in use."""
    return _load().pi0o_set_threads(int(n))


def sinusoid(t: float, dim: int, min_period: float = 4e-3, max_period: float = 4.0) -> np.ndarray:
    out = np.empty(dim, dtype=np.float64)
    _load().pi0o_sinusoid(float(t), int(dim), float(min_period), float(max_period), _p(out))
    return out


def rmsnorm(h, w, eps: float = 1e-6) -> np.ndarray:
    h, w = _f64(h), _f64(w)
    out = np.empty_like(h)
    _load().pi0o_rmsnorm(_p(h), _p(w), h.size, float(eps), _p(out))
    return out


def rope(u, pos: float, base: float = 10000.0) -> np.ndarray:
    u = _f64(u).copy()
    _load().pi0o_rope(_p(u), u.size, float(pos), float(base))
    return u


def gelu_tanh(x: float) -> float:
    return _load().pi0o_gelu_tanh(float(x))


def silu(x: float) -> float:
    return _load().pi0o_silu(float(x))


def step_time(k: int, num_steps: int) -> float:
    return _load().pi0o_step_time(int(k), int(num_steps))


SCHEDULES = {"pi0": 0, "zero_to_one": 1}


def step_schedule(k: int, num_steps: int, schedule: str = "pi0") -> tuple[float, float]:
    """(t_k, dt_k) of step k: "pi0" runs t from 1 down (dt = -1/N), "zero_to_one"
    the float32 grid k/N from 0 up (dt_k = t_{k+1} - t_k)."""
    t, dt = ctypes.c_double(), ctypes.c_double()
    _load().pi0o_step_schedule(int(k), int(num_steps), SCHEDULES[schedule], ctypes.byref(t), ctypes.byref(dt))
    return t.value, dt.value


def apply_norm(x, stats: dict | None, inverse: bool) -> np.ndarray:
    """Boundary (un)normalization of the last axis (page 1, _apply_norm) in
    fp64; stats in the page's format ({"mode": "mean_std", "mean", "std"} or
    {"mode": "min_max", "min", "max"}), None: unchanged.  The statistics go
    through float32 first, as the boundary takes them."""
    x = _f64(x).copy()
    if not stats:
        return x
    mode = str(stats.get("mode", "mean_std")).lower()
    if mode == "mean_std":
        a, b, m = stats["mean"], stats["std"], 1
    elif mode == "min_max":
        a, b, m = stats["min"], stats["max"], 2
    else:
        raise ValueError(mode)
    a = _f64(np.asarray(a, dtype=np.float32))
    b = _f64(np.asarray(b, dtype=np.float32))
    rows = x.reshape(-1, x.shape[-1])
    for r in range(rows.shape[0]):
        row = np.ascontiguousarray(rows[r])
        _load().pi0o_apply_norm(_p(row), row.size, m, _p(a), _p(b), a.size, int(bool(inverse)))
        rows[r] = row
    return rows.reshape(x.shape)


def attend_one(q, kp, vp, valid: int, ks, vs, r: int, scale: float, causal: bool = False) -> np.ndarray:
    """One query row r of the suffix against prefix keys [0, valid) and the
    suffix keys visible to r (causal: keys c <= r).  kp/vp: [L][dh], ks/vs: [S][dh]."""
    q, kp, vp, ks, vs = _f64(q), _f64(kp), _f64(vp), _f64(ks), _f64(vs)
    dh = q.size
    out = np.empty(dh, dtype=np.float64)
    _load().pi0o_attend_one(_p(q), dh, float(scale), _p(kp), _p(vp), int(valid), _p(ks), _p(vs),
                            ks.shape[0], int(r), int(bool(causal)), dh, _p(out))
    return out


class Oracle:
    """fp64 oracle for one expert shape.  Weights are the flat blob (any float dtype)."""

    def __init__(self, shape, weights):
        s = shape
        self.shape = s
        self.cfg = _Cfg(s.width, s.depth, s.mlp_dim, s.num_heads, s.num_kv_heads, s.head_dim,
                        s.horizon, s.action_dim, s.state_dim, s.rms_eps, s.rope_theta,
                        s.min_period, s.max_period)
        lib = _load()
        n = lib.pi0o_weight_count(ctypes.byref(self.cfg))
        w = _f64(weights)
        if w.size != n:
            raise ValueError(f"weight blob has {w.size} values, the shape needs {n}")
        self.w = w

    def _kv(self, kv_sample, L):
        s = self.shape
        kv = _f64(kv_sample)
        if kv.size != s.depth * 2 * L * s.num_kv_heads * s.head_dim:
            raise ValueError("prefix kv has the wrong size")
        return kv

    def layer(self, l: int, h, kp, vp, valid: int, pos, causal: bool = False) -> np.ndarray:
        s = self.shape
        h = _f64(h).copy()
        kp, vp, pos = _f64(kp), _f64(vp), _f64(pos)
        layer_size = (self.w.size - self._head_size()) // s.depth
        wl = self.w[l * layer_size:(l + 1) * layer_size]
        wl = np.ascontiguousarray(wl)
        _load().pi0o_expert_layer(ctypes.byref(self.cfg), _p(wl), _p(h), h.shape[0], _p(kp), _p(vp),
                                  int(valid), _p(pos), int(bool(causal)))
        return h

    # --- single stages, for per-kernel tests ------------------------------
    # One expert layer of page 1's _compute_layer_suffix_only split where the
    # library's kernels split it, each stage composed from the oracle's own
    # primitives (rmsnorm, rope, attend_one, gelu_tanh) and matrix products in
    # the order the page states; chained they give layer() (pinned in
    # tests/test_oracle_pins.py).  Rows are the suffix tokens of one sample.

    def layer_weights(self, l: int) -> dict:
        """Layer l's tensors in the blob's order: input norm, q, k, v, o, post
        norm, gate, up, down (matrices [out][in])."""
        s = self.shape
        W, M, dh = s.width, s.mlp_dim, s.head_dim
        qd, kd = s.num_heads * dh, s.num_kv_heads * dh
        size = (self.w.size - self._head_size()) // s.depth
        blob = self.w[l * size:(l + 1) * size]
        out, p = {}, 0
        for name, shp in [("in_norm", (W,)), ("wq", (qd, W)), ("wk", (kd, W)), ("wv", (kd, W)), ("wo", (W, qd)),
                          ("post_norm", (W,)), ("wgate", (M, W)), ("wup", (M, W)), ("wdown", (W, M))]:
            n = int(np.prod(shp))
            out[name] = blob[p:p + n].reshape(shp)
            p += n
        return out

    def stage_qkv(self, l: int, h, pos):
        """input_layernorm, q/k/v projections, rotary embedding of q and k at
        positions pos[r]: (q [S][qd], k [S][kd], v [S][kd])."""
        s, lw = self.shape, self.layer_weights(l)
        h = _f64(h)
        y = np.stack([rmsnorm(h[r], lw["in_norm"], s.rms_eps) for r in range(h.shape[0])])
        q, k, v = y @ lw["wq"].T, y @ lw["wk"].T, y @ lw["wv"].T
        dh = s.head_dim
        for r in range(h.shape[0]):
            for n in range(s.num_heads):
                q[r, n * dh:(n + 1) * dh] = rope(q[r, n * dh:(n + 1) * dh], pos[r], s.rope_theta)
            for n in range(s.num_kv_heads):
                k[r, n * dh:(n + 1) * dh] = rope(k[r, n * dh:(n + 1) * dh], pos[r], s.rope_theta)
        return q, k, v

    def stage_attention(self, q, k, v, kp, vp, valid: int, causal: bool = False):
        """_attend for every suffix row and query head: prefix keys [0, valid)
        of the (single) kv head and the suffix keys the mask shows.
        q [S][qd]; k, v [S][dh]; kp, vp [L][dh].  Returns o [S][qd]."""
        s = self.shape
        dh, S = s.head_dim, q.shape[0]
        o = np.empty((S, s.num_heads * dh))
        for r in range(S):
            for n in range(s.num_heads):
                o[r, n * dh:(n + 1) * dh] = attend_one(q[r, n * dh:(n + 1) * dh], kp, vp, valid, k, v, r,
                                                       1.0 / np.sqrt(dh), causal)
        return o

    def stage_o_proj(self, l: int, h, o):
        """o_proj and the first residual add: h + o W_o^T."""
        return _f64(h) + _f64(o) @ self.layer_weights(l)["wo"].T

    def stage_gate_up(self, l: int, h):
        """post_attention_layernorm, then gelu_tanh(gate) * up: [S][mlp_dim]."""
        s, lw = self.shape, self.layer_weights(l)
        h = _f64(h)
        y = np.stack([rmsnorm(h[r], lw["post_norm"], s.rms_eps) for r in range(h.shape[0])])
        g, u = y @ lw["wgate"].T, y @ lw["wup"].T
        return np.vectorize(gelu_tanh)(g) * u

    def stage_down(self, l: int, h, g):
        """down projection and the second residual add: h + g W_down^T."""
        return _f64(h) + _f64(g) @ self.layer_weights(l)["wdown"].T

    def stage_head(self, h):
        """The expert's final norm on the action rows (1..H) and action_out_proj:
        the velocity [H][A] (page 1, denoise_step's last lines)."""
        s = self.shape
        W, A, Sd = s.width, s.action_dim, s.state_dim
        head = self.w[self.w.size - self._head_size():]
        final_norm = head[:W]
        tail = head[W + W * Sd + W + W * A + W + W * 2 * W + W + W * W + W:]
        w_out, b_out = tail[:A * W].reshape(A, W), tail[A * W:]
        h = _f64(h)
        y = np.stack([rmsnorm(h[r], final_norm, s.rms_eps) for r in range(1, h.shape[0])])
        return y @ w_out.T + b_out

    def _head_size(self):
        s = self.shape
        W, A, Sd = s.width, s.action_dim, s.state_dim
        return W + W * Sd + W + W * A + W + W * 2 * W + W + W * W + W + A * W + A

    def embed_suffix(self, state, x, t: float) -> np.ndarray:
        s = self.shape
        h = np.empty((s.suffix_len, s.width), dtype=np.float64)
        _load().pi0o_embed_suffix(ctypes.byref(self.cfg), _p(self.w), _p(_f64(state)), _p(_f64(x)), float(t),
                                  _p(h))
        return h

    def expert_forward(self, h, kv_sample, L: int, valid: int, pos_shift: float = 0.0,
                       causal: bool = False) -> np.ndarray:
        h = _f64(h).copy()
        kv = self._kv(kv_sample, L)
        _load().pi0o_expert_forward(ctypes.byref(self.cfg), _p(self.w), _p(h), _p(kv), int(L), int(valid),
                                    float(pos_shift), int(bool(causal)))
        return h

    def velocity(self, state, x, t: float, kv_sample, L: int, valid: int, pos_shift: float = 0.0,
                 causal: bool = False) -> np.ndarray:
        s = self.shape
        v = np.empty((s.horizon, s.action_dim), dtype=np.float64)
        kv = self._kv(kv_sample, L)
        _load().pi0o_velocity(ctypes.byref(self.cfg), _p(self.w), _p(_f64(state)), _p(_f64(x)), float(t),
                              _p(kv), int(L), int(valid), float(pos_shift), int(bool(causal)), _p(v))
        return v

    def denoise(self, state, noise, kv_sample, L: int, valid: int, num_steps: int,
                pos_shift: float = 0.0) -> np.ndarray:
        """One sample: state [state_dim], noise [H][A], kv_sample [depth][2][L][n_kv][dh]."""
        s = self.shape
        out = np.empty((s.horizon, s.action_dim), dtype=np.float64)
        kv = self._kv(kv_sample, L)
        _load().pi0o_denoise(ctypes.byref(self.cfg), _p(self.w), _p(_f64(state)), _p(_f64(noise)), _p(kv),
                             int(L), int(valid), int(num_steps), float(pos_shift), _p(out))
        return out

    def denoise_ex(self, state, noise, kv_sample, L: int, valid: int, num_steps: int, schedule: str = "pi0",
                   x_prediction: bool = False, causal: bool = False, dof_mask=None, padding=None,
                   pos_shift: float = 0.0) -> np.ndarray:
        """One sample with the Wall-X loop variants (page 3, generate_flow_action):
        schedule "pi0" or "zero_to_one", x_prediction (v = head - noise), causal
        suffix mask, and the first-step blend v = (padding - x)(1 - dof_mask) +
        v dof_mask when padding is given (dof_mask, padding: [H][A])."""
        s = self.shape
        out = np.empty((s.horizon, s.action_dim), dtype=np.float64)
        kv = self._kv(kv_sample, L)
        if (dof_mask is None) != (padding is None):
            raise ValueError("dof_mask and padding go together")
        m = p = None
        if padding is not None:
            m = _f64(np.broadcast_to(dof_mask, out.shape))
            p = _f64(np.broadcast_to(padding, out.shape))
        _load().pi0o_denoise_ex(ctypes.byref(self.cfg), _p(self.w), _p(_f64(state)), _p(_f64(noise)), _p(kv),
                                int(L), int(valid), int(num_steps), float(pos_shift), SCHEDULES[schedule],
                                int(bool(x_prediction)), int(bool(causal)), _p(m) if m is not None else None,
                                _p(p) if p is not None else None, _p(out))
        return out

    def denoise_batch(self, inputs: dict, num_steps: int, samples=None, state_norm: dict | None = None,
                      action_norm: dict | None = None, options: dict | None = None) -> np.ndarray:
        """Run samples (default: all) of a batch laid out as the boundary takes it.
        state_norm / action_norm: the state is normalized before the loop and the
        returned actions unnormalized (page 1, _normalize_state / _unnormalize_actions).
        options: loop variants for denoise_ex (schedule, x_prediction, causal, and
        per-batch dof_mask / padding arrays [B][H][A])."""
        kv = inputs["prefix_kv"]
        B, L = kv.shape[2], kv.shape[3]
        idx = range(B) if samples is None else samples
        outs = []
        for b in idx:
            state = apply_norm(inputs["state"][b], state_norm, inverse=False)
            if options is None:
                x = self.denoise(state, inputs["noise"][b], kv[:, :, b], L, int(inputs["valid_len"][b]), num_steps)
            else:
                o = dict(options)
                m, p = o.pop("dof_mask", None), o.pop("padding", None)
                x = self.denoise_ex(state, inputs["noise"][b], kv[:, :, b], L, int(inputs["valid_len"][b]),
                                    num_steps, dof_mask=None if m is None else m[b],
                                    padding=None if p is None else p[b], **o)
            outs.append(apply_norm(x, action_norm, inverse=True))
        return np.stack(outs)


class PrefillOracle:
    """fp64 oracle of the prefix pass for one decoder-stack shape.  Weights are
    the layers-only blob (synth.layer_layout order)."""

    def __init__(self, shape, weights):
        s = shape
        self.shape = s
        self.cfg = _Cfg(s.width, s.depth, s.mlp_dim, s.num_heads, s.num_kv_heads, s.head_dim,
                        s.horizon, s.action_dim, s.state_dim, s.rms_eps, s.rope_theta,
                        s.min_period, s.max_period)
        n = _load().pi0o_prefill_weight_count(ctypes.byref(self.cfg))
        w = _f64(weights)
        if w.size != n:
            raise ValueError(f"weight blob has {w.size} values, the shape needs {n}")
        self.w = w

    def layer(self, l: int, h, pos) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
        """One layer on real rows h [n][W] at positions pos [n]: (h_out, k, v)."""
        s = self.shape
        h = _f64(h).copy()
        n = h.shape[0]
        size = self.w.size // s.depth
        wl = np.ascontiguousarray(self.w[l * size:(l + 1) * size])
        k = np.empty((n, s.num_kv_heads * s.head_dim))
        v = np.empty_like(k)
        _load().pi0o_prefix_layer(ctypes.byref(self.cfg), _p(wl), _p(h), n, _p(_f64(pos)), _p(k), _p(v))
        return h, k, v

    def prefill(self, emb, valid: int, pos_shift: float = 0.0) -> np.ndarray:
        """One sample: emb [L][W] -> cache [depth][2][L][n_kv][dh] (rows >= valid zero)."""
        s = self.shape
        emb = _f64(emb)
        L = emb.shape[0]
        out = np.empty((s.depth, 2, L, s.num_kv_heads, s.head_dim))
        _load().pi0o_prefill(ctypes.byref(self.cfg), _p(self.w), _p(emb), int(L), int(valid), float(pos_shift),
                             _p(out))
        return out

    def prefill_batch(self, inputs: dict, samples=None) -> np.ndarray:
        """cache [depth][2][B][L][n_kv][dh] for the samples (default: all) of a batch
        laid out as the boundary takes it."""
        emb = inputs["embeddings"]
        idx = range(emb.shape[0]) if samples is None else samples
        outs = [self.prefill(emb[b], int(inputs["valid_len"][b])) for b in idx]
        return np.stack(outs, axis=2)
