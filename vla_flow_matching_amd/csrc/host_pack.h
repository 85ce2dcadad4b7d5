// host_pack.h -- the host-only part of the library: configuration checks,
// weight-blob sizes and the repacking of the blob into the layouts the
// kernels read.  Plain C++ with no HIP calls, so that a CPU build can run it
// under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// The blob follows the module order of page 1 (vllm-omni modeling_pi0.py,
// PI0Pytorch.__init__ and the Gemma layers it builds): per decoder layer
// input_layernorm, q/k/v/o projections, post_attention_layernorm, gate, up,
// down (each matrix [out][in], like torch's nn.Linear), then the action
// head: the expert's final norm, state_proj, action_in_proj,
// action_time_mlp_in, action_time_mlp_out and action_out_proj (weight, bias).
#pragma once

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "pi0x.h"

namespace pi0x {
namespace hostpack {

// float32 -> bfloat16, round to nearest even; NaNs stay (quiet) NaNs
inline uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// x in the model dtype, as float (bf16 mode: rounded to bf16)
inline float round_model(float x, bool bf16) {
  if (!bf16) return x;
  const uint32_t u = (uint32_t)to_bf16(x) << 16;
  float r;
  std::memcpy(&r, &u, 4);
  return r;
}

// Checks a denoise-handle configuration; PI0X_OK, or an error status with
// *msg set.  All products are formed in 64 bits.
inline pi0x_status config_error(const pi0x_config* c, std::string* msg) {
  auto bad = [&](pi0x_status st, const char* m) {
    *msg = m;
    return st;
  };
  if (!c) return bad(PI0X_ERR_INVALID_ARG, "config is NULL");
  if (c->width <= 0 || c->depth <= 0 || c->mlp_dim <= 0 || c->num_heads <= 0 || c->num_kv_heads <= 0 ||
      c->head_dim <= 0 || c->action_horizon <= 0 || c->action_dim <= 0 || c->state_dim <= 0 || c->max_batch <= 0 ||
      c->max_prefix_len < 0 || c->max_steps <= 0)
    return bad(PI0X_ERR_INVALID_ARG, "config has a non-positive dimension or capacity");
  if (c->dtype != PI0X_FP32 && c->dtype != PI0X_BF16) return bad(PI0X_ERR_DTYPE, "unknown dtype");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f) || !(c->time_min_period > 0.f) || !(c->time_max_period > 0.f))
    return bad(PI0X_ERR_INVALID_ARG, "config has an invalid rms_eps, rope_theta or time period");
  if (c->num_kv_heads != 1) return bad(PI0X_ERR_SHAPE, "only num_kv_heads == 1 is supported");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return bad(PI0X_ERR_SHAPE, "head_dim must be 32, 64, 128 or 256");
  if (c->width % 256 != 0) return bad(PI0X_ERR_SHAPE, "width must be a multiple of 256");
  if (c->mlp_dim % 128 != 0) return bad(PI0X_ERR_SHAPE, "mlp_dim must be a multiple of 128");
  if (((long long)c->num_heads * c->head_dim) % 128 != 0)
    return bad(PI0X_ERR_SHAPE, "num_heads*head_dim must be a multiple of 128");
  if (c->action_dim > 64 || c->state_dim > 64) return bad(PI0X_ERR_SHAPE, "action_dim and state_dim must be <= 64");
  // sizes the kernels index with 32-bit integers
  if (c->width > (1 << 16) || c->mlp_dim > (1 << 18) || (long long)c->num_heads * c->head_dim > (1 << 16) ||
      c->depth > 4096 || c->max_prefix_len > (1 << 20) || c->max_steps > (1 << 16))
    return bad(PI0X_ERR_CAPACITY, "a dimension exceeds the library's limits");
  if ((long long)c->max_batch * (c->action_horizon + 1LL) > (1LL << 24)) return bad(PI0X_ERR_CAPACITY, "max_batch too large");
  return PI0X_OK;
}

// The prefix-pass handle: the action-head fields do not apply.
inline pi0x_status prefix_config_error(const pi0x_config* c, long long max_rows, std::string* msg) {
  if (!c) {
    *msg = "config is NULL";
    return PI0X_ERR_INVALID_ARG;
  }
  pi0x_config k = *c;
  k.action_horizon = 1;
  k.action_dim = 1;
  k.state_dim = 1;
  k.max_steps = 1;
  k.time_min_period = k.time_max_period = 1.f;
  const pi0x_status st = config_error(&k, msg);
  if (st != PI0X_OK) return st;
  if (c->max_prefix_len < 1) {
    *msg = "max_prefix_len must be >= 1";
    return PI0X_ERR_INVALID_ARG;
  }
  if ((long long)c->max_batch * c->max_prefix_len > max_rows) {
    *msg = "max_batch * max_prefix_len exceeds " + std::to_string(max_rows) + " rows";
    return PI0X_ERR_CAPACITY;
  }
  return PI0X_OK;
}

// floats of one decoder layer in the blob
inline size_t layer_floats(size_t W, size_t M, size_t qd, size_t kd) {
  return W + qd * W + 2 * kd * W + W * qd + W + 3 * M * W;
}

inline size_t weight_count(const pi0x_config* c) {
  const size_t W = c->width, M = c->mlp_dim, qd = (size_t)c->num_heads * c->head_dim,
               kd = (size_t)c->num_kv_heads * c->head_dim;
  const size_t A = c->action_dim, Sd = c->state_dim;
  return layer_floats(W, M, qd, kd) * c->depth + W + (W * Sd + W) + (W * A + W) + (W * 2 * W + W) + (W * W + W) +
         (A * W + A);
}

inline size_t prefix_weight_count(const pi0x_config* c) {
  const size_t W = c->width, M = c->mlp_dim, qd = (size_t)c->num_heads * c->head_dim,
               kd = (size_t)c->num_kv_heads * c->head_dim;
  return layer_floats(W, M, qd, kd) * c->depth;
}

// Layer dimensions of a handle (one kv head).
struct Dims {
  int W, M, nh, dh, A, Sd;
  bool bf16;
  int qd() const { return nh * dh; }
};

template <typename E>
inline E to_elem(float v);
template <>
inline float to_elem<float>(float v) { return v; }
template <>
inline uint16_t to_elem<uint16_t>(float v) { return to_bf16(v); }

// Pointers to layer l's tensors in the blob.
struct LayerSrc {
  const float *in_norm, *wq, *wk, *wv, *wo, *post, *wg, *wu, *wd;
};
inline LayerSrc layer_src(const float* blob, const Dims& d, int l) {
  const size_t W = d.W, M = d.M, qd = d.qd(), dh = d.dh;
  LayerSrc s;
  s.in_norm = blob + (size_t)l * layer_floats(W, M, qd, dh);
  s.wq = s.in_norm + W;
  s.wk = s.wq + qd * W;
  s.wv = s.wk + dh * W;
  s.wo = s.wv + dh * W;
  s.post = s.wo + W * qd;
  s.wg = s.post + W;
  s.wu = s.wg + M * W;
  s.wd = s.wu + M * W;
  return s;
}

// q/k/v, [qd + 2 dh][W]: the query heads, then the key, then the value rows,
// with the input norm's (1 + w) folded into the columns.  Within each head
// (and the key) the rows are reordered so that rotary partners (i, i + dh/2)
// sit 16 rows apart in every 32-row group: packed row w of a head is the
// original row ((w % 32) / 16) * dh/2 + (w / 32) * 16 + w % 16.
template <typename E>
std::vector<E> pack_qkv(const LayerSrc& s, const Dims& d) {
  const int W = d.W, dh = d.dh, qd = d.qd(), half = dh / 2, rows = qd + 2 * dh;
  std::vector<float> scale(W);
  for (int k = 0; k < W; ++k) scale[k] = 1.0f + round_model(s.in_norm[k], d.bf16);
  std::vector<E> v((size_t)rows * W);
  for (int c = 0; c < rows; ++c) {
    const float* src;
    if (c < qd + dh) {
      const int head = c / dh, w = c % dh;
      const int orig = ((w % 32) / 16) * half + (w / 32) * 16 + (w % 16);
      src = head < d.nh ? s.wq + ((size_t)head * dh + orig) * W : s.wk + (size_t)orig * W;
    } else {
      src = s.wv + (size_t)(c - qd - dh) * W;
    }
    for (int k = 0; k < W; ++k) v[(size_t)c * W + k] = to_elem<E>(round_model(src[k], d.bf16) * scale[k]);
  }
  return v;
}

// a matrix as is, converted to the model dtype
template <typename E>
std::vector<E> pack_plain(const float* src, size_t n) {
  std::vector<E> v(n);
  for (size_t i = 0; i < n; ++i) v[i] = to_elem<E>(src[i]);
  return v;
}

// gate/up, [2M][W]: 16 gate rows then the same 16 up rows, repeated, with
// the post-attention norm's (1 + w) folded into the columns
template <typename E>
std::vector<E> pack_gate_up(const LayerSrc& s, const Dims& d) {
  const int W = d.W, M = d.M;
  std::vector<float> scale(W);
  for (int k = 0; k < W; ++k) scale[k] = 1.0f + round_model(s.post[k], d.bf16);
  std::vector<E> v((size_t)2 * M * W);
  for (int c = 0; c < 2 * M; ++c) {
    const int pblk = c / 32, sel = (c % 32) / 16, e = c % 16;
    const float* src = (sel == 0 ? s.wg : s.wu) + ((size_t)pblk * 16 + e) * W;
    for (int k = 0; k < W; ++k) v[(size_t)c * W + k] = to_elem<E>(round_model(src[k], d.bf16) * scale[k]);
  }
  return v;
}

// Pointers to the action head's tensors (after the decoder layers).
struct HeadSrc {
  const float *final_norm, *ws, *bs, *wi, *bi, *wmi, *bmi, *wmo, *bmo, *wout, *bout;
};
inline HeadSrc head_src(const float* blob, const Dims& d, int depth) {
  const size_t W = d.W;
  HeadSrc s;
  s.final_norm = blob + (size_t)depth * layer_floats(W, d.M, d.qd(), d.dh);
  s.ws = s.final_norm + W;
  s.bs = s.ws + W * d.Sd;
  s.wi = s.bs + W;
  s.bi = s.wi + W * d.A;
  s.wmi = s.bi + W;
  s.bmi = s.wmi + W * 2 * W;
  s.wmo = s.bmi + W;
  s.bmo = s.wmo + W * W;
  s.wout = s.bmo + W;
  s.bout = s.wout + (size_t)d.A * W;
  return s;
}

// the time half of action_time_mlp_in (its columns W..2W-1), [W][W]
template <typename E>
std::vector<E> pack_time_half(const HeadSrc& s, const Dims& d) {
  const int W = d.W;
  std::vector<E> v((size_t)W * W);
  for (int r = 0; r < W; ++r)
    for (int k = 0; k < W; ++k) v[(size_t)r * W + k] = to_elem<E>(s.wmi[(size_t)r * 2 * W + W + k]);
  return v;
}

// action_in_proj folded into the action half of action_time_mlp_in:
// W_mi,a (W_in x + b_in) = (W_mi,a W_in) x + W_mi,a b_in, products in double.
// comb is [A][W] (transposed), bias [W] includes action_time_mlp_in's own bias.
inline void fold_action_in(const HeadSrc& s, const Dims& d, std::vector<float>* comb, std::vector<float>* bias) {
  const int W = d.W, A = d.A;
  comb->assign((size_t)W * A, 0.f);
  bias->assign(W, 0.f);
  std::vector<double> win((size_t)W * A), bin(W), acc(A);
  for (size_t i = 0; i < win.size(); ++i) win[i] = round_model(s.wi[i], d.bf16);
  for (int k = 0; k < W; ++k) bin[k] = round_model(s.bi[k], d.bf16);
  for (int o = 0; o < W; ++o) {
    std::fill(acc.begin(), acc.end(), 0.0);
    double bacc = round_model(s.bmi[o], d.bf16);
    const float* wr = s.wmi + (size_t)o * 2 * W;
    for (int k = 0; k < W; ++k) {
      const double wk = round_model(wr[k], d.bf16);
      const double* wik = &win[(size_t)k * A];
      for (int a = 0; a < A; ++a) acc[a] += wk * wik[a];
      bacc += wk * bin[k];
    }
    for (int a = 0; a < A; ++a) (*comb)[(size_t)a * W + o] = (float)acc[a];
    (*bias)[o] = (float)bacc;
  }
}

// action_out_proj with the final norm's (1 + w) folded into its columns,
// zero rows up to Apad outputs
template <typename E>
std::vector<E> pack_out_proj(const HeadSrc& s, const Dims& d, int Apad) {
  const int W = d.W, A = d.A;
  std::vector<E> v((size_t)Apad * W);
  for (int r = 0; r < Apad; ++r)
    for (int k = 0; k < W; ++k)
      v[(size_t)r * W + k] = to_elem<E>(
          r < A ? round_model(s.wout[(size_t)r * W + k], d.bf16) * (1.0f + round_model(s.final_norm[k], d.bf16)) : 0.f);
  return v;
}

// a small float32 tensor in the model dtype's values (bf16 mode: rounded,
// held exactly in float32)
inline std::vector<float> pack_small(const float* src, size_t n, bool bf16) {
  std::vector<float> v(n);
  for (size_t i = 0; i < n; ++i) v[i] = round_model(src[i], bf16);
  return v;
}

}  // namespace hostpack
}  // namespace pi0x
