// Bandwidth-light kernels around the GEMMs: the suffix-embedding inputs, the
// sinusoidal time features and the rotary table.
#pragma once

#include "common.h"

namespace pi0x {

// Writes the per-call descriptor (one thread).
__global__ void set_desc_kernel(CallDesc* d, const void* kv, const int32_t* valid, const float* state,
                                const float* x_in, float* out, float t, const float* dof_mask,
                                const float* padding) {
  d->kv = kv;
  d->valid = valid;
  d->state = state;
  d->x_in = x_in;
  d->out = out;
  d->t = t;
  d->dof_mask = dof_mask;
  d->padding = padding;
}

// Descriptor of a prefix-pass call: the cache it writes is also the key/value
// source its attention reads (kv).
__global__ void set_prefix_desc_kernel(CallDesc* d, const void* emb, const int32_t* valid, void* kv_out) {
  d->emb = emb;
  d->valid = valid;
  d->kv = kv_out;
  d->kv_out = kv_out;
}

// First hidden rows of the prefix pass: the embeddings [R][W] (model dtype)
// copied to the float32 residual stream (and its bf16 copy in bf16 mode), with
// the sum-of-squares partials over groups of G columns (G <= 256, 1024 % G ==
// 0) that the first layer's input norm consumes.  One block per row.
template <typename T>
__global__ __launch_bounds__(256) void prefix_in_kernel(const CallDesc* __restrict__ desc, int W,
                                                        float* __restrict__ hbuf, T* __restrict__ hb,
                                                        float* __restrict__ ssq, int G) {
  const size_t row = blockIdx.x;
  const T* e = reinterpret_cast<const T*>(desc->emb) + row * W;
  const int np = W / G, tpg = G / 4;  // threads per column group
  for (int c0 = threadIdx.x * 4; c0 < W; c0 += 1024) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float v = to_f32(e[c0 + k]);
      hbuf[row * W + c0 + k] = v;
      if (hb) hb[row * W + c0 + k] = e[c0 + k];
      ss += v * v;
    }
    for (int off = 1; off < tpg; off <<= 1) ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x % tpg) == 0) ssq[row * np + c0 / G] = ss;
  }
}

// State token of every sample (page 1, embed_suffix: state_proj(state)),
// once per call: hs[b][o] = W_s s_b + b_s (float32).  The token depends on
// neither x nor t.  One block per sample.
__global__ __launch_bounds__(256) void state_token_kernel(const CallDesc* __restrict__ desc, const NormDev* __restrict__ norm,
                                                          int Sd, int W, const float* __restrict__ w_s,
                                                          const float* __restrict__ b_s, float* __restrict__ hs) {
  __shared__ float xs[64];
  const int b = blockIdx.x;
  if (threadIdx.x < Sd) xs[threadIdx.x] = norm_state(norm, threadIdx.x, desc->state[(size_t)b * Sd + threadIdx.x]);
  __syncthreads();
  for (int o = threadIdx.x; o < W; o += 256) {
    const float* wr = w_s + (size_t)o * Sd;
    float s = b_s[o];
    for (int k = 0; k < Sd; ++k) s += wr[k] * xs[k];
    hs[(size_t)b * W + o] = s;
  }
}

// Suffix-embedding input of one Euler step (page 1, embed_suffix).
// action_in_proj is folded into the action half of action_time_mlp_in at create
// time (w_comb = W_mi,a W_in, and W_mi,a b_in is part of the step bias cb), so
// the first layer of the time MLP is u = SiLU(w_comb x + cb) with K =
// action_dim; u goes to the model dtype.  w_comb is stored transposed,
// wt[a][o].  Blocks < nA: 256 outputs o of RB action rows each (block id =
// row block * nchunks + output chunk).  Blocks >= nA: copy the state token of
// one sample into hidden row b*S (float32, its bf16 copy in bf16 mode, and its
// sum-of-squares partials over groups of G columns, G <= 256).  x comes from
// desc->x_in when from_input, else from the loop's own x buffer.
template <typename T>
__global__ __launch_bounds__(256) void suffix_in_kernel(const CallDesc* __restrict__ desc, const float* x_loop,
                                                        int from_input, int AR, int nA, int A, int W, int S,
                                                        const float* __restrict__ wt, const float* __restrict__ cb,
                                                        T* __restrict__ u, const float* __restrict__ hs,
                                                        float* __restrict__ hbuf, T* __restrict__ hb,
                                                        float* __restrict__ ssq, int G) {
  constexpr int RB = 4;
  __shared__ float xs[RB][64];
  if ((int)blockIdx.x < nA) {
    const int nchunks = (W + 255) / 256;
    const int r0 = (blockIdx.x / nchunks) * RB, o = (blockIdx.x % nchunks) * 256 + threadIdx.x;
    const float* xsrc = from_input ? desc->x_in : x_loop;
    for (int i = threadIdx.x; i < RB * 64; i += 256) {
      const int rr = i / 64, a = i - rr * 64;
      xs[rr][a] = (r0 + rr < AR && a < A) ? xsrc[(size_t)(r0 + rr) * A + a] : 0.f;
    }
    __syncthreads();
    if (o >= W) return;
    float acc[RB];
    const float bias = cb[o];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) acc[rr] = bias;
    for (int a = 0; a < A; ++a) {
      const float w = wt[(size_t)a * W + o];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) acc[rr] += w * xs[rr][a];
    }
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
      if (r0 + rr < AR) u[(size_t)(r0 + rr) * W + o] = from_f32<T>(silu(acc[rr]));
    return;
  }
  const int b = blockIdx.x - nA;
  const size_t hrow = (size_t)b * S;
  const int np = W / G, tpg = G / 4;  // threads per column group
  for (int c0 = threadIdx.x * 4; c0 < W; c0 += 1024) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = hs[(size_t)b * W + c0 + e];
      hbuf[hrow * W + c0 + e] = v;
      if (hb) hb[hrow * W + c0 + e] = from_f32<T>(v);
      ss += v * v;
    }
    for (int off = 1; off < tpg; off <<= 1) ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x % tpg) == 0) ssq[hrow * np + c0 / G] = ss;
  }
}

// Sinusoidal time features (page 1, create_sinusoidal_pos_embedding), one row
// per evaluated time: fraction_j = j/(W/2-1), period_j = min_p (max_p/min_p)^fraction_j,
// tau = [sin(2 pi t / period) ; cos(2 pi t / period)], evaluated in float64 and
// rounded once to the model dtype.  Denoise mode: row k uses t_k = 1 + k*dt with
// dt = -1/N, rounded to float32 as the sampler stores it (page 1,
// sample_actions), or with zero_to_one the float32 grid point k/N (page 3,
// Wall-X generate_flow_action: a linspace grid from 0 to 1); single-step mode
// (N == 0): one row with desc->t.
template <typename T>
__global__ void time_features_kernel(const CallDesc* __restrict__ desc, int N, int zero_to_one, int W, double min_p,
                                     double max_p, T* __restrict__ tau) {
  const int k = blockIdx.x, half = W / 2;
  double t;
  if (N > 0 && zero_to_one) t = (double)(float)((double)k / (double)N);
  else if (N > 0) t = (double)(float)(1.0 + (double)k * (-1.0 / (double)N));
  else t = (double)desc->t;
  for (int j = threadIdx.x; j < half; j += blockDim.x) {
    const double frac = half > 1 ? (double)j / (double)(half - 1) : 0.0;
    const double period = min_p * pow(max_p / min_p, frac);
    const double arg = (2.0 * M_PI / period) * t;
    tau[(size_t)k * W + j] = from_f32<T>((float)sin(arg));
    tau[(size_t)k * W + half + j] = from_f32<T>((float)cos(arg));
  }
}

// (cos, sin) of every row of the call: suffix row b*S + s sits at position
// valid_len[b] + s (valid_len clamped to [0, L]); with from_valid == 0 (the
// prefix pass, right padding: positions cumsum(pad) - 1) row s of a sample
// sits at position s.  cs[row][j] from the tables.
__global__ __launch_bounds__(128) void rope_rows_kernel(const CallDesc* __restrict__ desc, int S, int L, int half,
                                                        const float* __restrict__ cos_t, const float* __restrict__ sin_t,
                                                        float2* __restrict__ cs, int from_valid) {
  const int row = blockIdx.x, b = row / S, s = row - b * S;
  int v = 0;
  if (from_valid) {
    v = desc->valid[b];
    v = v < 0 ? 0 : (v > L ? L : v);
  }
  const size_t p = (size_t)(v + s) * half;
  for (int j = threadIdx.x; j < half; j += 128) cs[(size_t)row * half + j] = float2{cos_t[p + j], sin_t[p + j]};
}

// Rotary table for positions 0..P-1: theta = p * base^(-2j/d), j < d/2,
// in float64, stored as float32 cos and sin [p][d/2].
__global__ void rope_table_kernel(int P, int d, double base, float* __restrict__ cos_t, float* __restrict__ sin_t) {
  const int half = d / 2;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P * half) return;
  const int p = i / half, j = i - p * half;
  const double theta = (double)p * pow(base, -2.0 * (double)j / (double)d);
  cos_t[i] = (float)cos(theta);
  sin_t[i] = (float)sin(theta);
}

}  // namespace pi0x
