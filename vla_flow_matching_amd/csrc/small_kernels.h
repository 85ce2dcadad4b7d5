// Bandwidth-light kernels around the GEMMs: Gemma RMSNorm, the suffix
// embedding inputs, the sinusoidal time features, the rotary table, and the
// final norm + action_out_proj + Euler update.
#pragma once

#include "common.h"

namespace pi0x {

// Writes the per-call descriptor (one thread).
__global__ void set_desc_kernel(CallDesc* d, const void* kv, const int32_t* valid, const float* state,
                                const float* x_in, float* out, float t) {
  d->kv = kv;
  d->valid = valid;
  d->state = state;
  d->x_in = x_in;
  d->out = out;
  d->t = t;
}

// Gemma RMSNorm (HF GemmaRMSNorm): y = h / sqrt(mean(h^2) + eps) * (1 + w).
// One wave per row; scale1p holds (1 + w) in float32.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, int ldh,
                                                      const float* __restrict__ scale1p, T* __restrict__ y,
                                                      int ldy, int rows, int W, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* hr = h + (size_t)row * ldh;
  float ss = 0.f;
  for (int c = lane * 4; c < W; c += 256) {
    float4 v = *reinterpret_cast<const float4*>(hr + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)W + eps);
  T* yr = y + (size_t)row * ldy;
  for (int c = lane * 4; c < W; c += 256) {
    float4 v = *reinterpret_cast<const float4*>(hr + c);
    float4 s = *reinterpret_cast<const float4*>(scale1p + c);
    yr[c + 0] = from_f32<T>(v.x * inv * s.x);
    yr[c + 1] = from_f32<T>(v.y * inv * s.y);
    yr[c + 2] = from_f32<T>(v.z * inv * s.z);
    yr[c + 3] = from_f32<T>(v.w * inv * s.w);
  }
}

// Suffix-embedding inputs (page 1, embed_suffix).  Rows r < B*H: the action
// projection a = W_in x + b_in of action token r % H of sample r / H, written
// to ain (model dtype) as the first operand of action_time_mlp_in.  Rows
// r >= B*H: the state token W_s s + b_s of sample r - B*H, written to hidden
// row (r - B*H) * S (float32).  x comes from desc->x_in when from_input, else
// from the loop's own x buffer.  One 256-thread block per row.
template <typename T>
__global__ __launch_bounds__(256) void embed_inputs_kernel(const CallDesc* __restrict__ desc, const float* x_loop,
                                                           int from_input, int B, int H, int A, int Sd, int W, int S,
                                                           const float* __restrict__ w_in, const float* __restrict__ b_in,
                                                           const float* __restrict__ w_s, const float* __restrict__ b_s,
                                                           T* __restrict__ ain, float* __restrict__ hbuf, int ldh) {
  __shared__ float xs[64];
  const int r = blockIdx.x;
  const bool is_state = r >= B * H;
  const int K = is_state ? Sd : A;
  const float* src = is_state ? desc->state + (size_t)(r - B * H) * Sd
                              : (from_input ? desc->x_in : x_loop) + (size_t)r * A;
  if (threadIdx.x < K) xs[threadIdx.x] = src[threadIdx.x];
  __syncthreads();
  const float* Wm = is_state ? w_s : w_in;
  const float* bv = is_state ? b_s : b_in;
  for (int o = threadIdx.x; o < W; o += 256) {
    const float* wr = Wm + (size_t)o * K;
    float s = 0.f;
    for (int k = 0; k < K; ++k) s += wr[k] * xs[k];
    s += bv[o];
    if (is_state) hbuf[(size_t)(r - B * H) * S * ldh + o] = s;
    else ain[(size_t)r * W + o] = from_f32<T>(s);
  }
}

// Sinusoidal time features (page 1, create_sinusoidal_pos_embedding), one row
// per evaluated time: fraction_j = j/(W/2-1), period_j = min_p (max_p/min_p)^fraction_j,
// tau = [sin(2 pi t / period) ; cos(2 pi t / period)], evaluated in float64 and
// rounded once to the model dtype.  Denoise mode: row k uses t_k = 1 + k*dt with
// dt = -1/N, rounded to float32 as the sampler stores it; single-step mode
// (N == 0): one row with desc->t.
template <typename T>
__global__ void time_features_kernel(const CallDesc* __restrict__ desc, int N, int W, double min_p, double max_p,
                                     T* __restrict__ tau) {
  const int k = blockIdx.x, half = W / 2;
  double t;
  if (N > 0) t = (double)(float)(1.0 + (double)k * (-1.0 / (double)N));
  else t = (double)desc->t;
  for (int j = threadIdx.x; j < half; j += blockDim.x) {
    const double frac = half > 1 ? (double)j / (double)(half - 1) : 0.0;
    const double period = min_p * pow(max_p / min_p, frac);
    const double arg = (2.0 * M_PI / period) * t;
    tau[(size_t)k * W + j] = from_f32<T>((float)sin(arg));
    tau[(size_t)k * W + half + j] = from_f32<T>((float)cos(arg));
  }
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

// Final norm on the action rows, action_out_proj and the Euler step
// (page 1, denoise_step's last lines and sample_actions' update).  One wave
// per action row r = b*H + i (hidden row b*S + 1 + i).  mode 0: x <- x + dt v
// (x read from desc->x_in when from_input, else x_loop; written to x_loop, and
// also to desc->out when write_out); mode 1: v written to desc->out.
// W_out float32 [A][W]; A <= 64; W a multiple of 256.
__global__ __launch_bounds__(256) void final_kernel(const CallDesc* __restrict__ desc, const float* __restrict__ h,
                                                    int ldh, const float* __restrict__ scale1p,
                                                    const float* __restrict__ w_out, const float* __restrict__ b_out,
                                                    float* x_loop, int from_input, int write_out, int mode, float dt,
                                                    int rows, int H, int S, int W, int A, float eps) {
  __shared__ float red[4][64][65];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  const bool ok = r < rows;
  float part[64];
#pragma unroll
  for (int o = 0; o < 64; ++o) part[o] = 0.f;
  if (ok) {
    const int hrow = (r / H) * S + 1 + r % H;
    const float* hr = h + (size_t)hrow * ldh;
    float ss = 0.f;
    for (int c = lane * 4; c < W; c += 256) {
      float4 v = *reinterpret_cast<const float4*>(hr + c);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)W + eps);
    for (int c = lane * 4; c < W; c += 256) {
      float4 v = *reinterpret_cast<const float4*>(hr + c);
      float4 s = *reinterpret_cast<const float4*>(scale1p + c);
      const float y0 = v.x * inv * s.x, y1 = v.y * inv * s.y, y2 = v.z * inv * s.z, y3 = v.w * inv * s.w;
#pragma unroll
      for (int o = 0; o < 64; ++o) {
        if (o < A) {
          float4 wv = *reinterpret_cast<const float4*>(w_out + (size_t)o * W + c);
          part[o] += wv.x * y0 + wv.y * y1 + wv.z * y2 + wv.w * y3;
        }
      }
    }
  }
#pragma unroll
  for (int o = 0; o < 64; ++o) red[wave][lane][o] = part[o];
  __syncthreads();
  if (!ok || lane >= A) return;
  float v = b_out[lane];
  for (int l = 0; l < 64; ++l) v += red[wave][l][lane];
  const size_t idx = (size_t)r * A + lane;
  if (mode == 1) {
    desc->out[idx] = v;
  } else {
    const float x = (from_input ? desc->x_in : x_loop)[idx];
    const float xn = x + dt * v;
    x_loop[idx] = xn;
    if (write_out) desc->out[idx] = xn;
  }
}

}  // namespace pi0x
