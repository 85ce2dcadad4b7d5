/*
 * pi0_oracle.c -- plain fp64 CPU oracle of the pi0 action-expert flow-matching
 * denoise loop.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  The product path never
 * links, loads or calls it, and it shares no code, header or table with the
 * HIP library: it re-derives everything from the method's definition.
 *
 * Source of the method: the vllm-omni page "vllm_omni/diffusion/models/pi0/
 * modeling_pi0.py" (page 1), sections create_sinusoidal_pos_embedding,
 * make_att_2d_masks, _attend, _compute_layer_suffix_only, embed_suffix,
 * denoise_step and sample_actions; the Gemma building blocks it calls
 * (GemmaRMSNorm with the (1 + w) scale, the gate/up/down GeGLU MLP with the
 * tanh GELU, rotate-half rotary embedding) are the Hugging Face Gemma ones
 * that page imports.  The loop variants of pi0o_denoise_ex (0 -> 1 time grid,
 * x-prediction head, dof-mask padding blend, causal action mask) follow page 3,
 * the Wall-X modeling walk-through, generate_flow_action.  The prefix pass of
 * pi0o_prefill (the PaliGemma language model producing the per-layer K/V
 * cache) follows page 1, _compute_layer_prefix_only and the prefix-only branch
 * of PaliGemmaWithExpertModel.forward as sample_actions calls it.
 *
 * Everything is computed in double precision with straightforward loops, one
 * sample at a time, in the order the page states the computation.  OpenMP
 * only splits independent output elements of a loop across threads; it does
 * not change any summation order.
 *
 * Parity pins (see tests/test_oracle_pins.py): every function below is
 * checked against closed forms, invariants, library routines (torch /
 * Hugging Face Gemma modules in float64) or brute force.  The composed model
 * at random weights has no printed value on the pages; it is pinned by those
 * pieces plus an independent second formulation on the tiny configuration.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int width, depth, mlp_dim, num_heads, num_kv_heads, head_dim;
  int horizon, action_dim, state_dim;
  double rms_eps, rope_theta, min_period, max_period;
} pi0o_cfg;

/* ------------------------------------------------------------------------ */
/* Weight blob layout.  Every matrix is stored like torch's nn.Linear weight:  */
/* [out_features][in_features], row-major.                                     */
/* ------------------------------------------------------------------------ */
typedef struct {
  size_t in_norm, wq, wk, wv, wo, post_norm, wgate, wup, wdown, size;
} layer_offsets;

typedef struct {
  size_t final_norm, state_w, state_b, ain_w, ain_b, tin_w, tin_b, tout_w, tout_b, aout_w, aout_b, total;
} head_offsets;

static layer_offsets layer_layout(const pi0o_cfg* c) {
  layer_offsets o;
  size_t W = (size_t)c->width, qd = (size_t)c->num_heads * c->head_dim, kd = (size_t)c->num_kv_heads * c->head_dim;
  size_t M = (size_t)c->mlp_dim;
  size_t p = 0;
  o.in_norm = p;   p += W;
  o.wq = p;        p += qd * W;
  o.wk = p;        p += kd * W;
  o.wv = p;        p += kd * W;
  o.wo = p;        p += W * qd;
  o.post_norm = p; p += W;
  o.wgate = p;     p += M * W;
  o.wup = p;       p += M * W;
  o.wdown = p;     p += W * M;
  o.size = p;
  return o;
}

static head_offsets head_layout(const pi0o_cfg* c) {
  head_offsets o;
  size_t W = (size_t)c->width, A = (size_t)c->action_dim, Sd = (size_t)c->state_dim;
  size_t p = layer_layout(c).size * (size_t)c->depth;
  o.final_norm = p; p += W;
  o.state_w = p;    p += W * Sd;
  o.state_b = p;    p += W;
  o.ain_w = p;      p += W * A;
  o.ain_b = p;      p += W;
  o.tin_w = p;      p += W * 2 * W;
  o.tin_b = p;      p += W;
  o.tout_w = p;     p += W * W;
  o.tout_b = p;     p += W;
  o.aout_w = p;     p += A * W;
  o.aout_b = p;     p += A;
  o.total = p;
  return o;
}

size_t pi0o_weight_count(const pi0o_cfg* c) { return head_layout(c).total; }

int pi0o_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Building blocks                                                           */
/* ------------------------------------------------------------------------ */

/* Sine/cosine embedding of a scalar time (page 1, create_sinusoidal_pos_embedding):
 * fraction_j = j / (dim/2 - 1) for j = 0..dim/2-1 (an inclusive linspace of [0, 1]),
 * period_j = min_p * (max_p / min_p)^fraction_j, omega_j = 2*pi / period_j,
 * out = [sin(omega * t) ; cos(omega * t)]. */
void pi0o_sinusoid(double t, int dim, double min_p, double max_p, double* out) {
  int half = dim / 2;
  for (int j = 0; j < half; ++j) {
    double fraction = (half > 1) ? (double)j / (double)(half - 1) : 0.0;
    double period = min_p * pow(max_p / min_p, fraction);
    double omega = 2.0 * M_PI / period;
    out[j] = sin(omega * t);
    out[half + j] = cos(omega * t);
  }
}

/* Gemma RMSNorm: y = h / sqrt(mean(h^2) + eps) * (1 + w). */
void pi0o_rmsnorm(const double* h, const double* w, int n, double eps, double* y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += h[i] * h[i];
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int i = 0; i < n; ++i) y[i] = h[i] * inv * (1.0 + w[i]);
}

/* Rotate-half rotary embedding at integer position pos (Hugging Face Gemma
 * rotary_emb + apply_rotary_pos_emb, which page 1 calls on q and the suffix k):
 * for j < d/2, theta_j = pos * base^(-2j/d),
 * (u_j, u_{j+d/2}) <- (u_j cos - u_{j+d/2} sin, u_{j+d/2} cos + u_j sin). */
void pi0o_rope(double* u, int d, double pos, double base) {
  int half = d / 2;
  for (int j = 0; j < half; ++j) {
    double theta = pos * pow(base, -2.0 * (double)j / (double)d);
    double c = cos(theta), s = sin(theta);
    double a = u[j], b = u[j + half];
    u[j] = a * c - b * s;
    u[j + half] = b * c + a * s;
  }
}

/* tanh-approximate GELU ("gelu_pytorch_tanh", the expert's hidden activation). */
double pi0o_gelu_tanh(double x) {
  const double k = sqrt(2.0 / M_PI);
  return 0.5 * x * (1.0 + tanh(k * (x + 0.044715 * x * x * x)));
}

/* SiLU / swish: x * sigmoid(x). */
double pi0o_silu(double x) { return x / (1.0 + exp(-x)); }

/* Y[r] = W X[r] + b for r < rows; W is [out][in]; b may be NULL. */
static void linear_rows(const double* W, const double* b, const double* X, int rows, int out, int in, double* Y) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int r = 0; r < rows; ++r)
    for (int o = 0; o < out; ++o) {
      const double* wr = W + (size_t)o * in;
      const double* xr = X + (size_t)r * in;
      double s = 0.0;
      for (int i = 0; i < in; ++i) s += wr[i] * xr[i];
      Y[(size_t)r * out + o] = s + (b ? b[o] : 0.0);
    }
}

/* Attention visibility inside the suffix.  Default (page 1, make_att_2d_masks
 * applied to embed_suffix's autoregressive mask [1, 1, 0, ..., 0]): key c is
 * visible to query r iff cumsum(ar)[c] <= cumsum(ar)[r].  causal != 0 (page 3,
 * the Wall-X modeling walk-through, generate_flow_action with
 * causal_action_attention_mask set): the whole
 * suffix-to-suffix block is replaced by a lower triangle, so key c is visible
 * to query r iff c <= r.  All suffix tokens are real (no suffix padding). */
static int suffix_visible(int r, int c, int causal) {
  if (causal) return c <= r;
  /* cumsum of [1, 1, 0, 0, ...] is [1, 2, 2, 2, ...] */
  int cum_r = (r == 0) ? 1 : 2;
  int cum_c = (c == 0) ? 1 : 2;
  return cum_c <= cum_r;
}

/* Softmax attention of one query over the visible keys (page 1, _attend:
 * softmax(q k^T * scale + mask) v, masked keys get exactly zero weight).
 * Prefix keys j < valid are visible, keys j >= valid are padding and are not
 * read.  kp/vp: prefix keys/values of this query's kv head, row stride kstride.
 * ks/vs: suffix keys/values, row stride kstride.  r: suffix index of the query;
 * causal selects the suffix rule (suffix_visible). */
void pi0o_attend_one(const double* q, int dh, double scale,
                     const double* kp, const double* vp, int valid,
                     const double* ks, const double* vs, int S, int r, int causal,
                     size_t kstride, double* out) {
  int nk = valid + S;
  double* s = (double*)malloc(sizeof(double) * (size_t)nk);
  unsigned char* vis = (unsigned char*)malloc((size_t)nk);
  double mx = -INFINITY;
  for (int j = 0; j < nk; ++j) {
    const double* k;
    if (j < valid) { k = kp + (size_t)j * kstride; vis[j] = 1; }
    else { int c = j - valid; k = ks + (size_t)c * kstride; vis[j] = (unsigned char)suffix_visible(r, c, causal); }
    if (!vis[j]) { s[j] = 0.0; continue; }
    double d = 0.0;
    for (int i = 0; i < dh; ++i) d += q[i] * k[i];
    s[j] = d * scale;
    if (s[j] > mx) mx = s[j];
  }
  double den = 0.0;
  for (int j = 0; j < nk; ++j) { s[j] = vis[j] ? exp(s[j] - mx) : 0.0; den += s[j]; }
  for (int i = 0; i < dh; ++i) out[i] = 0.0;
  for (int j = 0; j < nk; ++j) {
    if (!vis[j]) continue;
    const double* v = (j < valid) ? vp + (size_t)j * kstride : vs + (size_t)(j - valid) * kstride;
    double p = s[j] / den;
    for (int i = 0; i < dh; ++i) out[i] += p * v[i];
  }
  free(s);
  free(vis);
}

/* One action-expert decoder layer on the S suffix rows (page 1,
 * _compute_layer_suffix_only): pre-norm, q/k/v projections, rotary embedding
 * of q and the suffix k at the rows' positions, attention over
 * [cached prefix K/V ; suffix K/V] with grouped kv heads, o_proj + residual,
 * post-attention norm, GeGLU MLP + residual.  h is updated in place.
 * kp/vp: this layer's prefix keys/values, [L][n_kv][dh], already rotated.
 * causal: suffix mask rule (suffix_visible). */
void pi0o_expert_layer(const pi0o_cfg* c, const double* lw, double* h, int S,
                       const double* kp, const double* vp, int valid, const double* pos, int causal) {
  layer_offsets lo = layer_layout(c);
  int W = c->width, nh = c->num_heads, nkv = c->num_kv_heads, dh = c->head_dim, M = c->mlp_dim;
  int qd = nh * dh, kd = nkv * dh, group = nh / nkv;
  double scale = 1.0 / sqrt((double)dh);
  double* y = (double*)malloc(sizeof(double) * (size_t)S * W);
  double* q = (double*)malloc(sizeof(double) * (size_t)S * qd);
  double* k = (double*)malloc(sizeof(double) * (size_t)S * kd);
  double* v = (double*)malloc(sizeof(double) * (size_t)S * kd);
  double* o = (double*)malloc(sizeof(double) * (size_t)S * qd);
  double* t = (double*)malloc(sizeof(double) * (size_t)S * W);
  double* g = (double*)malloc(sizeof(double) * (size_t)S * M);
  double* u = (double*)malloc(sizeof(double) * (size_t)S * M);

  for (int r = 0; r < S; ++r) pi0o_rmsnorm(h + (size_t)r * W, lw + lo.in_norm, W, c->rms_eps, y + (size_t)r * W);
  linear_rows(lw + lo.wq, NULL, y, S, qd, W, q);
  linear_rows(lw + lo.wk, NULL, y, S, kd, W, k);
  linear_rows(lw + lo.wv, NULL, y, S, kd, W, v);
  for (int r = 0; r < S; ++r) {
    for (int n = 0; n < nh; ++n) pi0o_rope(q + (size_t)r * qd + (size_t)n * dh, dh, pos[r], c->rope_theta);
    for (int n = 0; n < nkv; ++n) pi0o_rope(k + (size_t)r * kd + (size_t)n * dh, dh, pos[r], c->rope_theta);
  }
#pragma omp parallel for collapse(2) schedule(static)
  for (int r = 0; r < S; ++r)
    for (int n = 0; n < nh; ++n) {
      int gi = n / group;
      pi0o_attend_one(q + (size_t)r * qd + (size_t)n * dh, dh, scale,
                      kp + (size_t)gi * dh, vp + (size_t)gi * dh, valid,
                      k + (size_t)gi * dh, v + (size_t)gi * dh, S, r, causal,
                      (size_t)kd, o + (size_t)r * qd + (size_t)n * dh);
    }
  linear_rows(lw + lo.wo, NULL, o, S, W, qd, t);
  for (size_t i = 0; i < (size_t)S * W; ++i) h[i] += t[i];

  for (int r = 0; r < S; ++r) pi0o_rmsnorm(h + (size_t)r * W, lw + lo.post_norm, W, c->rms_eps, y + (size_t)r * W);
  linear_rows(lw + lo.wgate, NULL, y, S, M, W, g);
  linear_rows(lw + lo.wup, NULL, y, S, M, W, u);
  for (size_t i = 0; i < (size_t)S * M; ++i) g[i] = pi0o_gelu_tanh(g[i]) * u[i];
  linear_rows(lw + lo.wdown, NULL, g, S, W, M, t);
  for (size_t i = 0; i < (size_t)S * W; ++i) h[i] += t[i];

  free(y); free(q); free(k); free(v); free(o); free(t); free(g); free(u);
}

/* Suffix embedding (page 1, embed_suffix): row 0 is the state token
 * state_proj(state); rows 1..H are action_time_mlp_out(silu(action_time_mlp_in(
 * [action_in_proj(x_i) ; tau(t)]))), action half first, time half second. */
void pi0o_embed_suffix(const pi0o_cfg* c, const double* w, const double* state, const double* x,
                       double t, double* h) {
  head_offsets ho = head_layout(c);
  int W = c->width, H = c->horizon, A = c->action_dim, Sd = c->state_dim;
  double* tau = (double*)malloc(sizeof(double) * (size_t)W);
  double* a = (double*)malloc(sizeof(double) * (size_t)H * W);
  double* cat = (double*)malloc(sizeof(double) * (size_t)H * 2 * W);
  double* m = (double*)malloc(sizeof(double) * (size_t)H * W);
  pi0o_sinusoid(t, W, c->min_period, c->max_period, tau);
  linear_rows(w + ho.state_w, w + ho.state_b, state, 1, W, Sd, h);
  linear_rows(w + ho.ain_w, w + ho.ain_b, x, H, W, A, a);
  for (int i = 0; i < H; ++i) {
    memcpy(cat + (size_t)i * 2 * W, a + (size_t)i * W, sizeof(double) * (size_t)W);
    memcpy(cat + (size_t)i * 2 * W + W, tau, sizeof(double) * (size_t)W);
  }
  linear_rows(w + ho.tin_w, w + ho.tin_b, cat, H, W, 2 * W, m);
  for (size_t i = 0; i < (size_t)H * W; ++i) m[i] = pi0o_silu(m[i]);
  linear_rows(w + ho.tout_w, w + ho.tout_b, m, H, W, W, h + (size_t)W);
  free(tau); free(a); free(cat); free(m);
}

/* The action expert over the suffix (page 1, PaliGemmaWithActionExpert.forward,
 * suffix-only branch, without the final norm): h [S][W] in place.
 * kv: this sample's prefix cache [depth][2][L][n_kv][dh].  Positions continue
 * from the number of valid prefix tokens: pos_r = valid + r (+ pos_shift, a
 * test hook that shifts every suffix position; 0 in normal use).  causal:
 * suffix mask rule (suffix_visible). */
void pi0o_expert_forward(const pi0o_cfg* c, const double* w, double* h, const double* kv,
                         int L, int valid, double pos_shift, int causal) {
  layer_offsets lo = layer_layout(c);
  int S = 1 + c->horizon;
  size_t kd = (size_t)c->num_kv_heads * c->head_dim;
  double* pos = (double*)malloc(sizeof(double) * (size_t)S);
  for (int r = 0; r < S; ++r) pos[r] = (double)valid + (double)r + pos_shift;
  for (int l = 0; l < c->depth; ++l) {
    const double* kp = kv + ((size_t)l * 2 + 0) * (size_t)L * kd;
    const double* vp = kv + ((size_t)l * 2 + 1) * (size_t)L * kd;
    pi0o_expert_layer(c, w + (size_t)l * lo.size, h, S, kp, vp, valid, pos, causal);
  }
  free(pos);
}

/* Velocity v_t for one sample (page 1, denoise_step): embed the suffix, run the
 * expert, final norm on the action rows (the state row is dropped), then
 * action_out_proj.  v: [H][A].  causal: suffix mask rule (suffix_visible). */
void pi0o_velocity(const pi0o_cfg* c, const double* w, const double* state, const double* x, double t,
                   const double* kv, int L, int valid, double pos_shift, int causal, double* v) {
  head_offsets ho = head_layout(c);
  int W = c->width, H = c->horizon, A = c->action_dim, S = 1 + H;
  double* h = (double*)malloc(sizeof(double) * (size_t)S * W);
  double* hf = (double*)malloc(sizeof(double) * (size_t)H * W);
  pi0o_embed_suffix(c, w, state, x, t, h);
  pi0o_expert_forward(c, w, h, kv, L, valid, pos_shift, causal);
  for (int i = 0; i < H; ++i) pi0o_rmsnorm(h + (size_t)(1 + i) * W, w + ho.final_norm, W, c->rms_eps, hf + (size_t)i * W);
  linear_rows(w + ho.aout_w, w + ho.aout_b, hf, H, A, W, v);
  free(h);
  free(hf);
}

/* Euler flow-matching sampler for one sample (page 1, sample_actions):
 * x = noise at t = 1, dt = -1/N, for k = 0..N-1: t_k = 1 + k*dt (computed in
 * double, then stored as a float32 time value as the page does when it fills
 * the time tensor), x <- x + dt * v(x, t_k).  out: [H][A]. */
void pi0o_denoise(const pi0o_cfg* c, const double* w, const double* state, const double* noise,
                  const double* kv, int L, int valid, int num_steps, double pos_shift, double* out) {
  int H = c->horizon, A = c->action_dim;
  size_t n = (size_t)H * A;
  double* v = (double*)malloc(sizeof(double) * n);
  double dt = -1.0 / (double)num_steps;
  memcpy(out, noise, sizeof(double) * n);
  for (int k = 0; k < num_steps; ++k) {
    double t = (double)(float)(1.0 + (double)k * dt);
    pi0o_velocity(c, w, state, out, t, kv, L, valid, pos_shift, 0, v);
    for (size_t i = 0; i < n; ++i) out[i] = out[i] + dt * v[i];
  }
  free(v);
}

/* Boundary normalization (page 1, _build_norm_buffers and _apply_norm), in
 * place on x[n]: mode 1 mean/std (a = mean, b = std), mode 2 min/max (a = min,
 * b = max).  Only features j < count change.  Forward (the state):
 * mean/std (x - mean) / (std + 1e-8); min/max 2 (x - min) / d - 1 with
 * d = max(max - min, 1e-8).  Inverse (the actions): mean/std x std + mean;
 * min/max (x + 1) / 2 * d + min. */
void pi0o_apply_norm(double* x, int n, int mode, const double* a, const double* b, int count, int inverse) {
  const double eps = 1e-8;
  for (int j = 0; j < n && j < count; ++j) {
    if (mode == 1) {
      x[j] = inverse ? x[j] * b[j] + a[j] : (x[j] - a[j]) / (b[j] + eps);
    } else if (mode == 2) {
      double d = b[j] - a[j];
      if (d < eps) d = eps;
      x[j] = inverse ? (x[j] + 1.0) * 0.5 * d + a[j] : 2.0 * (x[j] - a[j]) / d - 1.0;
    }
  }
}

/* Time value the sampler evaluates at step k of N (exposed for tests). */
double pi0o_step_time(int k, int num_steps) {
  double dt = -1.0 / (double)num_steps;
  return (double)(float)(1.0 + (double)k * dt);
}

/* Time grid of the sampler, step k of N.  schedule 0 (page 1, sample_actions):
 * t_k = 1 + k*dt with dt = -1/N, t stored as float32, every step advances by
 * dt.  schedule 1 (the Wall-X flow-matching page, the Euler ODE integration of
 * the flow head): the N + 1 points k/N from 0 to 1 held as float32; step k
 * evaluates at t_k and advances by t_{k+1} - t_k (the Euler rule over
 * consecutive grid points). */
void pi0o_step_schedule(int k, int num_steps, int schedule, double* t, double* dt) {
  if (schedule == 1) {
    double t0 = (double)(float)((double)k / (double)num_steps);
    double t1 = (double)(float)((double)(k + 1) / (double)num_steps);
    *t = t0;
    *dt = t1 - t0;
  } else {
    *dt = -1.0 / (double)num_steps;
    *t = (double)(float)(1.0 + (double)k * *dt);
  }
}

/* Euler sampler with the Wall-X loop variants (page 3, the Wall-X modeling
 * walk-through, generate_flow_action: its first, prefill step and the later
 * step_with_kvcache steps), for one sample:
 *   x = noise; for k = 0..N-1: (t, dt) = pi0o_step_schedule(k, N, schedule);
 *   y = head output at (x, t) with the suffix mask rule causal;
 *   v = y - noise when x_pred (the head predicts the clean action; the noise
 *       subtracted is the initial one), else v = y;
 *   on the first step only, when padding != NULL:
 *       v = (padding - x) * (1 - dof_mask) + v * dof_mask;
 *   x = x + dt * v.
 * dof_mask, padding: [H][A] (padding != NULL needs dof_mask != NULL).  out: [H][A]. */
void pi0o_denoise_ex(const pi0o_cfg* c, const double* w, const double* state, const double* noise,
                     const double* kv, int L, int valid, int num_steps, double pos_shift, int schedule,
                     int x_pred, int causal, const double* dof_mask, const double* padding, double* out) {
  int H = c->horizon, A = c->action_dim;
  size_t n = (size_t)H * A;
  double* v = (double*)malloc(sizeof(double) * n);
  memcpy(out, noise, sizeof(double) * n);
  for (int k = 0; k < num_steps; ++k) {
    double t, dt;
    pi0o_step_schedule(k, num_steps, schedule, &t, &dt);
    pi0o_velocity(c, w, state, out, t, kv, L, valid, pos_shift, causal, v);
    if (x_pred)
      for (size_t i = 0; i < n; ++i) v[i] = v[i] - noise[i];
    if (k == 0 && padding)
      for (size_t i = 0; i < n; ++i) v[i] = (padding[i] - out[i]) * (1.0 - dof_mask[i]) + v[i] * dof_mask[i];
    for (size_t i = 0; i < n; ++i) out[i] = out[i] + dt * v[i];
  }
  free(v);
}

/* ------------------------------------------------------------------------ */
/* Prefix pass: the PaliGemma language model over the prefix embeddings       */
/* ------------------------------------------------------------------------ */

/* Values in a prefix-pass weight blob: depth decoder layers in the layer
 * layout above (no final norm, no action head). */
size_t pi0o_prefill_weight_count(const pi0o_cfg* c) { return layer_layout(c).size * (size_t)c->depth; }

/* One language-model layer of the prefix pass (page 1,
 * _compute_layer_prefix_only) on the n real prefix rows h [n][W], in place:
 * pre-norm, q/k/v projections, rotary embedding of q and k at positions
 * pos[r], attention of every row over every row (the prefix mask that
 * make_att_2d_masks builds from an all-zero autoregressive mask: real tokens
 * see each other both ways), o_proj + residual, post-attention norm, GeGLU
 * MLP + residual.  k_out / v_out [n][n_kv][dh] receive the layer's post-RoPE
 * keys and its values, the pair the suffix pass caches. */
void pi0o_prefix_layer(const pi0o_cfg* c, const double* lw, double* h, int n, const double* pos,
                       double* k_out, double* v_out) {
  layer_offsets lo = layer_layout(c);
  int W = c->width, nh = c->num_heads, nkv = c->num_kv_heads, dh = c->head_dim, M = c->mlp_dim;
  int qd = nh * dh, kd = nkv * dh, group = nh / nkv;
  double scale = 1.0 / sqrt((double)dh);
  size_t rows = n > 0 ? (size_t)n : 1;
  double* y = (double*)malloc(sizeof(double) * rows * W);
  double* q = (double*)malloc(sizeof(double) * rows * qd);
  double* o = (double*)malloc(sizeof(double) * rows * qd);
  double* t = (double*)malloc(sizeof(double) * rows * W);
  double* g = (double*)malloc(sizeof(double) * rows * M);
  double* u = (double*)malloc(sizeof(double) * rows * M);

  for (int r = 0; r < n; ++r) pi0o_rmsnorm(h + (size_t)r * W, lw + lo.in_norm, W, c->rms_eps, y + (size_t)r * W);
  linear_rows(lw + lo.wq, NULL, y, n, qd, W, q);
  linear_rows(lw + lo.wk, NULL, y, n, kd, W, k_out);
  linear_rows(lw + lo.wv, NULL, y, n, kd, W, v_out);
  for (int r = 0; r < n; ++r) {
    for (int hh = 0; hh < nh; ++hh) pi0o_rope(q + (size_t)r * qd + (size_t)hh * dh, dh, pos[r], c->rope_theta);
    for (int hh = 0; hh < nkv; ++hh) pi0o_rope(k_out + (size_t)r * kd + (size_t)hh * dh, dh, pos[r], c->rope_theta);
  }
  /* every row sees the n real keys: the "prefix" argument of pi0o_attend_one
   * with no suffix keys */
#pragma omp parallel for collapse(2) schedule(static)
  for (int r = 0; r < n; ++r)
    for (int hh = 0; hh < nh; ++hh) {
      int gi = hh / group;
      pi0o_attend_one(q + (size_t)r * qd + (size_t)hh * dh, dh, scale, k_out + (size_t)gi * dh,
                      v_out + (size_t)gi * dh, n, NULL, NULL, 0, r, 0, (size_t)kd,
                      o + (size_t)r * qd + (size_t)hh * dh);
    }
  linear_rows(lw + lo.wo, NULL, o, n, W, qd, t);
  for (size_t i = 0; i < (size_t)n * W; ++i) h[i] += t[i];

  for (int r = 0; r < n; ++r) pi0o_rmsnorm(h + (size_t)r * W, lw + lo.post_norm, W, c->rms_eps, y + (size_t)r * W);
  linear_rows(lw + lo.wgate, NULL, y, n, M, W, g);
  linear_rows(lw + lo.wup, NULL, y, n, M, W, u);
  for (size_t i = 0; i < (size_t)n * M; ++i) g[i] = pi0o_gelu_tanh(g[i]) * u[i];
  linear_rows(lw + lo.wdown, NULL, g, n, W, M, t);
  for (size_t i = 0; i < (size_t)n * W; ++i) h[i] += t[i];

  free(y); free(q); free(o); free(t); free(g); free(u);
}

/* Prefix pass of one sample (page 1: sample_actions builds the prefix masks and
 * positions, PaliGemmaWithExpertModel.forward runs the prefix-only branch and
 * keeps the per-layer cache).  emb [L][W]: the prefix embeddings, of which the
 * first `valid` rows are real tokens and the rest padding (right padding, so
 * positions cumsum(pad) - 1 are 0 .. valid-1, plus pos_shift, a test hook).
 * Padded rows are masked out of every real row's attention, so the real rows
 * are computed on their own.  kv_out [depth][2][L][n_kv][dh]: rows < valid get
 * each layer's post-RoPE keys (index 0) and values (index 1); rows >= valid are
 * set to 0 (their content is unspecified for the sampler, which never reads
 * them).  The final norm only shapes the discarded prefix output and is not
 * applied. */
void pi0o_prefill(const pi0o_cfg* c, const double* w, const double* emb, int L, int valid, double pos_shift,
                  double* kv_out) {
  layer_offsets lo = layer_layout(c);
  int W = c->width;
  size_t kd = (size_t)c->num_kv_heads * c->head_dim;
  int n = valid < 0 ? 0 : (valid > L ? L : valid);
  memset(kv_out, 0, sizeof(double) * (size_t)c->depth * 2 * (size_t)L * kd);
  if (n == 0) return;
  double* h = (double*)malloc(sizeof(double) * (size_t)n * W);
  double* pos = (double*)malloc(sizeof(double) * (size_t)n);
  memcpy(h, emb, sizeof(double) * (size_t)n * W);
  for (int r = 0; r < n; ++r) pos[r] = (double)r + pos_shift;
  for (int l = 0; l < c->depth; ++l) {
    double* k = kv_out + ((size_t)l * 2 + 0) * (size_t)L * kd;
    double* v = kv_out + ((size_t)l * 2 + 1) * (size_t)L * kd;
    pi0o_prefix_layer(c, w + (size_t)l * lo.size, h, n, pos, k, v);
  }
  free(h);
  free(pos);
}
