/*
 * pi0x.h -- C ABI of the pi0 action-expert flow-matching denoise loop on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page 1, "vllm_omni/diffusion/models/pi0/modeling_pi0.py",
 * sections sample_actions, denoise_step, embed_suffix and
 * _compute_layer_suffix_only): given the per-layer key/value cache of an
 * observation prefix, a proprioceptive state and Gaussian noise, integrate
 * the flow-matching ODE from t = 1 to t = 0 with num_steps explicit Euler
 * steps (dt = -1/num_steps, t_k = 1 + k*dt, x <- x + dt * v_t) and return the
 * action chunk x of shape (batch, horizon, action_dim).  Each velocity v_t
 * embeds the suffix [state token ; horizon action tokens fused with a
 * sinusoidal embedding of t through a swish MLP], runs the Gemma-shaped
 * action expert whose attention reads the cached prefix keys/values plus the
 * block-causal suffix, applies the final RMSNorm to the action rows and
 * projects them with action_out_proj.
 *
 * Every entry point is plain C: host pointers for configuration and weights,
 * device pointers for activations, a HIP stream for ordering.  All device
 * work runs in the library's own HIP kernels.
 *
 * Errors: every function returns a pi0x_status.  Argument errors are found on
 * the host before anything is enqueued; pi0x_last_error() then returns a
 * thread-local message.  Device-side failures surface when the caller
 * synchronises the stream.
 */
#ifndef PI0X_H_
#define PI0X_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PI0X_OK = 0,
  PI0X_ERR_INVALID_ARG = -1, /* null pointer, non-positive count, bad config value */
  PI0X_ERR_SHAPE = -2,       /* a shape the kernels do not support (see pi0x_config) */
  PI0X_ERR_DTYPE = -3,       /* unknown dtype */
  PI0X_ERR_OOM = -4,         /* device allocation failed */
  PI0X_ERR_HIP = -5,         /* a HIP runtime call failed */
  PI0X_ERR_CAPACITY = -6     /* batch, prefix length or steps above what the handle was created for */
} pi0x_status;

typedef enum {
  PI0X_FP32 = 0, /* float32 weights, activations and prefix K/V */
  PI0X_BF16 = 1  /* bfloat16 weights, activations and prefix K/V, float32 accumulation,
                    float32 residual stream and action state */
} pi0x_dtype;

/*
 * Expert shape and capacity.  The pi0 action expert is get_gemma_config
 * ("gemma_300m") on page 1: width 1024, depth 18, mlp 4096, 8 query heads,
 * 1 kv head, head_dim 256; horizon 50, action_dim 32, state_dim 32 are the
 * page's defaults.  Supported by the kernels: num_kv_heads == 1, head_dim in
 * {32, 64, 128, 256}, width a multiple of 256, mlp_dim and num_heads *
 * head_dim multiples of 128, action_dim and state_dim at most 64.
 */
typedef struct {
  int32_t width, depth, mlp_dim, num_heads, num_kv_heads, head_dim;
  int32_t action_horizon, action_dim, state_dim;
  int32_t max_batch;      /* largest batch a call may pass */
  int32_t max_prefix_len; /* largest padded prefix length a call may pass */
  int32_t max_steps;      /* largest num_steps a call may pass */
  float rms_eps;          /* Gemma RMSNorm epsilon (1e-6) */
  float rope_theta;       /* rotary base (10000, the Gemma default) */
  float time_min_period;  /* sinusoidal time embedding periods (4e-3, 4.0 on page 1) */
  float time_max_period;
  int32_t dtype;          /* pi0x_dtype */
  int32_t use_graphs;     /* 1: replay the N-step loop as one captured hipGraph; 0: launch eagerly */
} pi0x_config;

typedef struct pi0x_expert pi0x_expert;

/* Fills *cfg with the pi0 action-expert shape above, max_batch 64,
 * max_prefix_len 1024, max_steps 64, bf16, graphs on. */
void pi0x_config_default(pi0x_config* cfg);

/* Number of float32 values in the weight blob for cfg (0 if cfg is invalid).
 * Blob layout, every matrix [out_features][in_features] like nn.Linear:
 *   per layer l = 0..depth-1:
 *     input_norm[W], q_proj[H*D][W], k_proj[D][W], v_proj[D][W], o_proj[W][H*D],
 *     post_norm[W], gate_proj[M][W], up_proj[M][W], down_proj[W][M]
 *   final_norm[W],
 *   state_proj.weight[W][Sd], state_proj.bias[W],
 *   action_in_proj.weight[W][A], action_in_proj.bias[W],
 *   action_time_mlp_in.weight[W][2W], action_time_mlp_in.bias[W]   (input = [action ; time]),
 *   action_time_mlp_out.weight[W][W], action_time_mlp_out.bias[W],
 *   action_out_proj.weight[A][W], action_out_proj.bias[A]
 * with W = width, H = num_heads, D = head_dim, M = mlp_dim, A = action_dim,
 * Sd = state_dim.  Norm weights w enter as (1 + w) (Gemma RMSNorm). */
size_t pi0x_weight_count(const pi0x_config* cfg);

/* Creates a handle on the current HIP device.  weights_host: host float32
 * blob of pi0x_weight_count(cfg) values (weights_bytes must equal 4x that);
 * it is copied, repacked and converted to cfg->dtype (round to nearest even),
 * so the caller may free it on return.  The handle owns every device buffer
 * it needs for calls up to the capacities in cfg.  On error *out is NULL. */
pi0x_status pi0x_expert_create(const pi0x_config* cfg, const void* weights_host, size_t weights_bytes,
                               pi0x_expert** out);

/*
 * Full denoise loop (page 1, sample_actions after the prefix pass).
 *   prefix_kv        device, cfg dtype, [depth][2][batch][prefix_len][head_dim]:
 *                    per layer the keys (index 0, already rotary-embedded at
 *                    their prefix positions) and values (index 1) of the
 *                    single kv head.  Read only; 16-byte aligned
 *                    (PI0X_ERR_INVALID_ARG otherwise).
 *   prefix_valid_len device int32 [batch]: keys [0, v) of sample b are real,
 *                    [v, prefix_len) are padding and are never read.  Values
 *                    outside [0, prefix_len] are clamped into it.  The suffix
 *                    tokens take rotary positions v, v+1, ..., v+horizon.
 *   state            device float32 [batch][state_dim].
 *   noise            device float32 [batch][horizon][action_dim]: x at t = 1.
 *   num_steps        >= 1 and <= cfg->max_steps.
 *   actions_out      device float32 [batch][horizon][action_dim]: x at t = 0.
 *                    May alias noise; must not overlap the other inputs.
 *   stream           HIP stream the work is ordered on (0 = null stream).
 * Asynchronous: returns after enqueueing.  One handle serves one stream at a
 * time: calls on the same handle from different threads or streams race on
 * its workspaces. */
pi0x_status pi0x_denoise(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                         const int32_t* prefix_valid_len, const float* state, const float* noise,
                         int32_t num_steps, float* actions_out, hipStream_t stream);

/*
 * pi0x_denoise for callers that cannot allocate device memory during a call:
 * code under stream capture, tight serving loops and harnesses that forbid
 * hipMalloc.  Same arguments, result and errors as pi0x_denoise, computed by
 * the same kernels, but enqueued directly on `stream`: no graph is captured or
 * instantiated and timing is ignored.  The call's working buffers (residual
 * stream, activations, V^T copies, split partials, time features, call
 * descriptor) come from one static device array of
 * PI0X_NOALLOC_SCRATCH_BYTES per GPU, which the library holds from its load
 * on that GPU until the process ends; the handle's own workspaces are not
 * touched.  The call allocates nothing, on the device or in a library.
 * Limits, checked before anything is enqueued: a bf16 handle
 * (PI0X_ERR_DTYPE otherwise); at most 64 suffix rows, batch * (horizon + 1),
 * i.e. batch 1 at the pi0 shape; the call's buffers within the array (the
 * pi0 expert fits up to prefix_len 1024); PI0X_ERR_CAPACITY otherwise.
 * Every call on one GPU shares the array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (other streams, other
 * handles, other threads) race and must be serialised by the caller.
 */
#define PI0X_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pi0x_status pi0x_denoise_noalloc(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                                 const int32_t* prefix_valid_len, const float* state, const float* noise,
                                 int32_t num_steps, float* actions_out, hipStream_t stream);

/*
 * One velocity evaluation (page 1, denoise_step): v = v_theta(x_t, t) for
 * every sample, with the same prefix/state arguments as pi0x_denoise.
 *   x_t    device float32 [batch][horizon][action_dim]
 *   t      time value (the sampler uses 1 + k*dt rounded to float32)
 *   v_out  device float32 [batch][horizon][action_dim]; must not overlap inputs.
 */
pi0x_status pi0x_denoise_step(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                              const int32_t* prefix_valid_len, const float* state, const float* x_t, float t,
                              float* v_out, hipStream_t stream);

/*
 * The denoise loop with the loop variants of page 3 (the Wall-X modeling
 * walk-through, generate_flow_action), on the same expert.  Arguments as
 * pi0x_denoise; options == NULL, or all fields zero, is exactly pi0x_denoise.
 *   schedule        PI0X_SCHEDULE_PI0: t_k = 1 + k*dt, dt = -1/num_steps
 *                   (page 1, sample_actions).  PI0X_SCHEDULE_ZERO_TO_ONE:
 *                   the float32 grid t_k = k/num_steps, k = 0..num_steps;
 *                   step k evaluates at t_k and advances x by t_{k+1} - t_k,
 *                   so t = 1 is never evaluated.
 *   x_prediction    0: the head's output is the velocity.  1: the head
 *                   predicts the clean chunk; v = output - noise, with the
 *                   sample's initial noise.
 *   causal_actions  0: the pi0 suffix mask (the state token sees itself,
 *                   action tokens see the whole suffix).  1: suffix token s
 *                   sees suffix tokens 0..s (a lower triangle).
 *   dof_mask, padding_action  device float32 [batch][horizon][action_dim],
 *                   both NULL or both set; read only, must not overlap
 *                   actions_out.  When set, the first step's velocity becomes
 *                   (padding_action - x)(1 - dof_mask) + v dof_mask, x being
 *                   the noise; later steps are unchanged.
 * The loop runs in the normalized action space: padding_action is taken as
 * given, and the action unnormalization (pi0x_set_normalization) applies to
 * the returned chunk only.  Errors as pi0x_denoise, plus
 * PI0X_ERR_INVALID_ARG for an unknown schedule, flags other than 0 or 1, or
 * only one of dof_mask / padding_action set.
 */
typedef enum { PI0X_SCHEDULE_PI0 = 0, PI0X_SCHEDULE_ZERO_TO_ONE = 1 } pi0x_schedule;
typedef struct {
  int32_t schedule;              /* pi0x_schedule */
  int32_t x_prediction;          /* 0 or 1 */
  int32_t causal_actions;        /* 0 or 1 */
  const float* dof_mask;         /* device float32 [batch][horizon][action_dim] or NULL */
  const float* padding_action;   /* device float32 [batch][horizon][action_dim] or NULL */
} pi0x_loop_options;

pi0x_status pi0x_denoise_ex(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                            const int32_t* prefix_valid_len, const float* state, const float* noise,
                            int32_t num_steps, const pi0x_loop_options* options, float* actions_out,
                            hipStream_t stream);

/*
 * Boundary normalization (page 1, _build_norm_buffers and _apply_norm: the
 * LeRobot NormalizationMode semantics).  Statistics cover the first `count`
 * features; the remaining ones pass through unchanged.
 *   MEAN_STD  a = mean, b = std.  Forward (state):   (x - mean) / (std + 1e-8).
 *                                 Inverse (actions): x * std + mean.
 *   MIN_MAX   a = min,  b = max,  d = max(max - min, 1e-8).
 *                                 Forward (state):   2 (x - min) / d - 1.
 *                                 Inverse (actions): (x + 1) / 2 * d + min.
 * All arithmetic is float32.
 */
typedef enum { PI0X_NORM_NONE = 0, PI0X_NORM_MEAN_STD = 1, PI0X_NORM_MIN_MAX = 2 } pi0x_norm_mode;
typedef struct {
  int32_t mode;    /* pi0x_norm_mode */
  int32_t count;   /* features covered: 1 .. state_dim (state) or 1 .. action_dim (actions) */
  const float* a;  /* host float32 [count]: mean or min */
  const float* b;  /* host float32 [count]: std or max */
} pi0x_norm;

/* Sets the normalization of later calls on the handle; the statistics are
 * copied.  state: the proprioceptive state is normalized before state_proj
 * (pi0x_denoise and pi0x_denoise_step).  action: the action chunk returned by
 * pi0x_denoise is unnormalized; the loop itself runs in the normalized space
 * and pi0x_denoise_step returns the raw velocity.  NULL or PI0X_NORM_NONE
 * turns a side off (the state at creation).  Synchronous: the caller must
 * have synchronised every stream with calls in flight on the handle.
 * Errors: PI0X_ERR_INVALID_ARG for a NULL handle, an unknown mode, a count
 * outside the range above or NULL statistics; nothing changes then. */
pi0x_status pi0x_set_normalization(pi0x_expert* h, const pi0x_norm* state, const pi0x_norm* action);

/* Releases the handle and everything it owns (synchronises the device first).
 * NULL is ignored. */
void pi0x_expert_destroy(pi0x_expert* h);

/* Thread-local text of the last non-OK status returned on this thread. */
const char* pi0x_last_error(void);

/*
 * Kernel timing, for benchmarks.  While enabled, calls on the handle run
 * eagerly (the same kernels with the same arguments as the recorded graph,
 * launched one by one) and every launch of the classes below is bracketed by
 * a pair of HIP events on the call's stream.  pi0x_read_timing synchronises
 * with the last recorded event, writes per-class total milliseconds and launch
 * counts (arrays of PI0X_KERNEL_CLASSES entries) and clears the record.
 */
typedef enum {
  PI0X_KERNEL_SUFFIX_EMBED = 0, /* time features, state token, time MLP (prefix pass: the
                                   embedding copy and the rotary positions) */
  PI0X_KERNEL_RMSNORM = 1,      /* (unused: the norms are fused into the projections) */
  PI0X_KERNEL_QKV_ROPE = 2,     /* q/k/v projection + RoPE */
  PI0X_KERNEL_ATTENTION = 3,    /* prefix + suffix GQA attention (and the per-call transpose
                                   of the prefix values) */
  PI0X_KERNEL_O_PROJ = 4,       /* o_proj + residual */
  PI0X_KERNEL_GATE_UP = 5,      /* gate/up projection + GeGLU */
  PI0X_KERNEL_DOWN = 6,         /* down projection + residual */
  PI0X_KERNEL_FINAL = 7,        /* final norm + action_out_proj + Euler update */
  PI0X_KERNEL_CLASSES = 8
} pi0x_kernel_class;

pi0x_status pi0x_set_timing(pi0x_expert* h, int32_t enable);
pi0x_status pi0x_read_timing(pi0x_expert* h, double* total_ms, int64_t* launches);

/*
 * Test-only stage read-out, for per-kernel parity tests.  Runs the single
 * velocity evaluation of pi0x_denoise_step (page 1, denoise_step: embed_suffix,
 * then per expert layer of _compute_layer_suffix_only the normed q/k/v
 * projection with RoPE, _attend over the prefix cache and the suffix, o_proj
 * plus the residual, the normed gate/up projection with GeGLU, down plus the
 * residual) eagerly on `stream`, stops after `stage` of layer `layer` (the
 * layer is ignored for PI0X_DEBUG_AFTER_EMBED) and copies one of the handle's
 * working buffers, as it stands at that point, to dst (device memory, at
 * least the buffer's size; the copy is ordered on `stream`):
 *   PI0X_DEBUG_RESIDUAL  float32 [batch*S][width], S = horizon + 1: the
 *                        residual stream (row 0 of a sample is its state token)
 *   PI0X_DEBUG_QK        model dtype [batch*S][qd + head_dim]: the queries
 *                        (heads in order) then the key, after RoPE
 *   PI0X_DEBUG_VT        model dtype [batch][head_dim][Sp], Sp = S rounded up
 *                        to 64: the suffix values, transposed; key
 *                        s = 32a + 16b + 4c + d sits at column
 *                        32a + 8c + 4b + d (columns of keys >= S hold 0)
 *   PI0X_DEBUG_ATTN_OUT  model dtype [batch*S][qd]: attention output, heads in order
 *   PI0X_DEBUG_GEGLU     model dtype [batch*S][mlp_dim]: gelu_tanh(gate) * up
 * Arguments as pi0x_denoise_step (x_t, t); nothing is written to any output
 * of the call.  Errors as pi0x_denoise_step, plus PI0X_ERR_INVALID_ARG for an
 * unknown stage or buffer or a layer out of range and PI0X_ERR_CAPACITY for
 * a short dst.
 */
typedef enum {
  PI0X_DEBUG_AFTER_EMBED = 0,
  PI0X_DEBUG_AFTER_QKV = 1,
  PI0X_DEBUG_AFTER_ATTENTION = 2,
  PI0X_DEBUG_AFTER_O_PROJ = 3,
  PI0X_DEBUG_AFTER_GATE_UP = 4,
  PI0X_DEBUG_AFTER_DOWN = 5
} pi0x_debug_stage;
typedef enum {
  PI0X_DEBUG_RESIDUAL = 0,
  PI0X_DEBUG_QK = 1,
  PI0X_DEBUG_VT = 2,
  PI0X_DEBUG_ATTN_OUT = 3,
  PI0X_DEBUG_GEGLU = 4
} pi0x_debug_buffer;
pi0x_status pi0x_debug_velocity_until(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                                      const int32_t* prefix_valid_len, const float* state, const float* x_t, float t,
                                      int32_t stage, int32_t layer, int32_t buffer, void* dst, size_t dst_bytes,
                                      hipStream_t stream);

/*
 * Guard check, a debugging aid.  Every device buffer a handle allocates is
 * followed by a 4 KiB guard filled with the byte 0xA5 at creation; this
 * synchronises the device and sets *corrupted to the number of guards that
 * no longer hold the pattern, i.e. buffers some kernel wrote past.  0 is the
 * only correct result.  Errors: PI0X_ERR_INVALID_ARG for NULL arguments,
 * PI0X_ERR_HIP if a copy fails.
 */
pi0x_status pi0x_expert_check_guards(pi0x_expert* h, int32_t* corrupted);

/*
 * The prefix pass (page 1: sample_actions builds the prefix masks and
 * positions and runs the prefix-only branch of
 * PaliGemmaWithExpertModel.forward, _compute_layer_prefix_only per layer),
 * producing the cache pi0x_denoise reads.  The handle holds a PaliGemma
 * language-model decoder stack (get_gemma_config "gemma_2b": width 2048,
 * depth 18, mlp 16384, 8 query heads, 1 kv head, head_dim 256).  The image
 * and text embedding (SigLIP, the projector, the token table and its
 * sqrt(width) scale) happens before this boundary: it takes the prefix
 * embeddings.  Of the config, only the layer fields (width .. head_dim,
 * rms_eps, rope_theta), dtype, use_graphs, max_batch and max_prefix_len
 * apply; max_batch * max_prefix_len <= 65536 rows.
 *
 * Weight blob: float32, depth decoder layers in the per-layer order of
 * pi0x_expert_create (input_norm, q, k, v, o, post_norm, gate, up, down,
 * nn.Linear [out][in] layout); no final norm and no action head.
 */
typedef struct pi0x_prefix_model pi0x_prefix_model;

/* Gemma-2B layer fields, max_batch 1, max_prefix_len 1024, bfloat16, graphs on. */
void pi0x_prefix_config_default(pi0x_config* cfg);

/* Number of float32 values in a prefix-pass weight blob (0 for a NULL or
 * non-positive config). */
size_t pi0x_prefix_weight_count(const pi0x_config* cfg);

/* Creates a prefix-pass handle on the current HIP device (synchronous; the
 * blob is copied, repacked and converted as in pi0x_expert_create).  Errors
 * as pi0x_expert_create, plus PI0X_ERR_CAPACITY when max_batch *
 * max_prefix_len exceeds 65536.  On error *out is NULL. */
pi0x_status pi0x_prefix_create(const pi0x_config* cfg, const void* weights_host, size_t weights_bytes,
                               pi0x_prefix_model** out);

/*
 * Runs the prefix pass.
 *   prefix_embeddings  device, cfg dtype, [batch][prefix_len][width]: the
 *                      embedded image and text tokens.  Read only.
 *   prefix_valid_len   device int32 [batch]: tokens [0, v) are real and
 *                      [v, prefix_len) padding (right padding, so the real
 *                      tokens sit at positions 0 .. v-1, page 1's
 *                      cumsum(pad) - 1).  Values outside [0, prefix_len] are
 *                      clamped into it.  Padding never reaches a real token.
 *   prefix_kv_out      device, cfg dtype, [depth][2][batch][prefix_len][head_dim],
 *                      16-byte aligned: per layer the post-RoPE keys (index 0)
 *                      and the values (index 1) of the single kv head -- the
 *                      prefix_kv argument of pi0x_denoise for the same batch,
 *                      prefix_len and prefix_valid_len.  Rows >= v of a sample
 *                      are written with unspecified values (pi0x_denoise never
 *                      reads them).  Must not overlap the embeddings.
 * Real tokens attend to every real token (the prefix mask is bidirectional).
 * Asynchronous on stream; one handle serves one stream at a time.
 * prefix_len == 0 returns PI0X_OK without work.  Errors: PI0X_ERR_INVALID_ARG
 * for NULL pointers, batch < 1, a negative prefix_len, a misaligned
 * prefix_kv_out or another current device; PI0X_ERR_CAPACITY above the
 * handle's max_batch or max_prefix_len; PI0X_ERR_HIP for launch errors.
 */
pi0x_status pi0x_prefill(pi0x_prefix_model* p, int32_t batch, int32_t prefix_len, const void* prefix_embeddings,
                         const int32_t* prefix_valid_len, void* prefix_kv_out, hipStream_t stream);

/* Releases the handle (synchronises the device first); NULL is ignored. */
void pi0x_prefix_destroy(pi0x_prefix_model* p);

/* Kernel timing of the prefix pass, as pi0x_set_timing / pi0x_read_timing. */
pi0x_status pi0x_prefix_set_timing(pi0x_prefix_model* p, int32_t enable);
pi0x_status pi0x_prefix_read_timing(pi0x_prefix_model* p, double* total_ms, int64_t* launches);
/* pi0x_expert_check_guards for the prefix-pass handle. */
pi0x_status pi0x_prefix_check_guards(pi0x_prefix_model* p, int32_t* corrupted);

#ifdef __cplusplus
}
#endif

#endif /* PI0X_H_ */
