// pi0x runtime: the C ABI of include/pi0x.h on top of the gfx950 kernels.
//
// create() repacks the nn.Linear-layout weight blob into the layouts the
// kernels want (q/k rows paired for rotate-half RoPE, gate/up interleaved in
// blocks of 16, the time half of action_time_mlp_in split off), converts it to
// the model dtype and uploads it; it also builds the float32 rotary table on
// the device and allocates every workspace for the handle's capacity.
//
// A call writes a small device descriptor with its pointers and replays the
// hipGraph recorded for (batch, prefix length, steps, mode); the graph is
// recorded on first use, so later calls with new buffers or new valid lengths
// replay it unchanged.
#include "pi0x.h"

#include <cmath>
#include <cstring>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "attention.h"
#include "common.h"
#include "gemm.h"
#include "small_kernels.h"

using namespace pi0x;

namespace {

thread_local std::string g_err;

pi0x_status fail(pi0x_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

#define PI0X_HIP(x)                                                                      \
  do {                                                                                   \
    hipError_t e_ = (x);                                                                 \
    if (e_ != hipSuccess) return fail(PI0X_ERR_HIP, std::string(#x) + ": " + hipGetErrorString(e_)); \
  } while (0)

#define PI0X_TRY(x)                         \
  do {                                      \
    pi0x_status s_ = (x);                   \
    if (s_ != PI0X_OK) return s_;           \
  } while (0)

constexpr int kMaxGraphs = 32;
constexpr size_t kGemmPartialFloats = (size_t)16 << 20;  // 64 MiB of split-K partial tiles
constexpr int kCounters = 1 << 16;

struct Layer {
  void* wqkv;   // [(H+2)*D][W], q/k rows paired for RoPE
  void* wo;     // [W][H*D]
  void* wgu;    // [2M][W], gate/up interleaved by 16 rows
  void* wdown;  // [W][M]
  float* in1p;  // 1 + input_norm
  float* post1p;
};

struct Key {
  int B, L, N, mode;
  bool operator<(const Key& o) const { return std::tie(B, L, N, mode) < std::tie(o.B, o.L, o.N, o.mode); }
};

uint16_t host_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace

struct pi0x_expert {
  pi0x_config cfg;
  int device = 0;
  int esz = 4;
  int W, D, M, nh, dh, H, A, Sd, S, qd, nqkv, Bmax, Lmax;
  std::vector<void*> allocs;
  std::vector<Layer> layers;
  float* final1p = nullptr;
  void *w_ta = nullptr, *w_tt = nullptr, *w_mo = nullptr;
  float *b_mi = nullptr, *b_mo = nullptr, *w_in = nullptr, *b_in = nullptr, *w_s = nullptr, *b_s = nullptr;
  float *w_out = nullptr, *b_out = nullptr, *rope_cos = nullptr, *rope_sin = nullptr;
  float* hbuf = nullptr;
  void *y = nullptr, *qkv = nullptr, *o = nullptr, *gbuf = nullptr, *ain = nullptr, *u = nullptr, *tau = nullptr;
  float *x = nullptr, *tbias = nullptr;
  float* gemm_partial = nullptr;
  unsigned* gemm_counters = nullptr;
  float* attn_partial = nullptr;
  size_t attn_partial_floats = 0;
  unsigned* attn_counters = nullptr;
  CallDesc* desc = nullptr;
  hipStream_t cap_stream = nullptr;
  std::map<Key, std::pair<hipGraph_t, hipGraphExec_t>> graphs;
  std::vector<Key> graph_order;

  pi0x_status alloc(void** p, size_t bytes) {
    *p = nullptr;
    if (bytes == 0) bytes = 256;
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(PI0X_ERR_OOM, "hipMalloc of " + std::to_string(bytes) + " bytes failed");
    }
    allocs.push_back(*p);
    return PI0X_OK;
  }
  template <typename P>
  pi0x_status allocT(P** p, size_t bytes) {
    void* v;
    pi0x_status s = alloc(&v, bytes);
    *p = (P*)v;
    return s;
  }
};

namespace {

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WM, int WN, class Epi>
pi0x_status launch_gemm_cfg(pi0x_expert* h, hipStream_t s, const void* A, int lda, const void* W, int M, int N,
                            int K, const Epi& epi) {
  const int tiles = ((M + BM - 1) / BM) * (N / BN);
  const int KI = K / 32;
  int splits = 1;
  if (tiles < 160) {
    splits = (256 + tiles - 1) / tiles;
    if (splits > KI / 2) splits = KI / 2;
    if (splits > 16) splits = 16;
    if (splits < 1) splits = 1;
    while (splits > 1 && (size_t)tiles * splits * BM * BN > kGemmPartialFloats) --splits;
    if (tiles > kCounters) splits = 1;
  }
  GemmArgs g{A, lda, W, K, M, N, K, splits, h->gemm_partial, h->gemm_counters};
  dim3 grid(N / BN, (M + BM - 1) / BM, splits);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, Epi>), grid, dim3(256), 0, s, g, epi);
  PI0X_HIP(hipGetLastError());
  return PI0X_OK;
}

template <typename T, class Epi>
pi0x_status launch_gemm(pi0x_expert* h, hipStream_t s, const void* A, int lda, const void* W, int M, int N, int K,
                        const Epi& epi) {
  if (M <= 0) return PI0X_OK;
  if (K % 32 != 0 || N % 32 != 0) return fail(PI0X_ERR_SHAPE, "GEMM dims must be multiples of 32");
  if (M > 1024 && N % 128 == 0) return launch_gemm_cfg<T, 128, 128, 2, 2>(h, s, A, lda, W, M, N, K, epi);
  if (M > 64 && N % 64 == 0) return launch_gemm_cfg<T, 128, 64, 2, 2>(h, s, A, lda, W, M, N, K, epi);
  return launch_gemm_cfg<T, 64, 32, 4, 1>(h, s, A, lda, W, M, N, K, epi);
}

template <typename T, int DH>
pi0x_status launch_attn_dh(pi0x_expert* h, hipStream_t s, int B, int L, int layer) {
  const int ntiles = (h->nh * h->S + 63) / 64;
  const int wgs = B * ntiles;
  int splits = 1;
  if (wgs < 128) {
    splits = (256 + wgs - 1) / wgs;
    if (splits > 32) splits = 32;
  }
  const size_t per = (size_t)(2 + DH / 4) * 256;
  while (splits > 1 && (size_t)wgs * splits * per > h->attn_partial_floats) --splits;
  if (wgs > kCounters) splits = 1;
  AttnArgs a;
  a.qkv = h->qkv;
  a.ldqkv = h->nqkv;
  a.col_k = h->qd;
  a.col_v = h->qd + h->dh;
  a.desc = h->desc;
  a.kv_k_off = ((size_t)layer * 2 + 0) * B * L * DH;
  a.kv_v_off = ((size_t)layer * 2 + 1) * B * L * DH;
  a.B = B;
  a.L = L;
  a.S = h->S;
  a.nh = h->nh;
  a.out = h->o;
  a.ldo = h->qd;
  a.scale = 1.0f / std::sqrt((float)DH);
  a.splits = splits;
  a.partial = h->attn_partial;
  a.counters = h->attn_counters;
  hipLaunchKernelGGL((attn_kernel<T, DH>), dim3(ntiles, B, splits), dim3(256), 0, s, a);
  PI0X_HIP(hipGetLastError());
  return PI0X_OK;
}

template <typename T>
pi0x_status launch_attn(pi0x_expert* h, hipStream_t s, int B, int L, int layer) {
  switch (h->dh) {
    case 32: return launch_attn_dh<T, 32>(h, s, B, L, layer);
    case 64: return launch_attn_dh<T, 64>(h, s, B, L, layer);
    case 128: return launch_attn_dh<T, 128>(h, s, B, L, layer);
    case 256: return launch_attn_dh<T, 256>(h, s, B, L, layer);
  }
  return fail(PI0X_ERR_SHAPE, "unsupported head_dim");
}

// The whole loop: N > 0 is the N-step sampler, N == 0 one velocity evaluation.
template <typename T>
pi0x_status enqueue(pi0x_expert* h, hipStream_t s, int B, int L, int N) {
  const int W = h->W, S = h->S, H = h->H, R = B * S, AR = B * H;
  const int steps = N > 0 ? N : 1;
  const float eps = h->cfg.rms_eps;
  const float dt = N > 0 ? (float)(-1.0 / (double)N) : 0.f;
  hipLaunchKernelGGL((time_features_kernel<T>), dim3(steps), dim3(256), 0, s, h->desc, N, W,
                     (double)h->cfg.time_min_period, (double)h->cfg.time_max_period, (T*)h->tau);
  PI0X_HIP(hipGetLastError());
  // time half of action_time_mlp_in (+ its bias) for every evaluated time
  PI0X_TRY(launch_gemm<T>(h, s, h->tau, W, h->w_tt, steps, W, W, EpiStore<float>{h->tbias, W, h->b_mi, 0}));
  for (int k = 0; k < steps; ++k) {
    const int first = (k == 0);
    hipLaunchKernelGGL((embed_inputs_kernel<T>), dim3(AR + B), dim3(256), 0, s, h->desc, h->x, first, B, H, h->A,
                       h->Sd, W, S, h->w_in, h->b_in, h->w_s, h->b_s, (T*)h->ain, h->hbuf, W);
    PI0X_HIP(hipGetLastError());
    PI0X_TRY(launch_gemm<T>(h, s, h->ain, W, h->w_ta, AR, W, W, EpiStore<T>{(T*)h->u, W, h->tbias + (size_t)k * W, 1}));
    PI0X_TRY(launch_gemm<T>(h, s, h->u, W, h->w_mo, AR, W, W, EpiSuffixRows{h->hbuf, W, H, S, h->b_mo}));
    for (int l = 0; l < h->D; ++l) {
      const Layer& ly = h->layers[l];
      hipLaunchKernelGGL((rmsnorm_kernel<T>), dim3((R + 3) / 4), dim3(256), 0, s, h->hbuf, W, ly.in1p, (T*)h->y, W,
                         R, W, eps);
      PI0X_HIP(hipGetLastError());
      PI0X_TRY(launch_gemm<T>(h, s, h->y, W, ly.wqkv, R, h->nqkv, W,
                              EpiQkvRope<T>{(T*)h->qkv, h->nqkv, h->qd + h->dh, h->dh, S, L, h->desc, h->rope_cos,
                                            h->rope_sin}));
      PI0X_TRY(launch_attn<T>(h, s, B, L, l));
      PI0X_TRY(launch_gemm<T>(h, s, h->o, h->qd, ly.wo, R, W, h->qd, EpiResidual{h->hbuf, W}));
      hipLaunchKernelGGL((rmsnorm_kernel<T>), dim3((R + 3) / 4), dim3(256), 0, s, h->hbuf, W, ly.post1p, (T*)h->y,
                         W, R, W, eps);
      PI0X_HIP(hipGetLastError());
      PI0X_TRY(launch_gemm<T>(h, s, h->y, W, ly.wgu, R, 2 * h->M, W, EpiGeglu<T>{(T*)h->gbuf, h->M}));
      PI0X_TRY(launch_gemm<T>(h, s, h->gbuf, h->M, ly.wdown, R, W, h->M, EpiResidual{h->hbuf, W}));
    }
    const int last = (k == steps - 1);
    hipLaunchKernelGGL(final_kernel, dim3((AR + 3) / 4), dim3(256), 0, s, h->desc, h->hbuf, W, h->final1p, h->w_out,
                       h->b_out, h->x, first, last, N > 0 ? 0 : 1, dt, AR, H, S, W, h->A, eps);
    PI0X_HIP(hipGetLastError());
  }
  return PI0X_OK;
}

pi0x_status run(pi0x_expert* h, int B, int L, int N, hipStream_t stream) {
  const Key key{B, L, N, N > 0 ? 0 : 1};
  auto launch_eager = [&](hipStream_t s) -> pi0x_status {
    return h->cfg.dtype == PI0X_BF16 ? enqueue<bf16>(h, s, B, L, N) : enqueue<float>(h, s, B, L, N);
  };
  if (!h->cfg.use_graphs) return launch_eager(stream);
  auto it = h->graphs.find(key);
  if (it == h->graphs.end()) {
    if ((int)h->graphs.size() >= kMaxGraphs) {
      const Key old = h->graph_order.front();
      h->graph_order.erase(h->graph_order.begin());
      auto o = h->graphs.find(old);
      (void)hipGraphExecDestroy(o->second.second);
      (void)hipGraphDestroy(o->second.first);
      h->graphs.erase(o);
    }
    PI0X_HIP(hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal));
    pi0x_status st = launch_eager(h->cap_stream);
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamEndCapture(h->cap_stream, &graph);
    if (st != PI0X_OK) {
      if (graph) (void)hipGraphDestroy(graph);
      return st;
    }
    if (e != hipSuccess) return fail(PI0X_ERR_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      (void)hipGraphDestroy(graph);
      return fail(PI0X_ERR_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
    }
    it = h->graphs.emplace(key, std::make_pair(graph, exec)).first;
    h->graph_order.push_back(key);
  }
  PI0X_HIP(hipGraphLaunch(it->second.second, stream));
  return PI0X_OK;
}

pi0x_status check_config(const pi0x_config* c) {
  if (!c) return fail(PI0X_ERR_INVALID_ARG, "config is NULL");
  if (c->width <= 0 || c->depth <= 0 || c->mlp_dim <= 0 || c->num_heads <= 0 || c->num_kv_heads <= 0 ||
      c->head_dim <= 0 || c->action_horizon <= 0 || c->action_dim <= 0 || c->state_dim <= 0 || c->max_batch <= 0 ||
      c->max_prefix_len < 0 || c->max_steps <= 0)
    return fail(PI0X_ERR_INVALID_ARG, "config has a non-positive dimension or capacity");
  if (c->dtype != PI0X_FP32 && c->dtype != PI0X_BF16) return fail(PI0X_ERR_DTYPE, "unknown dtype");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f) || !(c->time_min_period > 0.f) || !(c->time_max_period > 0.f))
    return fail(PI0X_ERR_INVALID_ARG, "config has an invalid rms_eps, rope_theta or time period");
  if (c->num_kv_heads != 1) return fail(PI0X_ERR_SHAPE, "only num_kv_heads == 1 is supported");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return fail(PI0X_ERR_SHAPE, "head_dim must be 32, 64, 128 or 256");
  if (c->width % 256 != 0) return fail(PI0X_ERR_SHAPE, "width must be a multiple of 256");
  if (c->mlp_dim % 64 != 0) return fail(PI0X_ERR_SHAPE, "mlp_dim must be a multiple of 64");
  if ((c->num_heads * c->head_dim) % 64 != 0) return fail(PI0X_ERR_SHAPE, "num_heads*head_dim must be a multiple of 64");
  if (c->action_dim > 64 || c->state_dim > 64) return fail(PI0X_ERR_SHAPE, "action_dim and state_dim must be <= 64");
  if ((long)c->max_batch * (c->action_horizon + 1) > (1L << 24)) return fail(PI0X_ERR_CAPACITY, "max_batch too large");
  return PI0X_OK;
}

size_t weight_count(const pi0x_config* c) {
  const size_t W = c->width, M = c->mlp_dim, qd = (size_t)c->num_heads * c->head_dim, kd = (size_t)c->num_kv_heads * c->head_dim;
  const size_t A = c->action_dim, Sd = c->state_dim;
  const size_t layer = W + qd * W + 2 * kd * W + W * qd + W + 3 * M * W;
  return layer * c->depth + W + (W * Sd + W) + (W * A + W) + (W * 2 * W + W) + (W * W + W) + (A * W + A);
}

template <typename T>
void put(std::vector<T>& dst, size_t i, float v);
template <>
void put<float>(std::vector<float>& dst, size_t i, float v) { dst[i] = v; }
template <>
void put<uint16_t>(std::vector<uint16_t>& dst, size_t i, float v) { dst[i] = host_bf16(v); }

template <typename E>
pi0x_status upload_weights(pi0x_expert* h, const float* blob) {
  const int W = h->W, M = h->M, qd = h->qd, dh = h->dh, half = dh / 2;
  const size_t layer_sz = (size_t)W + (size_t)qd * W + 2 * (size_t)dh * W + (size_t)W * qd + W + 3 * (size_t)M * W;
  auto up = [&](void** dst, const std::vector<E>& v) -> pi0x_status {
    PI0X_TRY(h->alloc(dst, v.size() * sizeof(E)));
    PI0X_HIP(hipMemcpy(*dst, v.data(), v.size() * sizeof(E), hipMemcpyHostToDevice));
    return PI0X_OK;
  };
  auto upf = [&](float** dst, const float* src, size_t n, bool one_plus) -> pi0x_status {
    std::vector<float> v(src, src + n);
    if (one_plus)
      for (auto& x : v) x = 1.0f + x;
    PI0X_TRY(h->allocT(dst, n * sizeof(float)));
    PI0X_HIP(hipMemcpy(*dst, v.data(), n * sizeof(float), hipMemcpyHostToDevice));
    return PI0X_OK;
  };
  h->layers.resize(h->D);
  for (int l = 0; l < h->D; ++l) {
    const float* p = blob + (size_t)l * layer_sz;
    const float* in_norm = p;
    const float* wq = in_norm + W;
    const float* wk = wq + (size_t)qd * W;
    const float* wv = wk + (size_t)dh * W;
    const float* wo = wv + (size_t)dh * W;
    const float* post = wo + (size_t)W * qd;
    const float* wg = post + W;
    const float* wu = wg + (size_t)M * W;
    const float* wd = wu + (size_t)M * W;
    Layer& ly = h->layers[l];
    // q/k/v with q and k rows paired for rotate-half RoPE
    {
      const int rows = qd + 2 * dh;
      std::vector<E> v((size_t)rows * W);
      for (int c = 0; c < rows; ++c) {
        const float* src;
        if (c < qd + dh) {
          const int head = c / dh, w = c % dh;
          const int orig = ((w % 32) / 16) * half + (w / 32) * 16 + (w % 16);
          src = head < h->nh ? wq + ((size_t)head * dh + orig) * W : wk + (size_t)orig * W;
        } else {
          src = wv + (size_t)(c - qd - dh) * W;
        }
        for (int k = 0; k < W; ++k) put<E>(v, (size_t)c * W + k, src[k]);
      }
      PI0X_TRY(up(&ly.wqkv, v));
    }
    {
      std::vector<E> v((size_t)W * qd);
      for (size_t i = 0; i < v.size(); ++i) put<E>(v, i, wo[i]);
      PI0X_TRY(up(&ly.wo, v));
    }
    {
      std::vector<E> v((size_t)2 * M * W);
      for (int c = 0; c < 2 * M; ++c) {
        const int pblk = c / 32, sel = (c % 32) / 16, e = c % 16;
        const float* src = (sel == 0 ? wg : wu) + ((size_t)pblk * 16 + e) * W;
        for (int k = 0; k < W; ++k) put<E>(v, (size_t)c * W + k, src[k]);
      }
      PI0X_TRY(up(&ly.wgu, v));
    }
    {
      std::vector<E> v((size_t)W * M);
      for (size_t i = 0; i < v.size(); ++i) put<E>(v, i, wd[i]);
      PI0X_TRY(up(&ly.wdown, v));
    }
    PI0X_TRY(upf(&ly.in1p, in_norm, W, true));
    PI0X_TRY(upf(&ly.post1p, post, W, true));
  }
  const float* p = blob + (size_t)h->D * layer_sz;
  const float* final_norm = p;
  const float* ws = final_norm + W;
  const float* bs = ws + (size_t)W * h->Sd;
  const float* wi = bs + W;
  const float* bi = wi + (size_t)W * h->A;
  const float* wmi = bi + W;
  const float* bmi = wmi + (size_t)W * 2 * W;
  const float* wmo = bmi + W;
  const float* bmo = wmo + (size_t)W * W;
  const float* wout = bmo + W;
  const float* bout = wout + (size_t)h->A * W;
  PI0X_TRY(upf(&h->final1p, final_norm, W, true));
  {
    std::vector<E> va((size_t)W * W), vt((size_t)W * W), vo((size_t)W * W);
    for (int r = 0; r < W; ++r)
      for (int k = 0; k < W; ++k) {
        put<E>(va, (size_t)r * W + k, wmi[(size_t)r * 2 * W + k]);
        put<E>(vt, (size_t)r * W + k, wmi[(size_t)r * 2 * W + W + k]);
        put<E>(vo, (size_t)r * W + k, wmo[(size_t)r * W + k]);
      }
    PI0X_TRY(up(&h->w_ta, va));
    PI0X_TRY(up(&h->w_tt, vt));
    PI0X_TRY(up(&h->w_mo, vo));
  }
  // small head matrices and every bias stay float32 (bf16 mode: the blob's
  // values rounded to bf16, held exactly in float32)
  auto small = [&](float** dst, const float* src, size_t n) -> pi0x_status {
    std::vector<float> v(src, src + n);
    if (h->cfg.dtype == PI0X_BF16)
      for (auto& x : v) {
        uint32_t u = (uint32_t)host_bf16(x) << 16;
        std::memcpy(&x, &u, 4);
      }
    PI0X_TRY(h->allocT(dst, n * sizeof(float)));
    PI0X_HIP(hipMemcpy(*dst, v.data(), n * sizeof(float), hipMemcpyHostToDevice));
    return PI0X_OK;
  };
  PI0X_TRY(small(&h->b_mi, bmi, W));
  PI0X_TRY(small(&h->b_mo, bmo, W));
  PI0X_TRY(small(&h->w_in, wi, (size_t)W * h->A));
  PI0X_TRY(small(&h->b_in, bi, W));
  PI0X_TRY(small(&h->w_s, ws, (size_t)W * h->Sd));
  PI0X_TRY(small(&h->b_s, bs, W));
  PI0X_TRY(small(&h->w_out, wout, (size_t)h->A * W));
  PI0X_TRY(small(&h->b_out, bout, h->A));
  return PI0X_OK;
}

pi0x_status create_impl(const pi0x_config* cfg, const void* weights_host, size_t weights_bytes, pi0x_expert* h) {
  h->cfg = *cfg;
  PI0X_HIP(hipGetDevice(&h->device));
  h->esz = cfg->dtype == PI0X_BF16 ? 2 : 4;
  h->W = cfg->width; h->D = cfg->depth; h->M = cfg->mlp_dim; h->nh = cfg->num_heads; h->dh = cfg->head_dim;
  h->H = cfg->action_horizon; h->A = cfg->action_dim; h->Sd = cfg->state_dim; h->S = h->H + 1;
  h->qd = h->nh * h->dh; h->nqkv = h->qd + 2 * h->dh; h->Bmax = cfg->max_batch; h->Lmax = cfg->max_prefix_len;
  const float* blob = static_cast<const float*>(weights_host);
  // weights stored in bf16 mode may hold non-finite values; nothing to check
  if (cfg->dtype == PI0X_BF16) PI0X_TRY(upload_weights<uint16_t>(h, blob));
  else PI0X_TRY(upload_weights<float>(h, blob));

  const size_t R = (size_t)h->Bmax * h->S, AR = (size_t)h->Bmax * h->H, e = h->esz;
  PI0X_TRY(h->allocT(&h->hbuf, R * h->W * 4));
  PI0X_TRY(h->alloc(&h->y, R * h->W * e));
  PI0X_TRY(h->alloc(&h->qkv, R * h->nqkv * e));
  PI0X_TRY(h->alloc(&h->o, R * h->qd * e));
  PI0X_TRY(h->alloc(&h->gbuf, R * h->M * e));
  PI0X_TRY(h->alloc(&h->ain, AR * h->W * e));
  PI0X_TRY(h->alloc(&h->u, AR * h->W * e));
  PI0X_TRY(h->allocT(&h->x, AR * h->A * 4));
  PI0X_TRY(h->alloc(&h->tau, (size_t)cfg->max_steps * h->W * e));
  PI0X_TRY(h->allocT(&h->tbias, (size_t)cfg->max_steps * h->W * 4));
  PI0X_TRY(h->allocT(&h->gemm_partial, kGemmPartialFloats * 4));
  PI0X_TRY(h->allocT(&h->gemm_counters, (size_t)kCounters * 4));
  PI0X_HIP(hipMemset(h->gemm_counters, 0, (size_t)kCounters * 4));
  // split-KV partials for up to 512 (query tile, split) pairs; the launcher
  // only splits when fewer than 128 query tiles exist
  h->attn_partial_floats = (size_t)512 * (2 + h->dh / 4) * 256;
  PI0X_TRY(h->allocT(&h->attn_partial, h->attn_partial_floats * 4));
  PI0X_TRY(h->allocT(&h->attn_counters, (size_t)kCounters * 4));
  PI0X_HIP(hipMemset(h->attn_counters, 0, (size_t)kCounters * 4));
  PI0X_TRY(h->allocT(&h->desc, sizeof(CallDesc)));
  PI0X_HIP(hipMemset(h->desc, 0, sizeof(CallDesc)));
  const int P = h->Lmax + h->S + 1;
  PI0X_TRY(h->allocT(&h->rope_cos, (size_t)P * (h->dh / 2) * 4));
  PI0X_TRY(h->allocT(&h->rope_sin, (size_t)P * (h->dh / 2) * 4));
  const int n = P * (h->dh / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, P, h->dh, (double)cfg->rope_theta,
                     h->rope_cos, h->rope_sin);
  PI0X_HIP(hipGetLastError());
  PI0X_HIP(hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking));
  PI0X_HIP(hipDeviceSynchronize());
  (void)weights_bytes;
  return PI0X_OK;
}

void destroy_impl(pi0x_expert* h) {
  (void)hipDeviceSynchronize();
  for (auto& kv : h->graphs) {
    (void)hipGraphExecDestroy(kv.second.second);
    (void)hipGraphDestroy(kv.second.first);
  }
  h->graphs.clear();
  if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
  for (void* p : h->allocs) (void)hipFree(p);
  h->allocs.clear();
}

pi0x_status check_call(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                       const int32_t* valid, const float* state, const float* xin, const float* out) {
  if (!h) return fail(PI0X_ERR_INVALID_ARG, "handle is NULL");
  if (!valid || !state || !xin || !out) return fail(PI0X_ERR_INVALID_ARG, "a device pointer argument is NULL");
  if (prefix_len > 0 && !prefix_kv) return fail(PI0X_ERR_INVALID_ARG, "prefix_kv is NULL");
  if (batch < 1) return fail(PI0X_ERR_INVALID_ARG, "batch must be >= 1");
  if (prefix_len < 0) return fail(PI0X_ERR_INVALID_ARG, "prefix_len must be >= 0");
  if (batch > h->Bmax) return fail(PI0X_ERR_CAPACITY, "batch exceeds max_batch");
  if (prefix_len > h->Lmax) return fail(PI0X_ERR_CAPACITY, "prefix_len exceeds max_prefix_len");
  int dev = -1;
  PI0X_HIP(hipGetDevice(&dev));
  if (dev != h->device) return fail(PI0X_ERR_INVALID_ARG, "the current HIP device is not the handle's device");
  return PI0X_OK;
}

}  // namespace

extern "C" {

void pi0x_config_default(pi0x_config* c) {
  if (!c) return;
  c->width = 1024;
  c->depth = 18;
  c->mlp_dim = 4096;
  c->num_heads = 8;
  c->num_kv_heads = 1;
  c->head_dim = 256;
  c->action_horizon = 50;
  c->action_dim = 32;
  c->state_dim = 32;
  c->max_batch = 64;
  c->max_prefix_len = 1024;
  c->max_steps = 64;
  c->rms_eps = 1e-6f;
  c->rope_theta = 10000.0f;
  c->time_min_period = 4e-3f;
  c->time_max_period = 4.0f;
  c->dtype = PI0X_BF16;
  c->use_graphs = 1;
}

size_t pi0x_weight_count(const pi0x_config* cfg) {
  if (!cfg || cfg->width <= 0 || cfg->depth <= 0 || cfg->mlp_dim <= 0 || cfg->num_heads <= 0 ||
      cfg->num_kv_heads <= 0 || cfg->head_dim <= 0 || cfg->action_dim <= 0 || cfg->state_dim <= 0)
    return 0;
  return weight_count(cfg);
}

pi0x_status pi0x_expert_create(const pi0x_config* cfg, const void* weights_host, size_t weights_bytes,
                               pi0x_expert** out) {
  if (!out) return fail(PI0X_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  PI0X_TRY(check_config(cfg));
  if (!weights_host) return fail(PI0X_ERR_INVALID_ARG, "weights_host is NULL");
  const size_t n = weight_count(cfg);
  if (weights_bytes != n * sizeof(float))
    return fail(PI0X_ERR_SHAPE, "weights_bytes is " + std::to_string(weights_bytes) + ", expected " +
                                    std::to_string(n * sizeof(float)));
  pi0x_expert* h = new (std::nothrow) pi0x_expert();
  if (!h) return fail(PI0X_ERR_OOM, "host allocation failed");
  pi0x_status s = create_impl(cfg, weights_host, weights_bytes, h);
  if (s != PI0X_OK) {
    std::string msg = g_err;
    destroy_impl(h);
    delete h;
    g_err = msg;
    return s;
  }
  *out = h;
  return PI0X_OK;
}

pi0x_status pi0x_denoise(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                         const int32_t* prefix_valid_len, const float* state, const float* noise, int32_t num_steps,
                         float* actions_out, hipStream_t stream) {
  PI0X_TRY(check_call(h, batch, prefix_len, prefix_kv, prefix_valid_len, state, noise, actions_out));
  if (num_steps < 1) return fail(PI0X_ERR_INVALID_ARG, "num_steps must be >= 1");
  if (num_steps > h->cfg.max_steps) return fail(PI0X_ERR_CAPACITY, "num_steps exceeds max_steps");
  hipLaunchKernelGGL(set_desc_kernel, dim3(1), dim3(1), 0, stream, h->desc, prefix_kv, prefix_valid_len, state, noise,
                     actions_out, 0.f);
  PI0X_HIP(hipGetLastError());
  return run(h, batch, prefix_len, num_steps, stream);
}

pi0x_status pi0x_denoise_step(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                              const int32_t* prefix_valid_len, const float* state, const float* x_t, float t,
                              float* v_out, hipStream_t stream) {
  PI0X_TRY(check_call(h, batch, prefix_len, prefix_kv, prefix_valid_len, state, x_t, v_out));
  hipLaunchKernelGGL(set_desc_kernel, dim3(1), dim3(1), 0, stream, h->desc, prefix_kv, prefix_valid_len, state, x_t,
                     v_out, t);
  PI0X_HIP(hipGetLastError());
  return run(h, batch, prefix_len, 0, stream);
}

void pi0x_expert_destroy(pi0x_expert* h) {
  if (!h) return;
  (void)hipSetDevice(h->device);
  destroy_impl(h);
  delete h;
}

const char* pi0x_last_error(void) { return g_err.c_str(); }

}  // extern "C"
