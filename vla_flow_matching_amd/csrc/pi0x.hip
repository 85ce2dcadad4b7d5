// pi0x runtime: the C ABI of include/pi0x.h on top of the gfx950 kernels.
//
// create() repacks the nn.Linear-layout weight blob into the layouts the
// kernels want and uploads it:
//  * q/k rows of every head paired for rotate-half RoPE (stored row block 2p =
//    head elements 16p.., block 2p+1 = half+16p..), v rows after them;
//  * gate/up rows interleaved in blocks of 16 (block 2p = gate rows 16p..,
//    block 2p+1 = up rows 16p..);
//  * the Gemma norm scales (1 + w) of the input and post-attention norms folded
//    into the columns of the q/k/v and gate/up weights (the kernels apply the
//    1/rms row factor in the GEMM epilogue);
//  * action_time_mlp_in split into its time half (a GEMM once per call for
//    every step's time features) and its action half, which is multiplied
//    into action_in_proj (both linear) to a width x action_dim matrix;
//  * action_out_proj with the final norm's (1 + w) folded into its columns.
// It also builds the float32 rotary table on the device and allocates every
// workspace for the handle's capacity.
//
// One Euler step is 3 + 5 * depth kernels: the first layer of the time MLP
// (plus the state token copy), action_time_mlp_out (writes the action rows of
// the residual stream), per layer [q/k/v + RoPE, attention, o_proj + residual,
// gate/up + GeGLU, down + residual], and action_out_proj + Euler update (the
// final norm's 1/rms applied as a row scale), plus a reduce launch for every
// projection split over K and a combine launch for attention split over keys
// (small and mid batches).  Once per call: the time
// features of every step, the time half of action_time_mlp_in for every step,
// the transpose of the prefix values and the state tokens.  A call writes a
// small device descriptor with its pointers and replays the hipGraph recorded
// for (batch, prefix length, steps, mode, loop options); the graph is recorded
// on first use, so later calls with new buffers or new valid lengths replay it
// unchanged.
//
// The prefix pass (pi0x_prefill) runs on a handle of its own that holds only
// decoder layers; it reuses the same GEMM, attention and epilogue kernels and
// writes the per-layer K/V cache the denoise loop reads.
#include "pi0x.h"

#include <cmath>
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <type_traits>
#include <vector>

#include "attention.h"
#include "host_pack.h"
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

#define PI0X_HIP(x)                                                                                 \
  do {                                                                                              \
    hipError_t e_ = (x);                                                                            \
    if (e_ != hipSuccess) return fail(PI0X_ERR_HIP, std::string(#x) + ": " + hipGetErrorString(e_)); \
  } while (0)

#define PI0X_TRY(x)               \
  do {                            \
    pi0x_status s_ = (x);         \
    if (s_ != PI0X_OK) return s_; \
  } while (0)

constexpr int kMaxGraphs = 32;
constexpr size_t kGemmPartialFloats = (size_t)16 << 20;  // split-K partial tiles (float32 path)
// K-split partials of the bf16 tile GEMM (128x128 tiles): used while
// splits x tiles <= 512, so splits x rows x N <= 512 x 128 x 128 floats
// whatever the shape.
constexpr size_t kSplitPartialFloats = (size_t)512 * 128 * 128;
// Attention key splits: used while fewer than kAttnSplitMinBlocks 128-query
// tiles exist; at most kAttnPartialBlocks split blocks per launch.
constexpr int kAttnSplitMinBlocks = 128;
constexpr int kAttnPartialBlocks = 256;
// Key counts are padded to 64 (the bf16 key block; float32 uses 32).
inline int prefix_pad(int L) { return ((L > 0 ? L : 1) + 63) / 64 * 64; }
constexpr int kCounters = 1 << 16;

struct Layer {
  void* wqkv;   // [(H+2)*D][W], q/k rows paired for RoPE, columns scaled by (1 + input_norm)
  void* wo;     // [W][H*D]
  void* wgu;    // [2M][W], gate/up interleaved by 16 rows, columns scaled by (1 + post_norm)
  void* wdown;  // [W][M]
};

// Loop variants of page 3 (Wall-X, generate_flow_action); all zero is the pi0
// sampler of page 1.
struct LoopOpts {
  int zero_to_one = 0, xpred = 0, causal = 0, blend = 0;
  // pi0x_debug_velocity_until: stop after this stage (PI0X_DEBUG_AFTER_*) of
  // this layer; -1 runs everything (the debug calls never use graphs)
  int stop_stage = -1, stop_layer = -1;
  int bits() const { return zero_to_one | xpred << 1 | causal << 2 | blend << 3; }
  bool stop_at(int stage, int layer) const {
    return stop_stage == stage && (stage == PI0X_DEBUG_AFTER_EMBED || stop_layer == layer);
  }
};

struct Key {
  int B, L, N, mode, opts;
  bool operator<(const Key& o) const {
    return std::tie(B, L, N, mode, opts) < std::tie(o.B, o.L, o.N, o.mode, o.opts);
  }
};

int round_up(int x, int m) { return (x + m - 1) / m * m; }

}  // namespace

struct pi0x_expert {
  pi0x_config cfg;
  int device = 0;
  int esz = 4;
  int W, D, M, nh, dh, H, A, Sd, S, qd, nqkv, Bmax, Lmax, Lpmax, Sp;
  std::vector<void*> allocs;
  std::vector<Layer> layers;
  void *w_tt = nullptr, *w_mo = nullptr;  // time half of action_time_mlp_in, action_time_mlp_out
  float* w_comb = nullptr;  // [A][W] (W_mi,a W_in)^T: action half of action_time_mlp_in times action_in_proj
  void* w_outp = nullptr;   // [Apad][W] action_out_proj, columns scaled by (1 + final_norm), rows >= A zero
  int Apad = 0;
  float *b_mi = nullptr, *b_mo = nullptr, *w_s = nullptr, *b_s = nullptr, *b_out = nullptr;
  float *rope_cos = nullptr, *rope_sin = nullptr;  // [position][head_dim/2]
  float2* rope_cs = nullptr;                        // per call: (cos, sin) of every suffix row [R][head_dim/2]
  float* hs = nullptr;  // state tokens of the call [B][W]
  float* hbuf = nullptr;  // residual stream [R][W] float32
  void* hb = nullptr;     // bf16 copy of the residual stream (bf16 mode)
  float* ssq = nullptr;   // per-row sum-of-squares partials of the residual stream [R][W/16]
  void *qk = nullptr, *o = nullptr, *gbuf = nullptr, *u = nullptr, *tau = nullptr;
  void *vts = nullptr, *vtp = nullptr;  // suffix / prefix values, transposed
  float *x = nullptr, *tbias = nullptr;
  float* gemm_partial = nullptr;
  float* stream_partial = nullptr;  // K-split partial tiles of the M <= 64 bf16 GEMMs
  size_t stream_partial_n = 0;
  float* attn_partial = nullptr;  // split attention states [blocks][2 + head_dim/4][512]
  size_t attn_partial_n = 0;      // its float32 words
  float* split_partial = nullptr;  // K-split partial tiles of the bf16 tile GEMM (prefix pass)
  unsigned* gemm_counters = nullptr;
  CallDesc* desc = nullptr;
  NormDev* norm = nullptr;  // boundary normalization statistics (all modes 0 at create)
  hipStream_t cap_stream = nullptr;
  struct Graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    hipEvent_t done = nullptr;  // recorded after each replay: the graph is idle once it completes
  };
  std::map<Key, Graph> graphs;
  std::vector<Key> graph_order;
  // kernel timing (pi0x_set_timing): event pairs recorded around launches
  bool timing = false;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  std::vector<std::pair<int, size_t>> ev_marks;  // (kernel class, index of the start event)

  bool bf16() const { return cfg.dtype == PI0X_BF16; }

  // Every buffer is followed by a guard of kGuardBytes holding kGuardByte
  // (set here, at creation); pi0x_expert_check_guards counts the guards a
  // kernel has written into.
  static constexpr size_t kGuardBytes = 4096;
  static constexpr int kGuardByte = 0xA5;
  std::vector<unsigned char*> guards;
  pi0x_status alloc(void** p, size_t bytes) {
    *p = nullptr;
    if (bytes == 0) bytes = 256;
    const size_t body = (bytes + 255) / 256 * 256;
    hipError_t e = hipMalloc(p, body + kGuardBytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(PI0X_ERR_OOM, "hipMalloc of " + std::to_string(bytes) + " bytes failed");
    }
    allocs.push_back(*p);
    unsigned char* g = static_cast<unsigned char*>(*p) + body;
    e = hipMemset(g, kGuardByte, kGuardBytes);
    if (e != hipSuccess) return fail(PI0X_ERR_HIP, std::string("hipMemset of a guard: ") + hipGetErrorString(e));
    guards.push_back(g);
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

// The prefix-pass handle: the same core (decoder layers, workspaces, graphs)
// without an action head.
struct pi0x_prefix_model {
  pi0x_expert core;
};

namespace {

// ---------------------------------------------------------------------------
// Kernel timing: while enabled, calls run eagerly and every launch of a
// tracked kernel class is bracketed by a pair of HIP events on its stream.
// ---------------------------------------------------------------------------
pi0x_status next_event(pi0x_expert* h, hipEvent_t* e) {
  if (h->ev_used == h->ev_pool.size()) {
    hipEvent_t ev;
    PI0X_HIP(hipEventCreate(&ev));
    h->ev_pool.push_back(ev);
  }
  *e = h->ev_pool[h->ev_used++];
  return PI0X_OK;
}

struct Timed {
  pi0x_expert* h;
  hipStream_t s;
  int cls;
  size_t start = 0;
  bool on;
  pi0x_status st = PI0X_OK;
  Timed(pi0x_expert* h_, hipStream_t s_, int c) : h(h_), s(s_), cls(c), on(h_->timing) {
    if (!on) return;
    hipEvent_t e;
    st = next_event(h, &e);
    if (st == PI0X_OK && hipEventRecord(e, s) != hipSuccess) st = fail(PI0X_ERR_HIP, "hipEventRecord failed");
    start = h->ev_used - 1;
  }
  pi0x_status done() {
    if (!on || st != PI0X_OK) return st;
    hipEvent_t e;
    PI0X_TRY(next_event(h, &e));
    PI0X_HIP(hipEventRecord(e, s));
    h->ev_marks.push_back({cls, start});
    return PI0X_OK;
  }
};

#define PI0X_TIMED(cls, call) \
  do {                        \
    Timed t_(h, s, (cls));    \
    PI0X_TRY(t_.st);          \
    PI0X_TRY(call);           \
    PI0X_TRY(t_.done());      \
  } while (0)

// ---------------------------------------------------------------------------
// GEMM dispatch
// ---------------------------------------------------------------------------
// Column-group width of the sum-of-squares partials a residual producer writes
// for M rows (the wave or block width of the kernel launch_gemm picks for it).
// The bf16 path picks the batch-1 kernels when the call's suffix rows (B * S)
// fit 64; every GEMM of the call then follows that choice, so the residual
// producers of one call (suffix embedding, o_proj, down) write partials of one
// group width.
constexpr int kSmallRows = 64;
int producer_group(bool bf16, int M) {
  if (bf16) return M <= kSmallRows ? kStreamGroup : 32;  // stream reduce waves / tile kernel's 32-column wave tiles
  return M <= 1024 ? 32 : 64;
}

struct NormIn {
  const float* ssq = nullptr;
  int np = 0;
};

GemmArgs make_args(pi0x_expert* h, const void* A, int lda, const void* W, int M, int N, int K, NormIn nin) {
  GemmArgs g;
  g.A = A;
  g.lda = lda;
  g.W = W;
  g.ldw = K;
  g.M = M;
  g.N = N;
  g.K = K;
  g.splits = 1;
  g.partial = h->gemm_partial;
  g.counters = h->gemm_counters;
  g.ssq_in = nin.ssq;
  g.ssq_np = nin.np;
  g.norm_dim = h->W;
  g.norm_eps = h->cfg.rms_eps;
  return g;
}

template <typename T, int BM, int BN, int WM, int WN, class Epi>
pi0x_status launch_gemm_cfg(pi0x_expert* h, hipStream_t s, GemmArgs g, const Epi& epi) {
  (void)h;
  const int tiles = ((g.M + BM - 1) / BM) * (g.N / BN);
  const int KI = g.K / 32;
  int splits = 1;
  if (tiles < 160) {
    splits = (256 + tiles - 1) / tiles;
    if (splits > KI / 2) splits = KI / 2;
    if (splits > 16) splits = 16;
    if (splits < 1) splits = 1;
    while (splits > 1 && (size_t)tiles * splits * BM * BN > kGemmPartialFloats) --splits;
    if (tiles > kCounters) splits = 1;
  }
  g.splits = splits;
  dim3 grid(g.N / BN, (g.M + BM - 1) / BM, splits);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, Epi>), grid, dim3(256), 0, s, g, epi);
  PI0X_HIP(hipGetLastError());
  return PI0X_OK;
}

// Tile kernel configurations (128-row tiles, 2x2 waves, K slices of 64):
// wide N (gate/up) takes 128x128 tiles double-buffered (64 KB of LDS, 2 blocks
// per CU); the narrower projections take 128x64 tiles, so twice as many
// blocks share the CUs -- double-buffered (48 KB, 3 blocks per CU) for
// K <= 1024, three stages (72 KB, 2 blocks per CU) for the long-K o_proj and
// down.  Residual producers (N = width) are always 128x64: their
// sum-of-squares groups are the 32-column wave tiles.
// Tile order (gemm_tile_kernel): each XCD takes a contiguous run of tiles
// in groups of kGroupM row tiles by every column tile.  Measured at batch 64
// (3264 rows, per launch): groups of 2 row tiles for the 128x64 tiles took
// down from 50.6 to 42.4 us and o_proj from 30.7 to 26.7 us against groups
// of 8 (widths 1-4 within 2%); the 128x128 gate/up tiles are fastest with 8
// (70.7 us; 2, 4, 16 and 26 were 0.2-6% slower).
template <int BN>
constexpr int kGroupM = BN == 128 ? 8 : 2;

template <int BN, int ST, class Epi, int BM = 128, int NWM = 2, int NWN = 2>
pi0x_status launch_gemm_tile_cfg(hipStream_t s, GemmArgs g, const Epi& epi, int group_m = kGroupM<BN>) {
  constexpr int BK = 64;
  const int tm = (g.M + BM - 1) / BM, tn = g.N / BN;
  const int blocks = 8 * ((tm * tn * g.splits + 7) / 8);
  constexpr size_t smem = tile_smem_bytes<BM, BN, BK, ST, NWM, NWN>();
  gemm_tile_kernel<BM, BN, BK, ST, NWM, NWN, Epi><<<dim3(blocks), dim3(256), smem, s>>>(g, epi, tm, tn, group_m);
  PI0X_HIP(hipGetLastError());
  return PI0X_OK;
}

template <class Epi>
pi0x_status launch_gemm_tile(hipStream_t s, GemmArgs g, const Epi& epi) {
  if constexpr (std::is_same_v<Epi, EpiQkvRope<bf16>>) {
    // 64x256 tiles (4 waves of 64x64, two blocks per CU) when they make one
    // nearly full round of the chip's 512 resident blocks: batch 64's 3264
    // rows are 51 x 10 = 510 tiles, where 128x64 tiles make 1.35 rounds
    const int t64 = ((g.M + 63) / 64) * (g.N / 256);
    if (g.N % 256 == 0 && t64 > 448 && t64 <= 512) return launch_gemm_tile_cfg<256, 2, Epi, 64, 1, 4>(s, g, epi, 8);
  }
  if (g.N > 4096 && g.N % 128 == 0 && !Epi::kSsq) return launch_gemm_tile_cfg<128, 2>(s, g, epi);
  if (g.K >= 2048) return launch_gemm_tile_cfg<64, 3>(s, g, epi);
  return launch_gemm_tile_cfg<64, 2>(s, g, epi);
}

// The 128x128 tile GEMM split over K (g.K / 64 divisible by splits, N a
// multiple of 128): raw float32 partial tiles, then gemm_reduce_kernel adds
// them in split order and runs the epilogue (residual producers then write
// sum-of-squares partials per kStreamGroup columns).  For long-K projections
// with too few tiles to fill the chip: more tiles in flight per CU hide the
// latency of the weight stream.
template <class Epi>
pi0x_status launch_gemm_tile_split(pi0x_expert* h, hipStream_t s, GemmArgs g, const Epi& epi, int splits) {
  if ((g.K / 64) % splits != 0 || g.N % 128 != 0) return fail(PI0X_ERR_SHAPE, "unsupported K-split GEMM shape");
  if (!h->split_partial || (size_t)splits * g.M * g.N > kSplitPartialFloats)
    return fail(PI0X_ERR_SHAPE, "K-split partials exceed the workspace");
  g.splits = splits;
  g.partial = h->split_partial;
  PI0X_TRY((launch_gemm_tile_cfg<128, 2>(s, g, epi)));
  const int cols = Epi::kPaired ? 512 : kStreamGroup;
  gemm_reduce_kernel<Epi><<<dim3((g.N + cols - 1) / cols, g.M), dim3(64), 0, s>>>(g, epi);
  PI0X_HIP(hipGetLastError());
  return PI0X_OK;
}

template <int NW, int TN, class Epi>
pi0x_status launch_gemm_wide(hipStream_t s, GemmArgs g, const Epi& epi) {
  gemm_wide_kernel<NW, TN, Epi><<<dim3(g.N / (16 * TN)), dim3(NW * 64), 0, s>>>(g, epi);
  PI0X_HIP(hipGetLastError());
  return PI0X_OK;
}

// K slice of one stream block: 256 when it divides K, else 128 or 64.
inline int stream_kb(int K) { return K % 256 == 0 ? 256 : (K % 128 == 0 ? 128 : 64); }
inline size_t stream_partial_floats(int K, int N) { return (size_t)(K / stream_kb(K)) * 64 * N; }

template <class Epi>
pi0x_status launch_gemm_stream(pi0x_expert* h, hipStream_t s, GemmArgs g, const Epi& epi) {
  const int KB = stream_kb(g.K);
  g.splits = g.K / KB;
  g.partial = h->stream_partial;
  if ((size_t)g.splits * g.M * g.N > h->stream_partial_n) return fail(PI0X_ERR_SHAPE, "stream GEMM partials exceed the workspace");
  const dim3 grid(g.N / 64, g.splits);
  if (KB == 256) gemm_stream_kernel<256><<<grid, dim3(256), 0, s>>>(g);
  else if (KB == 128) gemm_stream_kernel<128><<<grid, dim3(256), 0, s>>>(g);
  else gemm_stream_kernel<64><<<grid, dim3(256), 0, s>>>(g);
  PI0X_HIP(hipGetLastError());
  const int cols = Epi::kPaired ? 512 : kStreamGroup;
  gemm_reduce_kernel<Epi><<<dim3((g.N + cols - 1) / cols, g.M), dim3(64), 0, s>>>(g, epi);
  PI0X_HIP(hipGetLastError());
  return PI0X_OK;
}

// The residual producers (kSsq) use the kernel whose column group matches
// producer_group(); the other GEMMs pick their tiling for parallelism.
template <typename T, class Epi>
pi0x_status launch_gemm(pi0x_expert* h, hipStream_t s, const void* A, int lda, const void* W, int M, int N, int K,
                        const Epi& epi, NormIn nin = NormIn(), int path_rows = 0) {
  if (M <= 0) return PI0X_OK;
  if (K % 64 != 0 || N % 64 != 0) return fail(PI0X_ERR_SHAPE, "GEMM dims must be multiples of 64");
  const GemmArgs g = make_args(h, A, lda, W, M, N, K, nin);
  if constexpr (sizeof(T) == 2) {
    if ((path_rows > 0 ? path_rows : M) <= kSmallRows) {
      // Residual producers (the long-K o_proj and down, N = width) split K
      // over blocks: every wide block would read the whole activation slice.
      // The others run one kernel over the whole K: blocks of 16 (32 for
      // paired epilogues) columns, K split over 8 waves where K allows.
      if constexpr (Epi::kSsq) {
        return launch_gemm_stream(h, s, g, epi);
      } else {
        constexpr int TN = Epi::kPaired ? 2 : 1;
        if (K % 512 == 0) return launch_gemm_wide<8, TN>(s, g, epi);
        if (K % 256 == 0) return launch_gemm_wide<4, TN>(s, g, epi);
        return launch_gemm_wide<1, TN>(s, g, epi);
      }
    }
    return launch_gemm_tile(s, g, epi);
  } else {
    // the tile follows the call's path rows, like producer_group(): the
    // action-row MLP output (M = B*H) writes sum-of-squares partials in the
    // column groups its consumers read with the suffix row count (B*S)
    const int rows = path_rows > 0 ? path_rows : M;
    if (rows > 1024 && N % 128 == 0) return launch_gemm_cfg<T, 128, 128, 2, 2>(h, s, g, epi);
    if (rows > 64) return launch_gemm_cfg<T, 128, 64, 2, 2>(h, s, g, epi);
    return launch_gemm_cfg<T, 64, 32, 4, 1>(h, s, g, epi);
  }
}

// Kernels that take more than 64 KiB of dynamic LDS must opt in once.
template <class Epi>
pi0x_status allow_tile_smem() {
  PI0X_HIP(hipFuncSetAttribute((const void*)gemm_tile_kernel<128, 128, 64, 2, 2, 2, Epi>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)tile_smem_bytes<128, 128, 64, 2>()));
  PI0X_HIP(hipFuncSetAttribute((const void*)gemm_tile_kernel<128, 64, 64, 2, 2, 2, Epi>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)tile_smem_bytes<128, 64, 64, 2>()));
  PI0X_HIP(hipFuncSetAttribute((const void*)gemm_tile_kernel<128, 64, 64, 3, 2, 2, Epi>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)tile_smem_bytes<128, 64, 64, 3>()));
  return PI0X_OK;
}

pi0x_status allow_tile_smem_all() {
  PI0X_HIP(hipFuncSetAttribute((const void*)gemm_tile_kernel<64, 256, 64, 2, 1, 4, EpiQkvRope<bf16>>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)tile_smem_bytes<64, 256, 64, 2, 1, 4>()));
  PI0X_TRY(allow_tile_smem<EpiStore<float>>());
  PI0X_TRY(allow_tile_smem<EpiStore<bf16>>());
  PI0X_TRY(allow_tile_smem<EpiSuffixRows<bf16>>());
  PI0X_TRY(allow_tile_smem<EpiResidual<bf16>>());
  PI0X_TRY(allow_tile_smem<EpiQkvRope<bf16>>());
  PI0X_TRY(allow_tile_smem<EpiGeglu<bf16>>());
  PI0X_TRY(allow_tile_smem<EpiEuler>());
  return PI0X_OK;
}

// ---------------------------------------------------------------------------
// Attention dispatch
// ---------------------------------------------------------------------------
// Key blocks of one split: large batches fill the chip with 128-query tiles
// alone; small ones divide each sample's key blocks over gridDim.z and merge
// the splits in attn_combine_kernel.
inline int attn_splits(int B, int tiles, int nblk) {
  if (B * tiles >= kAttnSplitMinBlocks) return 1;
  int sp = std::min(nblk, kAttnPartialBlocks / (B * tiles));
  return std::max(sp, 1);
}

// float32 words of the split partial states one attention launch writes: per
// 128-query tile of a sample and key split, (2 + head_dim/4) x 512 (the
// half-size 4-wave blocks hold half as many per tile and have twice the
// tiles); 0 when the launch does not split.
size_t attn_partial_floats(const pi0x_expert* h, int B, int L, int prefill) {
  const int KB = h->bf16() ? AttnCfg<bf16>::KB : AttnCfg<float>::KB;
  const int S = prefill ? L : h->S;
  const int tiles = (h->nh * S + kAttnQueries - 1) / kAttnQueries;
  const int nblk = (L + KB - 1) / KB + (prefill ? 0 : (h->S + KB - 1) / KB);
  const int splits = attn_splits(B, tiles, nblk);
  return splits > 1 ? (size_t)B * tiles * splits * (2 + h->dh / 4) * 512 : 0;
}

// prefill: the prefix pass, whose L prefix tokens are the queries and whose
// keys are the layer's own (cache + the single-layer V^T buffer vtp).
template <typename T, int DH>
pi0x_status launch_attn_dh(pi0x_expert* h, hipStream_t s, int B, int L, int layer, int causal, int prefill) {
  constexpr int KB = AttnCfg<T>::KB;
  const int Lp = prefix_pad(L);
  const int S = prefill ? L : h->S;
  AttnArgs a;
  a.qk = h->qk;
  a.ldqk = h->qd + DH;
  a.col_k = h->qd;
  a.desc = h->desc;
  a.kv_k_off = ((size_t)layer * 2 + 0) * B * L * DH;
  a.vtp = reinterpret_cast<const T*>(h->vtp) + (prefill ? 0 : (size_t)layer * B * DH * Lp);
  a.Lp = Lp;
  a.vts = prefill ? nullptr : h->vts;
  a.Sp = prefill ? 0 : h->Sp;
  a.B = B;
  a.L = L;
  a.S = S;
  a.nh = h->nh;
  a.out = h->o;
  a.ldo = h->qd;
  a.scale = 1.0f / std::sqrt((float)DH);
  a.causal = causal;
  a.prefill = prefill;
  const int nq = h->nh * S;
  const int nblk = (L + KB - 1) / KB + (prefill ? 0 : (h->S + KB - 1) / KB);
  constexpr size_t smem = attn_smem_bytes<T, DH>();
  a.partial = h->attn_partial;
  if (attn_partial_floats(h, B, L, prefill) > h->attn_partial_n)
    return fail(PI0X_ERR_SHAPE, "attention split partials exceed the workspace");
  // Key-split launches use half-size blocks (64 queries over 4 waves, one
  // wave per SIMD, twice the blocks) when that keeps the same number of key
  // splits: at batch 1, 98 blocks instead of 56 (attention + combine 14.6 ->
  // 13.9 us per layer).  Where the partial-state capacity would cut the splits
  // (batch 16, the prefix pass) the 8-wave blocks measured faster.
  int tiles = (nq + kAttnQueries - 1) / kAttnQueries;
  a.splits = attn_splits(B, tiles, nblk);
  if constexpr (sizeof(T) == 2) {
    constexpr int NW4 = 4;
    const int tiles4 = (nq + NW4 * 16 - 1) / (NW4 * 16);
    if (a.splits > 1 && attn_splits(B, tiles4, nblk) == a.splits) {
      a.tiles = tiles4;
      const int units = B * a.splits * tiles4;
      attn_kernel<T, DH, NW4><<<dim3(8 * ((units + 7) / 8)), dim3(NW4 * 64), smem, s>>>(a);
      PI0X_HIP(hipGetLastError());
      attn_combine_kernel<T, DH, NW4><<<dim3(NW4 / 2 * tiles4, B, attn_combine_chunks<DH>()), dim3(128), 0, s>>>(a);
      PI0X_HIP(hipGetLastError());
      return PI0X_OK;
    }
  }
  a.tiles = tiles;
  const int units = B * a.splits * tiles;
  attn_kernel<T, DH><<<dim3(8 * ((units + 7) / 8)), dim3(AttnCfg<T>::NW * 64), smem, s>>>(a);
  PI0X_HIP(hipGetLastError());
  if (a.splits > 1) {
    attn_combine_kernel<T, DH><<<dim3(AttnCfg<T>::NW / 2 * tiles, B, attn_combine_chunks<DH>()), dim3(128), 0, s>>>(a);
    PI0X_HIP(hipGetLastError());
  }
  return PI0X_OK;
}

template <typename T, int DH>
pi0x_status allow_attn_smem_dh() {
  PI0X_HIP(hipFuncSetAttribute((const void*)attn_kernel<T, DH>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)attn_smem_bytes<T, DH>()));
  if constexpr (sizeof(T) == 2)
    PI0X_HIP(hipFuncSetAttribute((const void*)attn_kernel<T, DH, 4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)attn_smem_bytes<T, DH>()));
  return PI0X_OK;
}

template <typename T>
pi0x_status allow_attn_smem(int dh) {
  switch (dh) {
    case 32: return allow_attn_smem_dh<T, 32>();
    case 64: return allow_attn_smem_dh<T, 64>();
    case 128: return allow_attn_smem_dh<T, 128>();
    case 256: return allow_attn_smem_dh<T, 256>();
  }
  return fail(PI0X_ERR_SHAPE, "unsupported head_dim");
}

template <typename T>
pi0x_status launch_attn(pi0x_expert* h, hipStream_t s, int B, int L, int layer, int causal, int prefill = 0) {
  switch (h->dh) {
    case 32: return launch_attn_dh<T, 32>(h, s, B, L, layer, causal, prefill);
    case 64: return launch_attn_dh<T, 64>(h, s, B, L, layer, causal, prefill);
    case 128: return launch_attn_dh<T, 128>(h, s, B, L, layer, causal, prefill);
    case 256: return launch_attn_dh<T, 256>(h, s, B, L, layer, causal, prefill);
  }
  return fail(PI0X_ERR_SHAPE, "unsupported head_dim");
}

template <typename T>
pi0x_status launch_transpose_v(pi0x_expert* h, hipStream_t s, int B, int L) {
  if (L <= 0) return PI0X_OK;
  const int Lp = prefix_pad(L);
  hipLaunchKernelGGL((transpose_v_kernel<T>), dim3(Lp / 64, (h->dh + 63) / 64, h->D * B), dim3(256), 0, s, h->desc, B,
                     L, h->dh, Lp, reinterpret_cast<T*>(h->vtp));
  PI0X_HIP(hipGetLastError());
  return PI0X_OK;
}

// ---------------------------------------------------------------------------
// The loop: N > 0 is the N-step sampler, N == 0 one velocity evaluation.
// ---------------------------------------------------------------------------
// Step size of step k of N: -1/N on the pi0 grid; t_{k+1} - t_k of the float32
// grid points k/N on the 0 -> 1 grid (exact in float32: neighbouring points
// are within a factor of two of each other).
float step_dt(int k, int N, bool zero_to_one) {
  if (N <= 0) return 0.f;
  if (!zero_to_one) return (float)(-1.0 / (double)N);
  return (float)((double)(k + 1) / (double)N) - (float)((double)k / (double)N);
}

template <typename T>
pi0x_status enqueue(pi0x_expert* h, hipStream_t s, int B, int L, int N, const LoopOpts& lo) {
  const int W = h->W, S = h->S, H = h->H, R = B * S, AR = B * H;
  const int steps = N > 0 ? N : 1;
  const bool bf = h->bf16();
  T* hb = bf ? reinterpret_cast<T*>(h->hb) : nullptr;
  // A operand of the norm-consuming projections: the residual stream itself
  // (its bf16 copy in bf16 mode)
  const void* hA = bf ? h->hb : (const void*)h->hbuf;
  // sum-of-squares partials: one per (row, producer column group); every
  // consumer reads them with its producer's group width
  const int G = producer_group(bf, R);  // state-token copy, action-row MLP output, o_proj
  const int np = W / G;
  const NormIn nin{h->ssq, np};
  // down (the longest-K residual producer): when its 128x64 tiles cannot fill
  // the chip (816 suffix rows at batch 16: 7 x 16 tiles) it runs as 128x128
  // tiles split over K (up to 8 ways, at most 512 blocks), reduced by
  // gemm_reduce_kernel, whose groups are kStreamGroup columns; the next
  // layer's q/k/v and the final projection read those.  o_proj and the
  // action-row MLP output (K <= 2048) measured no faster split and keep the
  // unsplit kernels.
  int dsplit = 1;
  if (bf && R > kSmallRows && ((R + 127) / 128) * (W / 64) < 256 && W % 128 == 0) {
    dsplit = std::min(8, 512 / (((R + 127) / 128) * (W / 128)));
    while (dsplit > 1 && (h->M / 64) % dsplit != 0) --dsplit;
  }
  const int np_down = dsplit > 1 ? W / kStreamGroup : np;
  const NormIn nin_down{h->ssq, np_down};
  auto down_proj = [&](const Layer& ly) -> pi0x_status {
    const EpiResidual<T> epi{h->hbuf, hb, W, h->ssq, np_down};
    if constexpr (sizeof(T) == 2) {
      if (dsplit > 1)
        return launch_gemm_tile_split(h, s, make_args(h, h->gbuf, h->M, ly.wdown, R, W, h->M, NormIn()), epi, dsplit);
    }
    return launch_gemm<T>(h, s, h->gbuf, h->M, ly.wdown, R, W, h->M, epi);
  };

  auto time_feats = [&]() -> pi0x_status {
    hipLaunchKernelGGL((time_features_kernel<T>), dim3(steps), dim3(256), 0, s, h->desc, N, lo.zero_to_one, W,
                       (double)h->cfg.time_min_period, (double)h->cfg.time_max_period, (T*)h->tau);
    PI0X_HIP(hipGetLastError());
    return PI0X_OK;
  };
  PI0X_TIMED(PI0X_KERNEL_SUFFIX_EMBED, time_feats());
  // time half of action_time_mlp_in (+ its bias) for every evaluated time
  PI0X_TIMED(PI0X_KERNEL_SUFFIX_EMBED,
             (launch_gemm<T>(h, s, h->tau, W, h->w_tt, steps, W, W, EpiStore<float>{h->tbias, W, h->b_mi, 0})));
  PI0X_TIMED(PI0X_KERNEL_ATTENTION, launch_transpose_v<T>(h, s, B, L));
  auto state_tok = [&]() -> pi0x_status {
    hipLaunchKernelGGL(state_token_kernel, dim3(B), dim3(256), 0, s, h->desc, h->norm, h->Sd, W, h->w_s, h->b_s,
                       h->hs);
    PI0X_HIP(hipGetLastError());
    return PI0X_OK;
  };
  PI0X_TIMED(PI0X_KERNEL_SUFFIX_EMBED, state_tok());
  auto rope_rows = [&]() -> pi0x_status {
    hipLaunchKernelGGL(rope_rows_kernel, dim3(R), dim3(128), 0, s, h->desc, S, L, h->dh / 2, h->rope_cos, h->rope_sin,
                       h->rope_cs, 1);
    PI0X_HIP(hipGetLastError());
    return PI0X_OK;
  };
  PI0X_TIMED(PI0X_KERNEL_QKV_ROPE, rope_rows());
  const int nA = (AR + 3) / 4 * ((W + 255) / 256);
  for (int k = 0; k < steps; ++k) {
    const int first = (k == 0);
    auto suffix_in = [&]() -> pi0x_status {
      hipLaunchKernelGGL((suffix_in_kernel<T>), dim3(nA + B), dim3(256), 0, s, h->desc, h->x, first, AR, nA, h->A, W,
                         S, h->w_comb, h->tbias + (size_t)k * W, (T*)h->u, h->hs, h->hbuf, hb, h->ssq, G);
      PI0X_HIP(hipGetLastError());
      return PI0X_OK;
    };
    PI0X_TIMED(PI0X_KERNEL_SUFFIX_EMBED, suffix_in());
    PI0X_TIMED(PI0X_KERNEL_SUFFIX_EMBED,
               (launch_gemm<T>(h, s, h->u, W, h->w_mo, AR, W, W,
                               EpiSuffixRows<T>{h->hbuf, hb, W, H, S, h->b_mo, h->ssq, np}, NormIn(), R)));
    if (lo.stop_at(PI0X_DEBUG_AFTER_EMBED, 0)) return PI0X_OK;
    for (int l = 0; l < h->D; ++l) {
      const Layer& ly = h->layers[l];
      PI0X_TIMED(PI0X_KERNEL_QKV_ROPE,
                 (launch_gemm<T>(h, s, hA, W, ly.wqkv, R, h->nqkv, W,
                                 EpiQkvRope<T>{(T*)h->qk, h->qd + h->dh, h->qd + h->dh, h->dh, S, h->rope_cs,
                                               (T*)h->vts, h->Sp},
                                 l == 0 ? nin : nin_down)));
      if (lo.stop_at(PI0X_DEBUG_AFTER_QKV, l)) return PI0X_OK;
      PI0X_TIMED(PI0X_KERNEL_ATTENTION, launch_attn<T>(h, s, B, L, l, lo.causal));
      if (lo.stop_at(PI0X_DEBUG_AFTER_ATTENTION, l)) return PI0X_OK;
      PI0X_TIMED(PI0X_KERNEL_O_PROJ, (launch_gemm<T>(h, s, h->o, h->qd, ly.wo, R, W, h->qd,
                                                     EpiResidual<T>{h->hbuf, hb, W, h->ssq, np})));
      if (lo.stop_at(PI0X_DEBUG_AFTER_O_PROJ, l)) return PI0X_OK;
      PI0X_TIMED(PI0X_KERNEL_GATE_UP,
                 (launch_gemm<T>(h, s, hA, W, ly.wgu, R, 2 * h->M, W, EpiGeglu<T>{(T*)h->gbuf, h->M}, nin)));
      if (lo.stop_at(PI0X_DEBUG_AFTER_GATE_UP, l)) return PI0X_OK;
      PI0X_TIMED(PI0X_KERNEL_DOWN, down_proj(ly));
      if (lo.stop_at(PI0X_DEBUG_AFTER_DOWN, l)) return PI0X_OK;
    }
    const int last = (k == steps - 1);
    const EpiEuler epi{h->x, h->desc, h->b_out, H, S, h->A, first, last, N > 0 ? 0 : 1,
                       step_dt(k, N, lo.zero_to_one != 0), h->norm, lo.xpred, lo.blend && first};
    // the final projection has Apad (128) columns: beyond batch 1 its few
    // tiles are split over K (at most 512 blocks) and reduced in split order
    auto final_proj = [&]() -> pi0x_status {
      if constexpr (sizeof(T) == 2) {
        if (R > kSmallRows) {
          int sp = std::min(8, 512 / (((R + 127) / 128) * (h->Apad / 128)));
          while (sp > 1 && (W / 64) % sp != 0) --sp;
          if (sp > 1) return launch_gemm_tile_split(h, s, make_args(h, hA, W, h->w_outp, R, h->Apad, W, nin_down), epi, sp);
        }
      }
      return launch_gemm<T>(h, s, hA, W, h->w_outp, R, h->Apad, W, epi, nin_down);
    };
    PI0X_TIMED(PI0X_KERNEL_FINAL, final_proj());
  }
  return PI0X_OK;
}

// Replays the graph recorded for key (recording it on first use), or runs
// eagerly when graphs are off or kernel timing is on.
template <class F>
pi0x_status run_graph(pi0x_expert* h, const Key& key, F launch_eager, hipStream_t stream) {
  if (!h->cfg.use_graphs || h->timing) return launch_eager(stream);
  auto it = h->graphs.find(key);
  if (it == h->graphs.end()) {
    if ((int)h->graphs.size() >= kMaxGraphs) {
      // the oldest graph may still be replaying from an earlier call: wait
      // for its last replay only (not the whole device) before destroying it
      const Key old = h->graph_order.front();
      h->graph_order.erase(h->graph_order.begin());
      auto o = h->graphs.find(old);
      PI0X_HIP(hipEventSynchronize(o->second.done));
      (void)hipGraphExecDestroy(o->second.exec);
      (void)hipGraphDestroy(o->second.graph);
      (void)hipEventDestroy(o->second.done);
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
    hipEvent_t done = nullptr;
    e = hipEventCreateWithFlags(&done, hipEventDisableTiming);
    if (e != hipSuccess) {
      (void)hipGraphExecDestroy(exec);
      (void)hipGraphDestroy(graph);
      return fail(PI0X_ERR_HIP, std::string("hipEventCreateWithFlags: ") + hipGetErrorString(e));
    }
    it = h->graphs.emplace(key, pi0x_expert::Graph{graph, exec, done}).first;
    h->graph_order.push_back(key);
  }
  PI0X_HIP(hipGraphLaunch(it->second.exec, stream));
  PI0X_HIP(hipEventRecord(it->second.done, stream));
  return PI0X_OK;
}

pi0x_status run(pi0x_expert* h, int B, int L, int N, const LoopOpts& lo, hipStream_t stream) {
  auto launch_eager = [&](hipStream_t s) -> pi0x_status {
    return h->bf16() ? enqueue<bf16>(h, s, B, L, N, lo) : enqueue<float>(h, s, B, L, N, lo);
  };
  return run_graph(h, Key{B, L, N, N > 0 ? 0 : 1, lo.bits()}, launch_eager, stream);
}

// ---------------------------------------------------------------------------
// The call variant that allocates nothing (pi0x_denoise_noalloc).  The call's
// working buffers -- the residual stream, activations, V^T copies, split
// partials, time features and the call descriptor -- are carved out of one
// static device array instead of the handle's workspaces; the kernels are
// the same and take the carved pointers as arguments.  The array's device
// address is resolved once per GPU (scratch_lookup, from pi0x_expert_create,
// with that GPU current): in host code the array's name is only a host-side
// stand-in and is never passed to a kernel or a copy.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = PI0X_NOALLOC_SCRATCH_BYTES;
constexpr int kScratchDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

struct ScratchSlot {
  bool looked_up = false;
  void* ptr = nullptr;  // device address of scratch on this GPU
  std::string err;
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kScratchDevices];

// once per device, with that device current
void scratch_lookup(int dev) {
  if (dev < 0 || dev >= kScratchDevices) return;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchSlot& sl = g_scratch[dev];
  if (sl.looked_up) return;
  sl.looked_up = true;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    sl.err = std::string("hipGetSymbolAddress of the scratch array: ") + hipGetErrorString(e);
    return;
  }
  sl.ptr = p;
}

pi0x_status scratch_of(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (dev < 0 || dev >= kScratchDevices || !g_scratch[dev].looked_up)
    return fail(PI0X_ERR_INVALID_ARG, "no scratch array for this device (create the handle on it first)");
  if (!g_scratch[dev].ptr) return fail(PI0X_ERR_HIP, g_scratch[dev].err);
  *out = g_scratch[dev].ptr;
  return PI0X_OK;
}

// the per-call buffers of a handle
struct CallBufs {
  float *hbuf, *ssq, *hs, *x, *tbias, *stream_partial, *attn_partial, *split_partial, *gemm_partial;
  void *hb, *qk, *vts, *vtp, *o, *gbuf, *u, *tau;
  unsigned* gemm_counters;
  CallDesc* desc;
  float2* rope_cs;
  size_t stream_partial_n, attn_partial_n;
};

CallBufs bufs_of(const pi0x_expert* h) {
  return CallBufs{h->hbuf, h->ssq, h->hs, h->x, h->tbias, h->stream_partial, h->attn_partial, h->split_partial,
                  h->gemm_partial, h->hb, h->qk, h->vts, h->vtp, h->o, h->gbuf, h->u, h->tau, h->gemm_counters,
                  h->desc, h->rope_cs, h->stream_partial_n, h->attn_partial_n};
}

void set_bufs(pi0x_expert* h, const CallBufs& b) {
  h->hbuf = b.hbuf; h->ssq = b.ssq; h->hs = b.hs; h->x = b.x; h->tbias = b.tbias;
  h->stream_partial = b.stream_partial; h->attn_partial = b.attn_partial; h->split_partial = b.split_partial;
  h->gemm_partial = b.gemm_partial; h->hb = b.hb; h->qk = b.qk; h->vts = b.vts; h->vtp = b.vtp; h->o = b.o;
  h->gbuf = b.gbuf; h->u = b.u; h->tau = b.tau; h->gemm_counters = b.gemm_counters; h->desc = b.desc;
  h->rope_cs = b.rope_cs; h->stream_partial_n = b.stream_partial_n; h->attn_partial_n = b.attn_partial_n;
}

// Lays out the buffers of a bf16 call of B samples (B * S <= 64 rows: the
// batch-1 kernels, which use no K-split tile partials), prefix length L and
// `steps` evaluated times from base (nullptr: sizes only), each region
// 256-byte aligned; returns the bytes the call needs.
size_t carve_call_bufs(const pi0x_expert* h, int B, int L, int steps, char* base, CallBufs* b) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += std::max<size_t>((bytes + 255) / 256 * 256, 256);
    return p;
  };
  const size_t R = (size_t)B * h->S, AR = (size_t)B * h->H, e = h->esz, W = h->W;
  *b = CallBufs{};
  b->hbuf = reinterpret_cast<float*>(take(R * W * 4));
  b->hb = take(R * W * e);
  b->ssq = reinterpret_cast<float*>(take(R * (W / 16) * 4));
  b->qk = take(R * (h->qd + h->dh) * e);
  b->vts = take((size_t)B * h->dh * h->Sp * e);
  b->vtp = take((size_t)h->D * B * h->dh * prefix_pad(L) * e);
  b->o = take(R * h->qd * e);
  b->gbuf = take(R * h->M * e);
  b->u = take(AR * W * e);
  b->hs = reinterpret_cast<float*>(take((size_t)B * W * 4));
  b->x = reinterpret_cast<float*>(take(AR * h->A * 4));
  b->tau = take((size_t)steps * W * e);
  b->tbias = reinterpret_cast<float*>(take((size_t)steps * W * 4));
  const int shapes[][2] = {{h->W, h->W}, {h->W, h->nqkv}, {h->qd, h->W}, {h->W, 2 * h->M}, {h->M, h->W}, {h->W, h->Apad}};
  for (const auto& kn : shapes)
    b->stream_partial_n = std::max(b->stream_partial_n, (size_t)(kn[0] / stream_kb(kn[0])) * R * kn[1]);
  b->stream_partial = reinterpret_cast<float*>(take(b->stream_partial_n * 4));
  b->attn_partial_n = attn_partial_floats(h, B, L, 0);
  b->attn_partial = reinterpret_cast<float*>(take(b->attn_partial_n * 4));
  b->desc = reinterpret_cast<CallDesc*>(take(sizeof(CallDesc)));
  b->rope_cs = reinterpret_cast<float2*>(take(R * (h->dh / 2) * sizeof(float2)));
  return off;
}

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// The prefix pass (page 1: the prefix-only branch of
// PaliGemmaWithExpertModel.forward, _compute_layer_prefix_only per layer, as
// sample_actions runs it) on a handle that holds only decoder layers.  Per
// layer: q/k/v + RoPE (the epilogue also stores the post-RoPE k and the v to
// the caller's cache), attention of the prefix tokens over the real ones,
// o_proj + residual, gate/up + GeGLU, down + residual -- the same kernels as
// the expert.  The last layer stops after its k/v: its attention output and
// MLP only feed the prefix hidden states, which the sampler discards (and so
// does the final norm, which is not applied).
// ---------------------------------------------------------------------------
template <typename T>
pi0x_status enqueue_prefix(pi0x_expert* h, hipStream_t s, int B, int L) {
  const int W = h->W, R = B * L, dh = h->dh, Lp = prefix_pad(L);
  const bool bf = h->bf16();
  T* hb = bf ? reinterpret_cast<T*>(h->hb) : nullptr;
  const void* hA = bf ? h->hb : (const void*)h->hbuf;
  // down (the long-K residual producer): when its tiles cannot fill the chip
  // (816 rows: 7 x 16 tiles of 128x128) it is split over K (up to 4 ways, at
  // most 512 blocks) and reduced by gemm_reduce_kernel, whose sum-of-squares
  // groups are kStreamGroup columns; the embedding copy then uses the same
  // groups, since both feed the next q/k/v projection.  o_proj keeps the
  // unsplit kernel's groups for gate/up.
  const int tiles_down = ((R + 127) / 128) * (W / 128);
  int dsplit = 1;
  if (bf && R > kSmallRows && tiles_down < 256 && W % 128 == 0) {
    dsplit = std::max(1, std::min(4, 512 / tiles_down));
    while (dsplit > 1 && (h->M / 64) % dsplit != 0) --dsplit;
  }
  const int G = dsplit > 1 ? kStreamGroup : producer_group(bf, R);  // embedding copy and down
  const int np = W / G;
  const NormIn nin{h->ssq, np};
  const int np_post = W / producer_group(bf, R);  // o_proj
  const NormIn nin_post{h->ssq, np_post};
  auto first = [&]() -> pi0x_status {
    hipLaunchKernelGGL((prefix_in_kernel<T>), dim3(R), dim3(256), 0, s, h->desc, W, h->hbuf, hb, h->ssq, G);
    PI0X_HIP(hipGetLastError());
    hipLaunchKernelGGL(rope_rows_kernel, dim3(R), dim3(128), 0, s, h->desc, L, L, dh / 2, h->rope_cos, h->rope_sin,
                       h->rope_cs, 0);
    PI0X_HIP(hipGetLastError());
    return PI0X_OK;
  };
  PI0X_TIMED(PI0X_KERNEL_SUFFIX_EMBED, first());
  for (int l = 0; l < h->D; ++l) {
    const Layer& ly = h->layers[l];
    EpiQkvRope<T> qe{(T*)h->qk, h->qd + dh, h->qd + dh, dh, L, h->rope_cs, (T*)h->vtp, Lp};
    qe.desc = h->desc;
    qe.k_off = ((size_t)l * 2 + 0) * R * dh;
    qe.v_off = ((size_t)l * 2 + 1) * R * dh;
    PI0X_TIMED(PI0X_KERNEL_QKV_ROPE, (launch_gemm<T>(h, s, hA, W, ly.wqkv, R, h->nqkv, W, qe, nin)));
    if (l == h->D - 1) break;
    PI0X_TIMED(PI0X_KERNEL_ATTENTION, launch_attn<T>(h, s, B, L, l, 0, 1));
    PI0X_TIMED(PI0X_KERNEL_O_PROJ, (launch_gemm<T>(h, s, h->o, h->qd, ly.wo, R, W, h->qd,
                                                   EpiResidual<T>{h->hbuf, hb, W, h->ssq, np_post})));
    PI0X_TIMED(PI0X_KERNEL_GATE_UP,
               (launch_gemm<T>(h, s, hA, W, ly.wgu, R, 2 * h->M, W, EpiGeglu<T>{(T*)h->gbuf, h->M}, nin_post)));
    const EpiResidual<T> down_epi{h->hbuf, hb, W, h->ssq, np};
    auto down = [&]() -> pi0x_status {
      if constexpr (sizeof(T) == 2) {
        if (dsplit > 1)
          return launch_gemm_tile_split(h, s, make_args(h, h->gbuf, h->M, ly.wdown, R, W, h->M, NormIn()), down_epi,
                                        dsplit);
      }
      return launch_gemm<T>(h, s, h->gbuf, h->M, ly.wdown, R, W, h->M, down_epi);
    };
    PI0X_TIMED(PI0X_KERNEL_DOWN, down());
  }
  return PI0X_OK;
}

pi0x_status run_prefix(pi0x_expert* h, int B, int L, hipStream_t stream) {
  auto launch_eager = [&](hipStream_t s) -> pi0x_status {
    return h->bf16() ? enqueue_prefix<bf16>(h, s, B, L) : enqueue_prefix<float>(h, s, B, L);
  };
  return run_graph(h, Key{B, L, 0, 2, 0}, launch_eager, stream);
}

pi0x_status check_config(const pi0x_config* c) {
  std::string msg;
  const pi0x_status st = hostpack::config_error(c, &msg);
  return st == PI0X_OK ? PI0X_OK : fail(st, msg);
}

size_t weight_count(const pi0x_config* c) { return hostpack::weight_count(c); }

// Repacks the blob (host_pack.h) and uploads it.  head == false: a
// prefix-pass blob (decoder layers only).
template <typename E>
pi0x_status upload_weights(pi0x_expert* h, const float* blob, bool head) {
  const hostpack::Dims d{h->W, h->M, h->nh, h->dh, h->A, h->Sd, h->bf16()};
  auto up = [&](void** dst, const std::vector<E>& v) -> pi0x_status {
    PI0X_TRY(h->alloc(dst, v.size() * sizeof(E)));
    PI0X_HIP(hipMemcpy(*dst, v.data(), v.size() * sizeof(E), hipMemcpyHostToDevice));
    return PI0X_OK;
  };
  auto up_f32 = [&](float** dst, const std::vector<float>& v) -> pi0x_status {
    PI0X_TRY(h->allocT(dst, v.size() * sizeof(float)));
    PI0X_HIP(hipMemcpy(*dst, v.data(), v.size() * sizeof(float), hipMemcpyHostToDevice));
    return PI0X_OK;
  };
  h->layers.resize(h->D);
  for (int l = 0; l < h->D; ++l) {
    const hostpack::LayerSrc src = hostpack::layer_src(blob, d, l);
    Layer& ly = h->layers[l];
    PI0X_TRY(up(&ly.wqkv, hostpack::pack_qkv<E>(src, d)));
    PI0X_TRY(up(&ly.wo, hostpack::pack_plain<E>(src.wo, (size_t)h->W * h->qd)));
    PI0X_TRY(up(&ly.wgu, hostpack::pack_gate_up<E>(src, d)));
    PI0X_TRY(up(&ly.wdown, hostpack::pack_plain<E>(src.wd, (size_t)h->W * h->M)));
  }
  if (!head) return PI0X_OK;
  const hostpack::HeadSrc hs = hostpack::head_src(blob, d, h->D);
  PI0X_TRY(up(&h->w_tt, hostpack::pack_time_half<E>(hs, d)));
  PI0X_TRY(up(&h->w_mo, hostpack::pack_plain<E>(hs.wmo, (size_t)h->W * h->W)));
  {
    std::vector<float> comb, bias;
    hostpack::fold_action_in(hs, d, &comb, &bias);
    PI0X_TRY(up_f32(&h->w_comb, comb));
    PI0X_TRY(up_f32(&h->b_mi, bias));
  }
  h->Apad = round_up(h->A, 128);
  PI0X_TRY(up(&h->w_outp, hostpack::pack_out_proj<E>(hs, d, h->Apad)));
  // state_proj and the remaining biases stay float32
  PI0X_TRY(up_f32(&h->b_mo, hostpack::pack_small(hs.bmo, h->W, d.bf16)));
  PI0X_TRY(up_f32(&h->w_s, hostpack::pack_small(hs.ws, (size_t)h->W * h->Sd, d.bf16)));
  PI0X_TRY(up_f32(&h->b_s, hostpack::pack_small(hs.bs, h->W, d.bf16)));
  PI0X_TRY(up_f32(&h->b_out, hostpack::pack_small(hs.bout, h->A, d.bf16)));
  return PI0X_OK;
}

pi0x_status create_impl(const pi0x_config* cfg, const void* weights_host, pi0x_expert* h) {
  h->cfg = *cfg;
  PI0X_HIP(hipGetDevice(&h->device));
  scratch_lookup(h->device);
  h->esz = cfg->dtype == PI0X_BF16 ? 2 : 4;
  h->W = cfg->width; h->D = cfg->depth; h->M = cfg->mlp_dim; h->nh = cfg->num_heads; h->dh = cfg->head_dim;
  h->H = cfg->action_horizon; h->A = cfg->action_dim; h->Sd = cfg->state_dim; h->S = h->H + 1;
  h->qd = h->nh * h->dh; h->nqkv = h->qd + 2 * h->dh; h->Bmax = cfg->max_batch; h->Lmax = cfg->max_prefix_len;
  h->Lpmax = prefix_pad(h->Lmax);
  h->Sp = round_up(h->S, 64);
  const float* blob = static_cast<const float*>(weights_host);
  if (h->bf16()) PI0X_TRY(upload_weights<uint16_t>(h, blob, true));
  else PI0X_TRY(upload_weights<float>(h, blob, true));

  const size_t R = (size_t)h->Bmax * h->S, AR = (size_t)h->Bmax * h->H, e = h->esz;
  PI0X_TRY(h->allocT(&h->hbuf, R * h->W * 4));
  if (h->bf16()) PI0X_TRY(h->alloc(&h->hb, R * h->W * e));
  PI0X_TRY(h->allocT(&h->ssq, R * (h->W / 16) * 4));
  PI0X_TRY(h->alloc(&h->qk, R * (h->qd + h->dh) * e));
  PI0X_TRY(h->alloc(&h->vts, (size_t)h->Bmax * h->dh * h->Sp * e));
  PI0X_HIP(hipMemset(h->vts, 0, (size_t)h->Bmax * h->dh * h->Sp * e));  // columns >= S stay zero
  PI0X_TRY(h->alloc(&h->vtp, (size_t)h->D * h->Bmax * h->dh * h->Lpmax * e));
  PI0X_TRY(h->alloc(&h->o, R * h->qd * e));
  PI0X_TRY(h->alloc(&h->gbuf, R * h->M * e));
  PI0X_TRY(h->alloc(&h->u, AR * h->W * e));
  PI0X_TRY(h->allocT(&h->hs, (size_t)h->Bmax * h->W * 4));
  PI0X_TRY(h->allocT(&h->x, AR * h->A * 4));
  PI0X_TRY(h->alloc(&h->tau, (size_t)cfg->max_steps * h->W * e));
  PI0X_TRY(h->allocT(&h->tbias, (size_t)cfg->max_steps * h->W * 4));
  if (h->bf16()) {
    const int shapes[][2] = {{h->W, h->W}, {h->W, h->nqkv}, {h->qd, h->W}, {h->W, 2 * h->M}, {h->M, h->W}, {h->W, h->Apad}};
    for (const auto& kn : shapes) h->stream_partial_n = std::max(h->stream_partial_n, stream_partial_floats(kn[0], kn[1]));
    PI0X_TRY(h->allocT(&h->stream_partial, h->stream_partial_n * 4));
  }
  h->attn_partial_n = (size_t)kAttnPartialBlocks * (2 + h->dh / 4) * 512;
  PI0X_TRY(h->allocT(&h->attn_partial, h->attn_partial_n * 4));
  if (h->bf16()) PI0X_TRY(h->allocT(&h->split_partial, kSplitPartialFloats * 4));
  if (!h->bf16()) {
    PI0X_TRY(h->allocT(&h->gemm_partial, kGemmPartialFloats * 4));
    PI0X_TRY(h->allocT(&h->gemm_counters, (size_t)kCounters * 4));
    PI0X_HIP(hipMemset(h->gemm_counters, 0, (size_t)kCounters * 4));
  }
  PI0X_TRY(h->allocT(&h->desc, sizeof(CallDesc)));
  PI0X_TRY(h->allocT(&h->norm, sizeof(NormDev)));
  {
    const NormDev none{};
    PI0X_HIP(hipMemcpy(h->norm, &none, sizeof(NormDev), hipMemcpyHostToDevice));
  }
  PI0X_HIP(hipMemset(h->desc, 0, sizeof(CallDesc)));
  const int P = h->Lmax + h->S + 1;
  PI0X_TRY(h->allocT(&h->rope_cos, (size_t)P * (h->dh / 2) * 4));
  PI0X_TRY(h->allocT(&h->rope_sin, (size_t)P * (h->dh / 2) * 4));
  PI0X_TRY(h->allocT(&h->rope_cs, (size_t)h->Bmax * h->S * (h->dh / 2) * sizeof(float2)));
  const int n = P * (h->dh / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, P, h->dh, (double)cfg->rope_theta,
                     h->rope_cos, h->rope_sin);
  PI0X_HIP(hipGetLastError());
  PI0X_HIP(hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking));
  if (h->bf16()) PI0X_TRY(allow_tile_smem_all());
  if (h->bf16()) PI0X_TRY(allow_attn_smem<bf16>(h->dh));
  else PI0X_TRY(allow_attn_smem<float>(h->dh));
  PI0X_HIP(hipDeviceSynchronize());
  return PI0X_OK;
}

// Prefix-pass handle: the decoder layers and the workspaces of
// max_batch x max_prefix_len rows.
constexpr long kMaxPrefixRows = 1L << 16;

pi0x_status check_prefix_config(const pi0x_config* c) {
  std::string msg;
  const pi0x_status st = hostpack::prefix_config_error(c, kMaxPrefixRows, &msg);
  return st == PI0X_OK ? PI0X_OK : fail(st, msg);
}

size_t prefix_weight_count(const pi0x_config* c) { return hostpack::prefix_weight_count(c); }

pi0x_status create_prefix_impl(const pi0x_config* cfg, const void* weights_host, pi0x_expert* h) {
  h->cfg = *cfg;
  PI0X_HIP(hipGetDevice(&h->device));
  h->esz = cfg->dtype == PI0X_BF16 ? 2 : 4;
  h->W = cfg->width; h->D = cfg->depth; h->M = cfg->mlp_dim; h->nh = cfg->num_heads; h->dh = cfg->head_dim;
  h->H = h->A = h->Sd = 0;
  h->qd = h->nh * h->dh; h->nqkv = h->qd + 2 * h->dh; h->Bmax = cfg->max_batch; h->Lmax = cfg->max_prefix_len;
  h->Lpmax = prefix_pad(h->Lmax);
  h->S = h->Lmax;
  h->Sp = 0;
  const float* blob = static_cast<const float*>(weights_host);
  if (h->bf16()) PI0X_TRY(upload_weights<uint16_t>(h, blob, false));
  else PI0X_TRY(upload_weights<float>(h, blob, false));

  const size_t R = (size_t)h->Bmax * h->Lmax, e = h->esz;
  PI0X_TRY(h->allocT(&h->hbuf, R * h->W * 4));
  if (h->bf16()) PI0X_TRY(h->alloc(&h->hb, R * h->W * e));
  PI0X_TRY(h->allocT(&h->ssq, R * (h->W / 16) * 4));
  PI0X_TRY(h->alloc(&h->qk, R * (h->qd + h->dh) * e));
  // one layer's transposed values; never holds a non-finite value the kernels
  // did not compute, so masked keys weigh exactly zero
  const size_t vt_bytes = (size_t)h->Bmax * h->dh * h->Lpmax * e;
  PI0X_TRY(h->alloc(&h->vtp, vt_bytes));
  PI0X_HIP(hipMemset(h->vtp, 0, vt_bytes));
  PI0X_TRY(h->alloc(&h->o, R * h->qd * e));
  PI0X_TRY(h->alloc(&h->gbuf, R * h->M * e));
  if (h->bf16()) {
    const int shapes[][2] = {{h->W, h->nqkv}, {h->qd, h->W}, {h->W, 2 * h->M}, {h->M, h->W}};
    for (const auto& kn : shapes) h->stream_partial_n = std::max(h->stream_partial_n, stream_partial_floats(kn[0], kn[1]));
    PI0X_TRY(h->allocT(&h->stream_partial, h->stream_partial_n * 4));
  }
  h->attn_partial_n = (size_t)kAttnPartialBlocks * (2 + h->dh / 4) * 512;
  PI0X_TRY(h->allocT(&h->attn_partial, h->attn_partial_n * 4));
  if (h->bf16()) PI0X_TRY(h->allocT(&h->split_partial, kSplitPartialFloats * 4));
  if (!h->bf16()) {
    PI0X_TRY(h->allocT(&h->gemm_partial, kGemmPartialFloats * 4));
    PI0X_TRY(h->allocT(&h->gemm_counters, (size_t)kCounters * 4));
    PI0X_HIP(hipMemset(h->gemm_counters, 0, (size_t)kCounters * 4));
  }
  PI0X_TRY(h->allocT(&h->desc, sizeof(CallDesc)));
  PI0X_HIP(hipMemset(h->desc, 0, sizeof(CallDesc)));
  const int P = h->Lmax + 1;
  PI0X_TRY(h->allocT(&h->rope_cos, (size_t)P * (h->dh / 2) * 4));
  PI0X_TRY(h->allocT(&h->rope_sin, (size_t)P * (h->dh / 2) * 4));
  PI0X_TRY(h->allocT(&h->rope_cs, R * (h->dh / 2) * sizeof(float2)));
  const int n = P * (h->dh / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, P, h->dh, (double)cfg->rope_theta,
                     h->rope_cos, h->rope_sin);
  PI0X_HIP(hipGetLastError());
  PI0X_HIP(hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking));
  if (h->bf16()) PI0X_TRY(allow_tile_smem_all());
  if (h->bf16()) PI0X_TRY(allow_attn_smem<bf16>(h->dh));
  else PI0X_TRY(allow_attn_smem<float>(h->dh));
  PI0X_HIP(hipDeviceSynchronize());
  return PI0X_OK;
}

void destroy_impl(pi0x_expert* h) {
  (void)hipDeviceSynchronize();
  for (auto& kv : h->graphs) {
    (void)hipGraphExecDestroy(kv.second.exec);
    (void)hipGraphDestroy(kv.second.graph);
    (void)hipEventDestroy(kv.second.done);
  }
  h->graphs.clear();
  if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
  for (hipEvent_t e : h->ev_pool) (void)hipEventDestroy(e);
  h->ev_pool.clear();
  for (void* p : h->allocs) (void)hipFree(p);
  h->allocs.clear();
}

pi0x_status check_call(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                       const int32_t* valid, const float* state, const float* xin, const float* out) {
  if (!h) return fail(PI0X_ERR_INVALID_ARG, "handle is NULL");
  if (!valid || !state || !xin || !out) return fail(PI0X_ERR_INVALID_ARG, "a device pointer argument is NULL");
  if (prefix_len > 0 && !prefix_kv) return fail(PI0X_ERR_INVALID_ARG, "prefix_kv is NULL");
  if (prefix_len > 0 && reinterpret_cast<uintptr_t>(prefix_kv) % 16 != 0)
    return fail(PI0X_ERR_INVALID_ARG, "prefix_kv must be 16-byte aligned");
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
  pi0x_status s = create_impl(cfg, weights_host, h);
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
  return pi0x_denoise_ex(h, batch, prefix_len, prefix_kv, prefix_valid_len, state, noise, num_steps, nullptr,
                         actions_out, stream);
}

pi0x_status pi0x_denoise_noalloc(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                                 const int32_t* prefix_valid_len, const float* state, const float* noise,
                                 int32_t num_steps, float* actions_out, hipStream_t stream) {
  PI0X_TRY(check_call(h, batch, prefix_len, prefix_kv, prefix_valid_len, state, noise, actions_out));
  if (num_steps < 1) return fail(PI0X_ERR_INVALID_ARG, "num_steps must be >= 1");
  if (num_steps > h->cfg.max_steps) return fail(PI0X_ERR_CAPACITY, "num_steps exceeds max_steps");
  if (!h->bf16()) return fail(PI0X_ERR_DTYPE, "pi0x_denoise_noalloc needs a bf16 handle");
  if ((long)batch * h->S > kSmallRows)
    return fail(PI0X_ERR_CAPACITY, "pi0x_denoise_noalloc takes at most " + std::to_string(kSmallRows) +
                                       " suffix rows (batch * (action_horizon + 1)), got " +
                                       std::to_string((long)batch * h->S));
  CallBufs mine;
  const size_t need = carve_call_bufs(h, batch, prefix_len, num_steps, nullptr, &mine);
  if (need > kNoAllocScratchBytes)
    return fail(PI0X_ERR_CAPACITY, "the call needs " + std::to_string(need) + " bytes of scratch, more than the " +
                                       std::to_string(kNoAllocScratchBytes) + " of PI0X_NOALLOC_SCRATCH_BYTES");
  void* base = nullptr;
  PI0X_TRY(scratch_of(h->device, &base));
  carve_call_bufs(h, batch, prefix_len, num_steps, static_cast<char*>(base), &mine);
  // the suffix values' columns >= S stand for keys that are never visible and
  // must hold zeros, whatever the previous call left in the array
  const size_t vts_words = (size_t)batch * h->dh * h->Sp * h->esz / 4;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)std::min<size_t>((vts_words + 255) / 256, 1024)), dim3(256), 0,
                     stream, reinterpret_cast<uint32_t*>(mine.vts), vts_words);
  PI0X_HIP(hipGetLastError());
  hipLaunchKernelGGL(set_desc_kernel, dim3(1), dim3(1), 0, stream, mine.desc, prefix_kv, prefix_valid_len, state, noise,
                     actions_out, 0.f, nullptr, nullptr);
  PI0X_HIP(hipGetLastError());
  // the handle's buffers are swapped for the carved ones during the enqueue
  const CallBufs saved = bufs_of(h);
  const bool timing = h->timing;
  set_bufs(h, mine);
  h->timing = false;
  const pi0x_status st = enqueue<bf16>(h, stream, batch, prefix_len, num_steps, LoopOpts{});
  set_bufs(h, saved);
  h->timing = timing;
  return st;
}

pi0x_status pi0x_denoise_ex(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                            const int32_t* prefix_valid_len, const float* state, const float* noise,
                            int32_t num_steps, const pi0x_loop_options* options, float* actions_out,
                            hipStream_t stream) {
  PI0X_TRY(check_call(h, batch, prefix_len, prefix_kv, prefix_valid_len, state, noise, actions_out));
  if (num_steps < 1) return fail(PI0X_ERR_INVALID_ARG, "num_steps must be >= 1");
  if (num_steps > h->cfg.max_steps) return fail(PI0X_ERR_CAPACITY, "num_steps exceeds max_steps");
  LoopOpts lo;
  const float *dof_mask = nullptr, *padding = nullptr;
  if (options) {
    if (options->schedule != PI0X_SCHEDULE_PI0 && options->schedule != PI0X_SCHEDULE_ZERO_TO_ONE)
      return fail(PI0X_ERR_INVALID_ARG, "unknown schedule");
    if ((options->x_prediction != 0 && options->x_prediction != 1) ||
        (options->causal_actions != 0 && options->causal_actions != 1))
      return fail(PI0X_ERR_INVALID_ARG, "x_prediction and causal_actions must be 0 or 1");
    if ((options->dof_mask == nullptr) != (options->padding_action == nullptr))
      return fail(PI0X_ERR_INVALID_ARG, "dof_mask and padding_action must both be set or both be NULL");
    lo.zero_to_one = options->schedule == PI0X_SCHEDULE_ZERO_TO_ONE;
    lo.xpred = options->x_prediction;
    lo.causal = options->causal_actions;
    lo.blend = options->padding_action != nullptr;
    dof_mask = options->dof_mask;
    padding = options->padding_action;
  }
  hipLaunchKernelGGL(set_desc_kernel, dim3(1), dim3(1), 0, stream, h->desc, prefix_kv, prefix_valid_len, state, noise,
                     actions_out, 0.f, dof_mask, padding);
  PI0X_HIP(hipGetLastError());
  return run(h, batch, prefix_len, num_steps, lo, stream);
}

pi0x_status pi0x_denoise_step(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                              const int32_t* prefix_valid_len, const float* state, const float* x_t, float t,
                              float* v_out, hipStream_t stream) {
  PI0X_TRY(check_call(h, batch, prefix_len, prefix_kv, prefix_valid_len, state, x_t, v_out));
  hipLaunchKernelGGL(set_desc_kernel, dim3(1), dim3(1), 0, stream, h->desc, prefix_kv, prefix_valid_len, state, x_t,
                     v_out, t, nullptr, nullptr);
  PI0X_HIP(hipGetLastError());
  return run(h, batch, prefix_len, 0, LoopOpts{}, stream);
}

pi0x_status pi0x_debug_velocity_until(pi0x_expert* h, int32_t batch, int32_t prefix_len, const void* prefix_kv,
                                      const int32_t* prefix_valid_len, const float* state, const float* x_t, float t,
                                      int32_t stage, int32_t layer, int32_t buffer, void* dst, size_t dst_bytes,
                                      hipStream_t stream) {
  float* const no_out = reinterpret_cast<float*>(dst);  // never written: every stop comes before the head
  PI0X_TRY(check_call(h, batch, prefix_len, prefix_kv, prefix_valid_len, state, x_t, no_out));
  if (stage < PI0X_DEBUG_AFTER_EMBED || stage > PI0X_DEBUG_AFTER_DOWN)
    return fail(PI0X_ERR_INVALID_ARG, "unknown debug stage");
  if (stage != PI0X_DEBUG_AFTER_EMBED && (layer < 0 || layer >= h->D))
    return fail(PI0X_ERR_INVALID_ARG, "layer out of range");
  const size_t R = (size_t)batch * h->S, e = h->esz;
  const void* src = nullptr;
  size_t bytes = 0;
  switch (buffer) {
    case PI0X_DEBUG_RESIDUAL: src = h->hbuf; bytes = R * h->W * 4; break;
    case PI0X_DEBUG_QK: src = h->qk; bytes = R * (h->qd + h->dh) * e; break;
    case PI0X_DEBUG_VT: src = h->vts; bytes = (size_t)batch * h->dh * h->Sp * e; break;
    case PI0X_DEBUG_ATTN_OUT: src = h->o; bytes = R * h->qd * e; break;
    case PI0X_DEBUG_GEGLU: src = h->gbuf; bytes = R * h->M * e; break;
    default: return fail(PI0X_ERR_INVALID_ARG, "unknown debug buffer");
  }
  if (!dst) return fail(PI0X_ERR_INVALID_ARG, "dst is NULL");
  if (dst_bytes < bytes) return fail(PI0X_ERR_CAPACITY, "dst needs " + std::to_string(bytes) + " bytes");
  hipLaunchKernelGGL(set_desc_kernel, dim3(1), dim3(1), 0, stream, h->desc, prefix_kv, prefix_valid_len, state, x_t,
                     nullptr, t, nullptr, nullptr);
  PI0X_HIP(hipGetLastError());
  LoopOpts lo;
  lo.stop_stage = stage;
  lo.stop_layer = layer;
  const bool timing = h->timing;
  h->timing = false;
  const pi0x_status st = h->bf16() ? enqueue<bf16>(h, stream, batch, prefix_len, 0, lo)
                                   : enqueue<float>(h, stream, batch, prefix_len, 0, lo);
  h->timing = timing;
  PI0X_TRY(st);
  PI0X_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, stream));
  return PI0X_OK;
}

pi0x_status pi0x_set_normalization(pi0x_expert* h, const pi0x_norm* state, const pi0x_norm* action) {
  if (!h) return fail(PI0X_ERR_INVALID_ARG, "handle is NULL");
  NormDev n{};
  auto fill = [](const pi0x_norm* in, int dim, bool forward, int* mode, int* count, float* a, float* d,
                 const char* what) -> pi0x_status {
    *mode = 0;
    *count = 0;
    if (!in || in->mode == PI0X_NORM_NONE) return PI0X_OK;
    if (in->mode != PI0X_NORM_MEAN_STD && in->mode != PI0X_NORM_MIN_MAX)
      return fail(PI0X_ERR_INVALID_ARG, std::string(what) + " normalization: unknown mode");
    if (in->count < 1 || in->count > dim)
      return fail(PI0X_ERR_INVALID_ARG, std::string(what) + " normalization: count must be in [1, " +
                                            std::to_string(dim) + "]");
    if (!in->a || !in->b) return fail(PI0X_ERR_INVALID_ARG, std::string(what) + " normalization: NULL statistics");
    *mode = in->mode;
    *count = in->count;
    for (int j = 0; j < in->count; ++j) {
      a[j] = in->a[j];
      if (in->mode == PI0X_NORM_MEAN_STD) d[j] = forward ? in->b[j] + 1e-8f : in->b[j];
      else d[j] = std::max(in->b[j] - in->a[j], 1e-8f);
    }
    return PI0X_OK;
  };
  PI0X_TRY(fill(state, h->Sd, true, &n.state_mode, &n.state_count, n.sa, n.sd, "state"));
  PI0X_TRY(fill(action, h->A, false, &n.action_mode, &n.action_count, n.aa, n.ad, "action"));
  int cur = 0;
  PI0X_HIP(hipGetDevice(&cur));
  PI0X_HIP(hipSetDevice(h->device));
  const hipError_t e = hipMemcpy(h->norm, &n, sizeof(NormDev), hipMemcpyHostToDevice);
  (void)hipSetDevice(cur);
  PI0X_HIP(e);
  return PI0X_OK;
}

void pi0x_expert_destroy(pi0x_expert* h) {
  if (!h) return;
  (void)hipSetDevice(h->device);
  destroy_impl(h);
  delete h;
}

const char* pi0x_last_error(void) { return g_err.c_str(); }

void pi0x_prefix_config_default(pi0x_config* c) {
  if (!c) return;
  pi0x_config_default(c);
  c->width = 2048;
  c->depth = 18;
  c->mlp_dim = 16384;
  c->num_heads = 8;
  c->num_kv_heads = 1;
  c->head_dim = 256;
  c->max_batch = 1;
  c->max_prefix_len = 1024;
}

size_t pi0x_prefix_weight_count(const pi0x_config* cfg) {
  if (!cfg || cfg->width <= 0 || cfg->depth <= 0 || cfg->mlp_dim <= 0 || cfg->num_heads <= 0 ||
      cfg->num_kv_heads <= 0 || cfg->head_dim <= 0)
    return 0;
  return prefix_weight_count(cfg);
}

pi0x_status pi0x_prefix_create(const pi0x_config* cfg, const void* weights_host, size_t weights_bytes,
                               pi0x_prefix_model** out) {
  if (!out) return fail(PI0X_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  PI0X_TRY(check_prefix_config(cfg));
  if (!weights_host) return fail(PI0X_ERR_INVALID_ARG, "weights_host is NULL");
  const size_t n = prefix_weight_count(cfg);
  if (weights_bytes != n * sizeof(float))
    return fail(PI0X_ERR_SHAPE, "weights_bytes is " + std::to_string(weights_bytes) + ", expected " +
                                    std::to_string(n * sizeof(float)));
  pi0x_prefix_model* p = new (std::nothrow) pi0x_prefix_model();
  if (!p) return fail(PI0X_ERR_OOM, "host allocation failed");
  pi0x_status st = create_prefix_impl(cfg, weights_host, &p->core);
  if (st != PI0X_OK) {
    std::string msg = g_err;
    destroy_impl(&p->core);
    delete p;
    g_err = msg;
    return st;
  }
  *out = p;
  return PI0X_OK;
}

pi0x_status pi0x_prefill(pi0x_prefix_model* p, int32_t batch, int32_t prefix_len, const void* prefix_embeddings,
                         const int32_t* prefix_valid_len, void* prefix_kv_out, hipStream_t stream) {
  if (!p) return fail(PI0X_ERR_INVALID_ARG, "handle is NULL");
  pi0x_expert* h = &p->core;
  if (batch < 1) return fail(PI0X_ERR_INVALID_ARG, "batch must be >= 1");
  if (prefix_len < 0) return fail(PI0X_ERR_INVALID_ARG, "prefix_len must be >= 0");
  if (batch > h->Bmax) return fail(PI0X_ERR_CAPACITY, "batch exceeds max_batch");
  if (prefix_len > h->Lmax) return fail(PI0X_ERR_CAPACITY, "prefix_len exceeds max_prefix_len");
  if (!prefix_embeddings || !prefix_valid_len || !prefix_kv_out)
    return fail(PI0X_ERR_INVALID_ARG, "a device pointer argument is NULL");
  if (reinterpret_cast<uintptr_t>(prefix_kv_out) % 16 != 0)
    return fail(PI0X_ERR_INVALID_ARG, "prefix_kv_out must be 16-byte aligned");
  int dev = -1;
  PI0X_HIP(hipGetDevice(&dev));
  if (dev != h->device) return fail(PI0X_ERR_INVALID_ARG, "the current HIP device is not the handle's device");
  if (prefix_len == 0) return PI0X_OK;
  hipLaunchKernelGGL(set_prefix_desc_kernel, dim3(1), dim3(1), 0, stream, h->desc, prefix_embeddings,
                     prefix_valid_len, prefix_kv_out);
  PI0X_HIP(hipGetLastError());
  return run_prefix(h, batch, prefix_len, stream);
}

void pi0x_prefix_destroy(pi0x_prefix_model* p) {
  if (!p) return;
  destroy_impl(&p->core);
  delete p;
}

pi0x_status pi0x_expert_check_guards(pi0x_expert* h, int32_t* corrupted) {
  if (!h || !corrupted) return fail(PI0X_ERR_INVALID_ARG, "a pointer argument is NULL");
  *corrupted = 0;
  PI0X_HIP(hipDeviceSynchronize());
  std::vector<unsigned char> host(pi0x_expert::kGuardBytes);
  for (unsigned char* g : h->guards) {
    PI0X_HIP(hipMemcpy(host.data(), g, host.size(), hipMemcpyDeviceToHost));
    for (unsigned char b : host)
      if (b != (unsigned char)pi0x_expert::kGuardByte) {
        ++*corrupted;
        break;
      }
  }
  return PI0X_OK;
}

pi0x_status pi0x_prefix_check_guards(pi0x_prefix_model* p, int32_t* corrupted) {
  if (!p) return fail(PI0X_ERR_INVALID_ARG, "handle is NULL");
  return pi0x_expert_check_guards(&p->core, corrupted);
}

pi0x_status pi0x_prefix_set_timing(pi0x_prefix_model* p, int32_t enable) {
  if (!p) return fail(PI0X_ERR_INVALID_ARG, "handle is NULL");
  return pi0x_set_timing(&p->core, enable);
}

pi0x_status pi0x_prefix_read_timing(pi0x_prefix_model* p, double* total_ms, int64_t* launches) {
  if (!p) return fail(PI0X_ERR_INVALID_ARG, "handle is NULL");
  return pi0x_read_timing(&p->core, total_ms, launches);
}

pi0x_status pi0x_set_timing(pi0x_expert* h, int32_t enable) {
  if (!h) return fail(PI0X_ERR_INVALID_ARG, "handle is NULL");
  h->timing = enable != 0;
  return PI0X_OK;
}

pi0x_status pi0x_read_timing(pi0x_expert* h, double* total_ms, int64_t* launches) {
  if (!h || !total_ms || !launches) return fail(PI0X_ERR_INVALID_ARG, "a pointer argument is NULL");
  for (int c = 0; c < PI0X_KERNEL_CLASSES; ++c) {
    total_ms[c] = 0.0;
    launches[c] = 0;
  }
  if (h->ev_used > 0) PI0X_HIP(hipEventSynchronize(h->ev_pool[h->ev_used - 1]));
  for (const auto& m : h->ev_marks) {
    float ms = 0.f;
    PI0X_HIP(hipEventElapsedTime(&ms, h->ev_pool[m.second], h->ev_pool[m.second + 1]));
    total_ms[m.first] += ms;
    launches[m.first] += 1;
  }
  h->ev_marks.clear();
  h->ev_used = 0;
  return PI0X_OK;
}

}  // extern "C"
