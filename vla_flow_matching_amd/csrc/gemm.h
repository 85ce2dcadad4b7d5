// Matrix-core GEMMs C = A * W^T for the expert's projections, with fused
// prologues and epilogues.  A is [M][K] row-major (activations), W is [N][K]
// row-major (nn.Linear layout, so both operands are contiguous along K); C is
// handed element by element (or in pairs, see below) to an epilogue functor.
//
// Three kernels share the epilogues:
//  * gemm_kernel      16x16 tiles, bf16 or fp32 operands (fp32 through eight
//                     v_mfma_f32_16x16x4_f32 per 32-wide K slice): the float32
//                     path and the fallback for any shape.
//  * gemm_tile_kernel bf16, v_mfma_f32_16x16x32_bf16, 128x128 or 128x64
//                     block tiles of 2x2 waves, K slices DMA'd straight into
//                     an LDS ring, XCD-aware tile order: the compute-bound
//                     shapes (more than 64 rows, i.e. batch >= 2).
//  * gemm_wide_kernel  bf16, M <= 64 (batch 1), every projection but the
//                     residual producers: one block per 16-32 columns over the
//                     whole K range, a K chunk's loads in flight at once,
//                     epilogue in the same kernel.
//  * gemm_stream_kernel + gemm_reduce_kernel  bf16, M <= 64, the residual
//                     producers (long K, N = width): split over N and K, the
//                     K-split partials summed by the epilogue kernel.
//
// RMSNorm fusion.  The Gemma norm in front of the q/k/v and gate/up
// projections is y = h / rms(h) * (1 + w); (1 + w) is folded into the weight
// columns at create time, so y W^T = inv_rms(row) * (h W'^T).  Consumers
// ("kRowScale" epilogues) therefore read h itself (its bf16 copy in bf16 mode)
// and scale each output row by inv_rms, which the kernel computes in its
// prologue from per-row partial sums of squares written by the producer of h.
// Producers ("kSsq" epilogues: the residual updates and the suffix embedding)
// return h_new^2 per element; the kernel sums them over each wave's (or
// block's) column group and stores one partial per (row, group).
//
// Split-K.  gemm_kernel (float32 path): the K range is divided over
// gridDim.z; each block writes its partial tile and the last block to arrive
// adds the shares in split order and runs the epilogue (a hand-off through
// device-scope fences, tens of microseconds on this part).  The bf16 tile
// kernel splits K without a hand-off: its blocks store raw partial tiles and
// gemm_reduce_kernel, a second launch, adds them in split order and runs the
// epilogue -- used for the long-K projections whose tiles cannot fill the
// chip on their own.
//
// Paired epilogues: the q/k weight rows of every head and the gate/up rows of
// the MLP are stored interleaved in blocks of 16 (see the runtime's weight
// repack), so stored columns c and c+16 with c % 32 < 16 belong together
// (rotate-half partners, or gate and up of one hidden unit).
#pragma once

#include "common.h"

namespace pi0x {

struct GemmArgs {
  const void* A;
  int lda;
  const void* W;
  int ldw;
  int M, N, K;
  int splits;
  float* partial;        // gemm_kernel with splits > 1: per-tile partial tiles
  unsigned* counters;    // gemm_kernel with splits > 1: per-tile arrival counters, zero between launches
  const float* ssq_in;   // kRowScale: [M][ssq_np] partial sums of squares of A's rows
  int ssq_np;
  int norm_dim;          // number of features the norm averages over
  float norm_eps;
};

// ---------------------------------------------------------------------------
// Epilogues.  Traits: kPaired (pair(row, col, lo, hi, pre), col % 32 < 16, hi
// is column col + 16; else one(row, col, x, pre)), kRowScale (the kernel
// multiplies by inv_rms of the row first), kSsq (one() returns the value
// whose per-group sum the kernel passes to ssq(row, group, sum)).  Rows are
// < M.  Each epilogue splits its global reads into fetch(row, col) -> Pre, so
// the kernels can issue the reads of a group of rows before any of the group's
// stores (the compiler cannot move a read past a store that may alias it).
// The *8 forms do the same for 8 consecutive columns col .. col+7 (col % 8 ==
// 0; for pairs col % 32 < 16 and the partners are col+16 .. col+23), with
// 16-byte loads and stores.
// ---------------------------------------------------------------------------
struct NoPre {};
struct Pre8f {
  float v[8];
};

// out[row][col] = act(x + bias[col]) in TO; act = SiLU when silu != 0.
template <typename TO>
struct EpiStore {
  static constexpr bool kPaired = false, kRowScale = false, kSsq = false;
  using Pre = float;
  TO* out;
  int ldo;
  const float* bias;  // may be null
  int silu;
  __device__ __forceinline__ Pre fetch(int, int col) const { return bias ? bias[col] : 0.f; }
  __device__ __forceinline__ float one(int row, int col, float x, Pre b) const {
    float v = x + b;
    if (silu) v = pi0x::silu(v);
    out[(size_t)row * ldo + col] = from_f32<TO>(v);
    return 0.f;
  }
  using Pre8 = Pre8f;
  __device__ __forceinline__ Pre8 fetch8(int, int col) const {
    Pre8 b;
    if (bias) load8f(bias + col, b.v);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) b.v[e] = 0.f;
    return b;
  }
  __device__ __forceinline__ float one8(int row, int col, const float* x, const Pre8& b) const {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = x[e] + b.v[e];
      if (silu) v[e] = pi0x::silu(v[e]);
    }
    store8(out + (size_t)row * ldo + col, v);
    return 0.f;
  }
  __device__ __forceinline__ void ssq(int, int, float) const {}
};

// Action rows of the suffix embedding: GEMM row r = b*H + i goes to hidden row
// b*S + 1 + i (row 0 of each sample is the state token); writes h, its bf16
// copy hb (bf16 mode) and the rows' sum-of-squares partials.
template <typename TB>
struct EpiSuffixRows {
  static constexpr bool kPaired = false, kRowScale = false, kSsq = true;
  using Pre = float;
  float* h;
  TB* hb;  // null in float32 mode
  int ldh, H, S;
  const float* bias;
  float* ssq_out;
  int np;
  __device__ __forceinline__ int hrow(int row) const { return (row / H) * S + 1 + row % H; }
  __device__ __forceinline__ Pre fetch(int, int col) const { return bias[col]; }
  __device__ __forceinline__ float one(int row, int col, float x, Pre b) const {
    const size_t i = (size_t)hrow(row) * ldh + col;
    const float v = x + b;
    h[i] = v;
    if (hb) hb[i] = from_f32<TB>(v);
    return v * v;
  }
  using Pre8 = Pre8f;
  __device__ __forceinline__ Pre8 fetch8(int, int col) const {
    Pre8 b;
    load8f(bias + col, b.v);
    return b;
  }
  __device__ __forceinline__ float one8(int row, int col, const float* x, const Pre8& b) const {
    const size_t i = (size_t)hrow(row) * ldh + col;
    float v[8], ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = x[e] + b.v[e];
      ss += v[e] * v[e];
    }
    store8(h + i, v);
    if (hb) store8(hb + i, v);
    return ss;
  }
  __device__ __forceinline__ void ssq(int row, int group, float s) const { ssq_out[(size_t)hrow(row) * np + group] = s; }
};

// Residual update h[row][col] += x (float32 residual stream), its bf16 copy
// and the rows' sum-of-squares partials for the next norm.
template <typename TB>
struct EpiResidual {
  static constexpr bool kPaired = false, kRowScale = false, kSsq = true;
  using Pre = float;
  float* h;
  TB* hb;  // null in float32 mode
  int ldh;
  float* ssq_out;
  int np;
  __device__ __forceinline__ Pre fetch(int row, int col) const { return h[(size_t)row * ldh + col]; }
  __device__ __forceinline__ float one(int row, int col, float x, Pre old) const {
    const size_t i = (size_t)row * ldh + col;
    const float v = old + x;
    h[i] = v;
    if (hb) hb[i] = from_f32<TB>(v);
    return v * v;
  }
  using Pre8 = Pre8f;
  __device__ __forceinline__ Pre8 fetch8(int row, int col) const {
    Pre8 o;
    load8f(h + (size_t)row * ldh + col, o.v);
    return o;
  }
  __device__ __forceinline__ float one8(int row, int col, const float* x, const Pre8& old) const {
    const size_t i = (size_t)row * ldh + col;
    float v[8], ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = old.v[e] + x[e];
      ss += v[e] * v[e];
    }
    store8(h + i, v);
    if (hb) store8(hb + i, v);
    return ss;
  }
  __device__ __forceinline__ void ssq(int row, int group, float s) const { ssq_out[(size_t)row * np + group] = s; }
};

// Fused q/k/v projection epilogue (after the inv_rms row scale): rotate-half
// RoPE on every q head and the k head at position valid_len[b] + s for suffix
// token s of sample b; the (cos, sin) pairs of every suffix row are tabulated
// once per call in cs[row][head_dim/2].  q and k go to out[row][q heads | k] in
// the natural layout; the values go transposed to vt[b][d][vt_ld] (column
// vt_pos(s)), the layout attention reads them in.
// Prefix pass (desc != nullptr; page 1, _compute_layer_prefix_only returns the
// post-RoPE k and v for the cache): S is the padded prefix length, the rotated
// k head and the values are also stored to the cache desc->kv_out at element
// offsets k_off / v_off ([B][S][head_dim] blocks, so cache row = GEMM row),
// and the transposed values of padded rows (s >= valid_len[b]) are zero, so
// that a masked key's value is exactly zero when attention weighs it by 0.
template <typename T>
struct EpiQkvRope {
  static constexpr bool kPaired = true, kRowScale = true, kSsq = false;
  using Pre = float2;  // (cos, sin) of the pair's angle
  T* out;
  int ldo;
  int qk_cols;  // (num_heads + 1) * head_dim
  int head_dim, S;
  const float2* cs;
  T* vt;
  int vt_ld;
  const CallDesc* desc = nullptr;  // prefix pass only
  size_t k_off = 0, v_off = 0;
  __device__ __forceinline__ int jj(int c) const {
    const int w = c % head_dim;
    return (w >> 5) * 16 + (w & 15);
  }
  __device__ __forceinline__ bool is_k(int c) const { return desc != nullptr && c >= qk_cols - head_dim; }
  __device__ __forceinline__ bool pad_row(int b, int s) const {
    if (desc == nullptr) return false;
    int v = desc->valid[b];
    v = v < 0 ? 0 : (v > S ? S : v);
    return s >= v;
  }
  __device__ __forceinline__ Pre fetch(int row, int c) const {
    if (c >= qk_cols) return float2{0.f, 0.f};
    return cs[(size_t)row * (head_dim >> 1) + jj(c)];
  }
  __device__ __forceinline__ void pair(int row, int c, float x1, float x2, Pre cs_) const {
    if (c < qk_cols) {
      const int half = head_dim >> 1;
      T* o = out + (size_t)row * ldo + (c / head_dim) * head_dim + jj(c);
      const T r1 = from_f32<T>(x1 * cs_.x - x2 * cs_.y), r2 = from_f32<T>(x2 * cs_.x + x1 * cs_.y);
      o[0] = r1;
      o[half] = r2;
      if (is_k(c)) {
        T* kc = reinterpret_cast<T*>(desc->kv_out) + k_off + (size_t)row * head_dim + jj(c);
        kc[0] = r1;
        kc[half] = r2;
      }
    } else {
      const int b = row / S, s = row - b * S, d = c - qk_cols;
      const bool pad = pad_row(b, s);
      T* o = vt + ((size_t)b * head_dim + d) * vt_ld + vt_pos(s);
      o[0] = from_f32<T>(pad ? 0.f : x1);
      o[(size_t)16 * vt_ld] = from_f32<T>(pad ? 0.f : x2);
      if (desc != nullptr) {
        T* vc = reinterpret_cast<T*>(desc->kv_out) + v_off + (size_t)row * head_dim + d;
        vc[0] = from_f32<T>(x1);
        vc[16] = from_f32<T>(x2);
      }
    }
  }
  struct Pre8 {
    float2 cs[8];
  };
  __device__ __forceinline__ Pre8 fetch8(int row, int c) const {
    Pre8 p;
    if (c < qk_cols) {
      const float4* src = reinterpret_cast<const float4*>(cs + (size_t)row * (head_dim >> 1) + jj(c));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 t = src[e];
        p.cs[2 * e] = float2{t.x, t.y};
        p.cs[2 * e + 1] = float2{t.z, t.w};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) p.cs[e] = float2{0.f, 0.f};
    }
    return p;
  }
  __device__ __forceinline__ void pair8(int row, int c, const float* x1, const float* x2, const Pre8& p) const {
    if (c < qk_cols) {
      const int half = head_dim >> 1;
      T* o = out + (size_t)row * ldo + (c / head_dim) * head_dim + jj(c);
      float r1[8], r2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        r1[e] = x1[e] * p.cs[e].x - x2[e] * p.cs[e].y;
        r2[e] = x2[e] * p.cs[e].x + x1[e] * p.cs[e].y;
      }
      store8(o, r1);
      if (is_k(c)) {
        T* kc = reinterpret_cast<T*>(desc->kv_out) + k_off + (size_t)row * head_dim + jj(c);
        store8(kc, r1);
        store8(kc + half, r2);
      }
      store8(o + half, r2);
    } else {
      const int b = row / S, s = row - b * S, d = c - qk_cols;
      const bool pad = pad_row(b, s);
      T* o = vt + ((size_t)b * head_dim + d) * vt_ld + vt_pos(s);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[(size_t)e * vt_ld] = from_f32<T>(pad ? 0.f : x1[e]);
        o[(size_t)(16 + e) * vt_ld] = from_f32<T>(pad ? 0.f : x2[e]);
      }
      if (desc != nullptr) {
        T* vc = reinterpret_cast<T*>(desc->kv_out) + v_off + (size_t)row * head_dim + d;
        store8(vc, x1);
        store8(vc + 16, x2);
      }
    }
  }
};

// GeGLU epilogue (after the inv_rms row scale): stored column c (gate of hidden
// unit (c/32)*16 + c%16) and c + 16 (its up): out[row][unit] = gelu_tanh(gate) * up.
template <typename T>
struct EpiGeglu {
  static constexpr bool kPaired = true, kRowScale = true, kSsq = false;
  using Pre = NoPre;
  T* out;
  int ldo;
  __device__ __forceinline__ Pre fetch(int, int) const { return NoPre{}; }
  __device__ __forceinline__ void pair(int row, int c, float g, float u, Pre) const {
    out[(size_t)row * ldo + (c >> 5) * 16 + (c & 15)] = from_f32<T>(gelu_tanh_fast<T>(g) * u);
  }
  using Pre8 = NoPre;
  __device__ __forceinline__ Pre8 fetch8(int, int) const { return NoPre{}; }
  __device__ __forceinline__ void pair8(int row, int c, const float* g, const float* u, const Pre8&) const {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = gelu_tanh_fast<T>(g[e]) * u[e];
    store8(out + (size_t)row * ldo + (c >> 5) * 16 + (c & 15), v);
  }
};

// Velocity projection and Euler update (page 1, the end of denoise_step and
// the update of sample_actions), after the inv_rms row scale of the final
// norm: GEMM row r is hidden row r of the suffix, column c < A an action
// feature.  The state rows (r % S == 0) and padding columns are dropped.
// v = acc + b_out[c]; mode 0: x <- x + dt v (x from desc->x_in on the first
// step, else x_loop; written to x_loop and, on the last step, to desc->out
// after the action unnormalization, page 1 _apply_norm inverse, when set);
// mode 1: v is written to desc->out.  Loop variants of page 3 (Wall-X,
// generate_flow_action), mode 0 only: xpred takes the head output as the
// predicted clean action, v = acc + b_out - noise (desc->x_in, the initial
// noise); blend (set on the first step only) mixes in the padding action,
// v = (p - x)(1 - m) + v m with m = desc->dof_mask, p = desc->padding.
// Each output element is owned by one thread, which reads desc->x_in[i]
// before it writes desc->out[i], so out may alias the noise.
struct EpiEuler {
  static constexpr bool kPaired = false, kRowScale = true, kSsq = false;
  using Pre = float;  // the current x
  float* x_loop;
  const CallDesc* desc;
  const float* b_out;
  int H, S, A;
  int from_input, write_out, mode;
  float dt;
  const NormDev* norm;  // action unnormalization of the returned chunk (write_out)
  int xpred, blend;
  __device__ __forceinline__ int idx(int row, int col) const {
    const int b = row / S, s = row - b * S;
    return (s == 0 || col >= A) ? -1 : (b * H + s - 1) * A + col;
  }
  __device__ __forceinline__ Pre fetch(int row, int col) const {
    const int i = idx(row, col);
    if (i < 0 || mode == 1) return 0.f;
    return (from_input ? desc->x_in : x_loop)[i];
  }
  __device__ __forceinline__ float one(int row, int col, float acc, Pre x) const {
    const int i = idx(row, col);
    if (i < 0) return 0.f;
    float v = acc + b_out[col];
    if (mode == 1) {
      desc->out[i] = v;
    } else {
      if (xpred) v -= desc->x_in[i];
      if (blend) {
        const float m = desc->dof_mask[i];
        v = (desc->padding[i] - x) * (1.0f - m) + v * m;
      }
      const float xn = x + dt * v;
      x_loop[i] = xn;
      if (write_out) desc->out[i] = unnorm_action(norm, col, xn);
    }
    return 0.f;
  }
  using Pre8 = Pre8f;
  __device__ __forceinline__ Pre8 fetch8(int row, int col) const {
    Pre8 p;
#pragma unroll
    for (int e = 0; e < 8; ++e) p.v[e] = fetch(row, col + e);
    return p;
  }
  __device__ __forceinline__ float one8(int row, int col, const float* acc, const Pre8& p) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) one(row, col + e, acc[e], p.v[e]);
    return 0.f;
  }
  __device__ __forceinline__ void ssq(int, int, float) const {}
};

// inv_rms of row m0 + t from its partial sums of squares (16-byte loads,
// eight in flight, when the partial count is a multiple of 4).
__device__ __forceinline__ float row_inv_rms(const GemmArgs& g, int m0, int t) {
  float s = 0.f;
  if (m0 + t < g.M) {
    const float* p = g.ssq_in + (size_t)(m0 + t) * g.ssq_np;
    if (g.ssq_np % 4 == 0) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int i = 0; i < g.ssq_np; i += 4) acc += *reinterpret_cast<const f32x4*>(p + i);
      s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    } else {
      for (int i = 0; i < g.ssq_np; ++i) s += p[i];
    }
  }
  return 1.0f / sqrtf(s / (float)g.norm_dim + g.norm_eps);
}

// inv_rms of rows m0 .. m0+n-1 into s_inv (threads < n): the same arithmetic
// as row_inv_rms, written to LDS.
__device__ __forceinline__ void row_scale_prologue(const GemmArgs& g, int m0, int n, float* s_inv) {
  const int t = threadIdx.x;
  if (t < n) {
    float s = 0.f;
    if (m0 + t < g.M) {
      const float* p = g.ssq_in + (size_t)(m0 + t) * g.ssq_np;
      if (g.ssq_np % 4 == 0) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int i = 0; i < g.ssq_np; i += 4) acc += *reinterpret_cast<const f32x4*>(p + i);
        s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      } else {
        for (int i = 0; i < g.ssq_np; ++i) s += p[i];
      }
    }
    s_inv[t] = 1.0f / sqrtf(s / (float)g.norm_dim + g.norm_eps);
  }
}

// ---------------------------------------------------------------------------
// gemm_kernel: 16x16 output tiles (both dtypes)
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g, Epi epi) {
  constexpr int BK = 32;
  constexpr int VE = 16 / (int)sizeof(T);  // elements per 16-byte vector
  constexpr int LDK = BK + VE;             // padded LDS row
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int VPR = BK / VE;             // vectors per row of a K slice
  constexpr int AV = BM * VPR, BV = BN * VPR;
  constexpr int AVT = (AV + 255) / 256, BVT = (BV + 255) / 256;
  static_assert(WM * WN == 4, "4 waves per block");
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  static_assert(!Epi::kPaired || TN % 2 == 0, "paired epilogues need column tiles in pairs");

  __shared__ __attribute__((aligned(16))) T As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * LDK];
  __shared__ float s_inv[BM];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int n_tile = blockIdx.x, m_tile = blockIdx.y, split = blockIdx.z;
  const int m0 = m_tile * BM, n0 = n_tile * BN;
  const int KI = g.K / BK;
  const int kb = (int)((long)split * KI / g.splits), ke = (int)((long)(split + 1) * KI / g.splits);
  const T* __restrict__ A = reinterpret_cast<const T*>(g.A);
  const T* __restrict__ W = reinterpret_cast<const T*>(g.W);

  u32x4 ra[AVT], rb[BVT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < AVT; ++i) {
      int v = tid + i * 256;
      if (v < AV) {
        int row = v / VPR, kc = (v % VPR) * VE, grow = m0 + row;
        ra[i] = grow < g.M ? *reinterpret_cast<const u32x4*>(A + (size_t)grow * g.lda + kt * BK + kc)
                           : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < BVT; ++i) {
      int v = tid + i * 256;
      if (v < BV) {
        int row = v / VPR, kc = (v % VPR) * VE, grow = n0 + row;
        rb[i] = grow < g.N ? *reinterpret_cast<const u32x4*>(W + (size_t)grow * g.ldw + kt * BK + kc)
                           : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < AVT; ++i) {
      int v = tid + i * 256;
      if (v < AV) *reinterpret_cast<u32x4*>(&As[st][(v / VPR) * LDK + (v % VPR) * VE]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BVT; ++i) {
      int v = tid + i * 256;
      if (v < BV) *reinterpret_cast<u32x4*>(&Bs[st][(v / VPR) * LDK + (v % VPR) * VE]) = rb[i];
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (Epi::kRowScale) row_scale_prologue(g, m0, BM, s_inv);
  if (kb < ke) {
    gload(kb);
    sstore(0);
  }
  __syncthreads();
  int st = 0;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int kt = kb; kt < ke; ++kt) {
    if (kt + 1 < ke) gload(kt + 1);
    Frag<T> af[TM], bfr[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) load8(af[i], &As[st][((wm * TM + i) * 16 + fr) * LDK + fk]);
#pragma unroll
    for (int j = 0; j < TN; ++j) load8(bfr[j], &Bs[st][((wn * TN + j) * 16 + fr) * LDK + fk]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) mma32(af[i], bfr[j], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < ke) sstore(st ^ 1);
    __syncthreads();
    st ^= 1;
  }

  if (g.splits > 1) {
    constexpr int NR = TM * TN * 4;
    const int tile = m_tile * gridDim.x + n_tile;
    float* P = g.partial + (size_t)tile * g.splits * NR * 256;
    float* mine = P + (size_t)split * NR * 256;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) mine[((i * TN + j) * 4 + e) * 256 + tid] = acc[i][j][e];
    // hand-off: every thread makes its own partial stores visible at device
    // scope before the barrier, then one thread publishes the arrival
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      s_last = atomicAdd(&g.counters[tile], 1u) == (unsigned)g.splits - 1u;
      __threadfence();
    }
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float s = 0.f;
          for (int z = 0; z < g.splits; ++z)
            s += __hip_atomic_load(&P[((size_t)z * NR + (i * TN + j) * 4 + e) * 256 + tid], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          acc[i][j][e] = s;
        }
    if (tid == 0) g.counters[tile] = 0u;
  }

  // element (i, j, e) of the wave is C[mb + 16 i + 4 (lane/16) + e][nb + 16 j + lane % 16]
  const int mb = m0 + wm * TM * 16, nb = n0 + wn * TN * 16;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    constexpr int NJ = Epi::kPaired ? TN / 2 : TN;
    typename Epi::Pre pre[4][NJ];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = min(mb + i * 16 + (lane >> 4) * 4 + e, g.M - 1);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        pre[e][j] = epi.fetch(row, nb + (Epi::kPaired ? 2 * j : j) * 16 + (lane & 15));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = mb + i * 16 + (lane >> 4) * 4 + e;
      const bool ok = row < g.M;
      float sc = 1.f;
      if constexpr (Epi::kRowScale) sc = s_inv[min(row, g.M - 1) - m0];
      if constexpr (Epi::kPaired) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          if (ok) epi.pair(row, nb + 2 * j * 16 + (lane & 15), sc * acc[i][2 * j][e], sc * acc[i][2 * j + 1][e], pre[e][j]);
      } else {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          if (ok) ss += epi.one(row, nb + j * 16 + (lane & 15), sc * acc[i][j][e], pre[e][j]);
        if constexpr (Epi::kSsq) {
          // the 16 lanes sharing lane/16 hold this row's TN*16 columns
          ss += __shfl_xor(ss, 1, 64);
          ss += __shfl_xor(ss, 2, 64);
          ss += __shfl_xor(ss, 4, 64);
          ss += __shfl_xor(ss, 8, 64);
          if (ok && (lane & 15) == 0) epi.ssq(row, nb / (TN * 16), ss);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// gemm_tile_kernel: bf16, 16x16x32 MFMA, NWM x NWN waves of (BM/NWM) x (BN/NWN)
// (4x4 tiles per wave at 128x128: sixteen independent accumulator chains),
// K slices of BK moved straight from global memory into an LDS ring of ST
// stages (global_load_lds_dwordx4, no register staging), so the loads of the
// next ST-1 slices are in flight while a slice feeds the matrix cores.  LDS
// rows are BK bf16 with the 16-byte chunks of row r stored at position
// chunk ^ ((r / RPS) % CPR) (CPR chunks per row, RPS rows per 256 bytes): the
// 16 rows one fragment read serves at a time then cover all 64 banks once,
// with no padding (the DMA writes 64 consecutive 16-byte slots per wave).
// One barrier per slice: a wave waits for its own loads of slice k, the
// barrier makes everyone's visible, and only then is slice k+ST-1 issued into
// the buffer slice k-1 used.
//
// Tile order: the blocks are dealt round-robin to the 8 XCDs (block L runs on
// XCD L % 8), so block L takes tile t = (L % 8) * ceil(T/8) + L / 8 -- each XCD
// owns a contiguous run of tiles -- and tiles run in groups of group_m row
// tiles by all column tiles, so the blocks resident on one XCD share their A
// row panels and W column panels in that XCD's L2.
//
// K split (g.splits > 1, for grids with fewer tiles than CUs): unit u of the
// T * splits units is K range u % splits of tile u / splits, and the block
// stores its raw float32 tile to g.partial[split][row][col]; gemm_reduce_kernel
// then adds the splits in order and runs the epilogue.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int ST, int NWM = 2, int NWN = 2>
constexpr size_t tile_smem_bytes() {
  // the ring, or the epilogue strips of the waves (32 rows x (BN/NWN + 4) floats each), whichever is larger
  return (size_t)ST * (BM + BN) * BK * 2 > (size_t)NWM * NWN * 32 * (BN / NWN + 4) * 4
             ? (size_t)ST * (BM + BN) * BK * 2
             : (size_t)NWM * NWN * 32 * (BN / NWN + 4) * 4;
}

// Waits until at most `ahead` ring stages of PER loads each are outstanding.
template <int PER, int ST>
__device__ __forceinline__ void wait_stages(int ahead) {
  static_assert(ST >= 2 && ST <= 4, "ring depth");
  if (ST >= 4 && ahead >= 2) wait_vmcnt<(ST >= 4 ? 2 * PER : 0)>();
  else if (ST >= 3 && ahead >= 1) wait_vmcnt<(ST >= 3 ? PER : 0)>();
  else wait_vmcnt<0>();
}

// Waves per SIMD that the kernel's LDS allows at once (its blocks of NWM * NWN
// waves, up to 160 KiB of LDS per CU).  Given to the compiler as the
// occupancy to allocate registers for: without it the compiler plans for
// more waves than can ever be resident, keeps the accumulators in the
// accumulation registers and copies them out for the epilogue; with it they
// stay in vector registers (batch-64 call 36.69 -> 36.49 ms on one box).
template <int BM, int BN, int BK, int ST, int NWM, int NWN>
constexpr int tile_waves_per_simd() {
  const int blocks = (int)((160 * 1024) / (tile_smem_bytes<BM, BN, BK, ST, NWM, NWN>() + 1024));
  const int w = blocks * NWM * NWN / 4;
  return w < 1 ? 1 : (w > 8 ? 8 : w);
}

// A ring of exactly 80 KiB (the 64x256 tiles of two stages) lets two blocks
// share a CU only with no static LDS beside it: such a kernel keeps each
// row's inverse RMS in a register through the main loop and stages it in the
// last bytes of the ring for the epilogue.
template <int BM, int BN, int BK, int ST, int NWM, int NWN>
constexpr bool tile_ring_staged() {
  return tile_smem_bytes<BM, BN, BK, ST, NWM, NWN>() == 80 * 1024;
}
template <int BM, int BN, int BK, int ST, int NWM, int NWN>
constexpr int tile_waves_per_simd_hint() {
  if constexpr (tile_ring_staged<BM, BN, BK, ST, NWM, NWN>()) return 2 * NWM * NWN / 4;
  else return tile_waves_per_simd<BM, BN, BK, ST, NWM, NWN>();
}

template <int BM, int BN, int BK, int ST, int NWM, int NWN, class Epi>
__global__ __launch_bounds__(NWM * NWN * 64) __attribute__((amdgpu_waves_per_eu(
    tile_waves_per_simd_hint<BM, BN, BK, ST, NWM, NWN>(), tile_waves_per_simd_hint<BM, BN, BK, ST, NWM, NWN>()))) void
gemm_tile_kernel(GemmArgs g, Epi epi, int tiles_m, int tiles_n, int group_m) {
  constexpr int NT = NWM * NWN * 64;
  constexpr int TM = BM / NWM / 16, TN = BN / NWN / 16;  // 16x16 MFMA tiles per wave
  constexpr int CPR = BK / 8, RPS = 256 / (BK * 2);  // 16-byte chunks per row, rows per 256 bytes
  constexpr int STAGE = (BM + BN) * BK;               // bf16 elements per ring stage
  constexpr int AJ = BM * CPR / NT, BJ = BN * CPR / NT;  // DMA chunks per thread per stage
  constexpr int ELD = TN * 16 + 4;                    // epilogue staging row (floats, 16-byte aligned)
  static_assert(BK == 32 || BK == 64, "slice width");
  static_assert(AJ >= 1 && BJ >= 1 && BM * CPR % NT == 0 && BN * CPR % NT == 0, "tile/thread mismatch");
  static_assert(TM % 2 == 0 && TN >= 1, "wave tile: 32-row strips of 16x16 tiles");
  static_assert((size_t)(NT / 64) * 32 * ELD * 4 <= tile_smem_bytes<BM, BN, BK, ST, NWM, NWN>(), "epilogue staging must fit");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16* ring = reinterpret_cast<bf16*>(smem_raw);
  constexpr bool STAGED = tile_ring_staged<BM, BN, BK, ST, NWM, NWN>();
  static_assert(!STAGED || (size_t)(NT / 64) * 32 * ELD * 4 + BM * 4 <= tile_smem_bytes<BM, BN, BK, ST, NWM, NWN>(),
                "staged inverse RMS must clear the epilogue strips");
  float* s_inv;
  if constexpr (STAGED) {
    s_inv = reinterpret_cast<float*>(smem_raw + tile_smem_bytes<BM, BN, BK, ST, NWM, NWN>() - BM * 4);
  } else {
    __shared__ float s_inv_static[BM];
    s_inv = s_inv_static;
  }
  float inv_reg = 0.f;  // STAGED: this thread's row (tid < BM) until the epilogue

  // tile (and K range) of this block
  const int S = g.splits;
  const int T = tiles_m * tiles_n, U = T * S, per_xcd = (U + 7) / 8;
  const int u = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (u >= U) return;
  const int t = u / S, split = u - t * S;
  const int gsize = group_m * tiles_n, grp = t / gsize, first_m = grp * group_m;
  const int gm = min(tiles_m - first_m, group_m), within = t - grp * gsize;
  const int m_tile = first_m + within % gm, n_tile = within / gm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int m0 = m_tile * BM, n0 = n_tile * BN;
  const int KI = g.K / BK / S, kbase = split * KI * BK;  // this block's K slices
  const bf16* __restrict__ A = reinterpret_cast<const bf16*>(g.A);
  const bf16* __restrict__ W = reinterpret_cast<const bf16*>(g.W);

  // DMA sources: slot (wave*J + j)*64 + lane of a stage holds row slot / CPR,
  // chunk (slot % CPR) ^ swizzle(row); rows past M repeat row M-1 (never stored)
  const bf16* asrc[AJ];
#pragma unroll
  for (int j = 0; j < AJ; ++j) {
    const int slot = (wave * AJ + j) * 64 + lane, row = slot / CPR, c = (slot % CPR) ^ ((row / RPS) % CPR);
    asrc[j] = A + (size_t)min(m0 + row, g.M - 1) * g.lda + kbase + c * 8;
  }
  const bf16* bsrc[BJ];
#pragma unroll
  for (int j = 0; j < BJ; ++j) {
    const int slot = (wave * BJ + j) * 64 + lane, row = slot / CPR, c = (slot % CPR) ^ ((row / RPS) % CPR);
    bsrc[j] = W + (size_t)(n0 + row) * g.ldw + kbase + c * 8;
  }
  auto issue = [&](int kt) {
    bf16* sa = ring + (kt % ST) * STAGE;
    bf16* sb = sa + BM * BK;
    const int ko = kt * BK;
#pragma unroll
    for (int j = 0; j < AJ; ++j) lds_dma16(asrc[j] + ko, sa + (wave * AJ + j) * 512);
#pragma unroll
    for (int j = 0; j < BJ; ++j) lds_dma16(bsrc[j] + ko, sb + (wave * BJ + j) * 512);
  };

  // the first slices go out before anything waits on memory
#pragma unroll
  for (int p = 0; p < ST - 1; ++p)
    if (p < KI) issue(p);
  if constexpr (Epi::kRowScale) {
    if constexpr (STAGED) {
      if (tid < BM) inv_reg = row_inv_rms(g, m0, tid);
    } else {
      row_scale_prologue(g, m0, BM, s_inv);
    }
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // fragment rows: lane % 16 of each 16-row MFMA tile (tile bases are multiples of 16),
  // K chunk 4*kk + lane/16 of the slice
  const int fr = lane & 15, fq = lane >> 4, sw = (fr / RPS) % CPR;
  for (int kt = 0; kt < KI; ++kt) {
    wait_stages<AJ + BJ, ST>(min(ST - 2, KI - 1 - kt));  // later slices may stay in flight
    ring_barrier();
    if (kt + ST - 1 < KI) issue(kt + ST - 1);
    const bf16* sa = ring + (kt % ST) * STAGE + (wm * TM * 16 + fr) * BK;
    const bf16* sb = ring + (kt % ST) * STAGE + BM * BK + (wn * TN * 16 + fr) * BK;
    // The fragments of the slice's first 32-wide K step are read, then the
    // second step's reads go out while the first step's MFMAs run.  (The
    // compiler counts the LDS DMA in flight against the LDS counter, so
    // before the first MFMA it waits for every LDS read issued so far; the
    // second step's reads therefore follow that wait.  With all 16 reads
    // ahead of the MFMAs, each slice waited for all of them.)  The
    // scheduling barriers keep this order against the compiler's habit of
    // sinking each read next to its MFMA.
    bf16x8 af[BK / 32][TM], bfr[BK / 32][TN];
    auto read_step = [&](int kk) {
      const int pos = ((kk * 4 + fq) ^ sw) * 8;
#pragma unroll
      for (int i = 0; i < TM; ++i) af[kk][i] = *reinterpret_cast<const bf16x8*>(sa + i * 16 * BK + pos);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[kk][j] = *reinterpret_cast<const bf16x8*>(sb + j * 16 * BK + pos);
    };
    read_step(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      if (kk + 1 < BK / 32) read_step(kk + 1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kk][i], bfr[kk][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // every wave is done reading the ring before it is reused for the epilogue
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (STAGED && Epi::kRowScale) {
    if (tid < BM) s_inv[tid] = inv_reg;
    __syncthreads();
  }

  // Epilogue through LDS, one 32-row strip (two 16-row MFMA tiles) of the wave
  // tile at a time: the strip is written in the MFMA layout (element e of tile
  // (ii, j) is row 16 ii + 4 (lane/16) + e, column 16 j + lane % 16) and read
  // back as 8 consecutive columns of one row per lane, so every global access
  // of the epilogue is 16 bytes or more.  Non-paired: CH = WC/8 lanes per row;
  // paired: one lane takes columns c .. c+7 and their partners c+16 .. c+23.
  // All fetches of the strip are issued before its stores.  Residual
  // producers sum h^2 over the CH lanes of a row.  Each wave owns its strip, so
  // only wave-level ordering is needed between the strip's LDS writes and
  // reads: no block barrier, which would also wait for the strip's global
  // stores to complete.
  float* strip = reinterpret_cast<float*>(smem_raw) + wave * 32 * ELD;
  const int mb = m0 + wm * TM * 16, nb = n0 + wn * TN * 16;
  constexpr int WC = TN * 16;                        // wave tile width
  constexpr int CH = Epi::kPaired ? WC / 16 : WC / 8;  // lanes per row
  constexpr int RPP = 64 / CH;                       // rows per pass
  constexpr int NPASS = 32 / RPP;                    // passes per strip
  static_assert(WC % 32 == 0 && 64 % CH == 0 && 32 % RPP == 0, "epilogue lane layout");
  const int rin = lane / CH, q = lane % CH;
  const int c = Epi::kPaired ? (q >> 1) * 32 + (q & 1) * 8 : q * 8;  // first column of this lane's chunk
#pragma unroll
  for (int i = 0; i < TM / 2; ++i) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          strip[(ii * 16 + (lane >> 4) * 4 + e) * ELD + j * 16 + (lane & 15)] = acc[2 * i + ii][j][e];
    wave_lds_fence();
    if (S > 1) {
      // K split: the raw partial (row scale and epilogue come after the sum)
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        const int row = mb + i * 32 + p * RPP + rin;
        if (row >= g.M) continue;
        float* dst = g.partial + ((size_t)split * g.M + row) * g.N + nb + c;
        float v[8];
        load8f(strip + (p * RPP + rin) * ELD + c, v);
        store8(dst, v);
        if constexpr (Epi::kPaired) {
          load8f(strip + (p * RPP + rin) * ELD + c + 16, v);
          store8(dst + 16, v);
        }
      }
      wave_lds_fence();
      continue;
    }
    typename Epi::Pre8 pre[NPASS];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int row = min(mb + i * 32 + p * RPP + rin, g.M - 1);
      pre[p] = epi.fetch8(row, nb + c);
    }
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int r = p * RPP + rin;
      const int row = mb + i * 32 + r;
      const bool ok = row < g.M;
      const float sc = Epi::kRowScale ? s_inv[min(row, g.M - 1) - m0] : 1.f;
      float lo[8];
      load8f(strip + r * ELD + c, lo);
#pragma unroll
      for (int e = 0; e < 8; ++e) lo[e] *= sc;
      if constexpr (Epi::kPaired) {
        float hi[8];
        load8f(strip + r * ELD + c + 16, hi);
#pragma unroll
        for (int e = 0; e < 8; ++e) hi[e] *= sc;
        if (ok) epi.pair8(row, nb + c, lo, hi, pre[p]);
      } else {
        float ss = ok ? epi.one8(row, nb + c, lo, pre[p]) : 0.f;
        if constexpr (Epi::kSsq) {
#pragma unroll
          for (int off = 1; off < CH; off <<= 1) ss += __shfl_xor(ss, off, 64);
          if (ok && q == 0) epi.ssq(row, nb / WC, ss);
        }
      }
    }
    wave_lds_fence();
  }
}

// ---------------------------------------------------------------------------
// gemm_wide_kernel: bf16, M <= 64 rows (batch 1), BN = 16*TN output columns
// per block and the whole K range, split evenly over NW waves.  A wave takes
// its K share in chunks of up to 256: it issues all loads of a chunk at once
// -- its weight rows and its slice of the 64 activation rows (rows past M
// repeat row M-1; their results are never stored) -- then runs the chunk's
// MFMAs, so a chunk costs one memory round trip.  The waves' tiles are summed
// through LDS and the epilogue runs in the same kernel: no K-split partials
// and no second launch.  Every block reads the whole activation slice, so the
// runtime keeps the long-K residual producers on the stream kernels; with
// kSsq the kernel writes one sum-of-squares partial per (row, block), i.e.
// per BN columns.
// ---------------------------------------------------------------------------
template <int NW, int TN, class Epi>
__global__ __launch_bounds__(NW * 64) void gemm_wide_kernel(GemmArgs g, Epi epi) {
  constexpr int NT = NW * 64, BN = TN * 16, LDR = BN + 1;
  constexpr int TPR = NT / 64;      // epilogue threads per row
  constexpr int CPT = BN / TPR;     // columns per thread in the epilogue
  constexpr int KW = 256, NP = KW / 64;  // K chunk of a wave, in 64-wide steps
  static_assert(!Epi::kPaired || (BN >= 32 && CPT % 2 == 0), "paired epilogues need 32-column groups");
  static_assert(CPT >= 1 && (TPR & (TPR - 1)) == 0, "epilogue threads per row");
  __shared__ float red[NW][64 * LDR];
  __shared__ float s_inv[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * BN;
  const int kw = g.K / NW, kb = wave * kw;  // this wave's K range [kb, kb + kw), kw % 64 == 0
  const bf16* __restrict__ A = reinterpret_cast<const bf16*>(g.A);
  const bf16* __restrict__ W = reinterpret_cast<const bf16*>(g.W);

  if constexpr (Epi::kRowScale) row_scale_prologue(g, 0, 64, s_inv);

  // lane (r, q) = (l % 16, l / 16): row/column r of each 16-tile, elements 16q .. 16q+15 of each
  // 64-wide step (two MFMA steps of 8)
  const int fr = lane & 15, fk = (lane >> 4) * 16;
  f32x4 acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < kw; kc += KW) {
    u32x4 wv[TN][NP][2], av[4][NP][2];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (kc + p * 64 >= kw) break;
      const int k = kb + kc + p * 64 + fk;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const bf16* src = W + (size_t)(n0 + j * 16 + fr) * g.ldw + k;
        wv[j][p][0] = gload16(src);
        wv[j][p][1] = gload16(src + 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16* src = A + (size_t)min(i * 16 + fr, g.M - 1) * g.lda + k;
        av[i][p][0] = gload16(src);
        av[i][p][1] = gload16(src + 8);
      }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (kc + p * 64 >= kw) break;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[i][p][hh]),
                                                                __builtin_bit_cast(bf16x8, wv[j][p][hh]), acc[i][j], 0, 0, 0);
    }
  }

  // sum the waves' tiles
  float* r = red[wave];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) r[(i * 16 + (lane >> 4) * 4 + e) * LDR + j * 16 + (lane & 15)] = acc[i][j][e];
  __syncthreads();
  const int row = tid / TPR, q = tid % TPR;
  const bool ok = row < g.M;
  const int frow = ok ? row : g.M - 1;
  const float sc = Epi::kRowScale ? s_inv[row] : 1.f;
  auto tot = [&](int c) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w][row * LDR + c];
    return sc * t;
  };
  if constexpr (Epi::kPaired) {
    // thread q of the row handles pairs q*CPT/2 .. +CPT/2 of the row's BN/2 pairs
    typename Epi::Pre pre[CPT / 2];
#pragma unroll
    for (int e = 0; e < CPT / 2; ++e) {
      const int p = q * (CPT / 2) + e;
      pre[e] = epi.fetch(frow, n0 + (p >> 4) * 32 + (p & 15));
    }
#pragma unroll
    for (int e = 0; e < CPT / 2; ++e) {
      const int p = q * (CPT / 2) + e, c = (p >> 4) * 32 + (p & 15);
      if (ok) epi.pair(row, n0 + c, tot(c), tot(c + 16), pre[e]);
    }
  } else {
    typename Epi::Pre pre[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) pre[e] = epi.fetch(frow, n0 + q * CPT + e);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const int c = q * CPT + e;
      if (ok) ss += epi.one(row, n0 + c, tot(c), pre[e]);
    }
    if constexpr (Epi::kSsq) {
      // the TPR threads of a row are consecutive lanes of one wave
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
      if (ok && q == 0) epi.ssq(row, blockIdx.x, ss);
    }
  }
}

// ---------------------------------------------------------------------------
// gemm_stream_kernel + gemm_reduce_kernel: bf16, M <= 64 rows (batch 1).
// The weights are the only large operand, so the work is split over both N
// (64 columns per block, 16 per wave) and K (KB per block) to put every CU on
// the weight stream: a block issues all its weight loads (KB/4 elements per
// lane) and its share of the activation slice [64][KB] at once, stages the
// activations in LDS for its 4 waves and writes a float32 partial tile
// [M][64] to partial[k-split].  gemm_reduce_kernel then adds the K-split
// partials in split order and runs the epilogue, one wave per (row, 256
// columns) -- 512 for paired epilogues.  Residual producers (kSsq) therefore
// write one sum-of-squares partial per 256 columns.
// ---------------------------------------------------------------------------
constexpr int kStreamGroup = 256;  // columns per reduce wave (non-paired)

template <int KB>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs g) {
  constexpr int LDA = KB + 8;          // padded LDS row (bf16 elements)
  constexpr int NP = KB / 64;          // 64-wide K chunks
  constexpr int AV = 64 * KB / 8 / 256;  // 16-byte activation vectors per thread
  __shared__ __attribute__((aligned(16))) bf16 As[64 * LDA];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 64 + wave * 16, k0 = blockIdx.y * KB;
  const bf16* __restrict__ A = reinterpret_cast<const bf16*>(g.A);
  const bf16* __restrict__ W = reinterpret_cast<const bf16*>(g.W);

  // lane (r, q) = (l % 16, l / 16): weight row n0 + r, elements 16q .. 16q+15 of every 64-wide chunk
  // (the first 8 feed one MFMA step, the next 8 another; the activations use the same K order)
  const bf16* wp = W + (size_t)(n0 + (lane & 15)) * g.ldw + k0 + (lane >> 4) * 16;
  u32x4 wv[NP][2];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    wv[p][0] = gload16(wp + p * 64);
    wv[p][1] = gload16(wp + p * 64 + 8);
  }
  // activation rows past M repeat row M-1; their results are never stored
  u32x4 av[AV];
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const int v = tid + i * 256, r = v / (KB / 8), c = (v % (KB / 8)) * 8;
    av[i] = gload16(A + (size_t)min(r, g.M - 1) * g.lda + k0 + c);
  }
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const int v = tid + i * 256, r = v / (KB / 8), c = (v % (KB / 8)) * 8;
    *reinterpret_cast<u32x4*>(&As[r * LDA + c]) = av[i];
  }
  __syncthreads();

  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&As[(i * 16 + (lane & 15)) * LDA + p * 64 + (lane >> 4) * 16 + hh * 8]);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, wv[p][hh]), acc[i], 0, 0, 0);
      }

  float* P = g.partial + (size_t)blockIdx.y * g.M * g.N + n0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = i * 16 + (lane >> 4) * 4 + e;
      if (row < g.M) P[(size_t)row * g.N] = acc[i][e];
    }
}

// Sum of the g.splits K-split partials of 4 consecutive columns of a row, in
// split order.  Loads go out 16 at a time (indices past the last split re-read
// it and are dropped), so a reduce costs one memory round trip per 16 splits.
__device__ __forceinline__ f32x4 sum_splits(const GemmArgs& g, int row, int c0) {
  const size_t plane = (size_t)g.M * g.N;
  const float* p = g.partial + (size_t)row * g.N + c0;
  f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < g.splits; k0 += 16) {
    f32x4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = *reinterpret_cast<const f32x4*>(p + (size_t)min(k0 + k, g.splits - 1) * plane);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k0 + k < g.splits) t += v[k];
  }
  return t;
}

template <class Epi>
__global__ __launch_bounds__(64) void gemm_reduce_kernel(GemmArgs g, Epi epi) {
  const int lane = threadIdx.x, row = blockIdx.y;
  float sc = 1.f;
  if constexpr (Epi::kRowScale) {
    float s = 0.f;
    const float* p = g.ssq_in + (size_t)row * g.ssq_np;
    for (int i = 0; i < g.ssq_np; ++i) s += p[i];
    sc = 1.0f / sqrtf(s / (float)g.norm_dim + g.norm_eps);
  }
  if constexpr (Epi::kPaired) {
    // lane: columns c0 .. c0+3 (c0 % 32 < 16) and their partners c0+16 .. c0+19
    const int q = blockIdx.x * 64 + lane;
    const int c0 = (q >> 2) * 32 + (q & 3) * 4;
    if (c0 >= g.N) return;
    typename Epi::Pre pre[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pre[e] = epi.fetch(row, c0 + e);
    const f32x4 lo = sum_splits(g, row, c0), hi = sum_splits(g, row, c0 + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) epi.pair(row, c0 + e, sc * lo[e], sc * hi[e], pre[e]);
  } else {
    const int c0 = (blockIdx.x * 64 + lane) * 4;
    const bool ok = c0 < g.N;
    const int cf = ok ? c0 : 0;
    typename Epi::Pre pre[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pre[e] = epi.fetch(row, cf + e);
    const f32x4 t = sum_splits(g, row, cf);
    float ss = 0.f;
    if (ok) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += epi.one(row, c0 + e, sc * t[e], pre[e]);
    }
    if constexpr (Epi::kSsq) {
      ss = wave_sum(ss);
      if (lane == 0) epi.ssq(row, blockIdx.x, ss);
    }
  }
}

}  // namespace pi0x
