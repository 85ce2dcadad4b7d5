// Matrix-core GEMMs C = A * W^T for the expert's projections, with fused
// prologues and epilogues.  A is [M][K] row-major (activations), W is [N][K]
// row-major (nn.Linear layout, so both operands are contiguous along K); C is
// handed element by element (or in pairs, see below) to an epilogue functor.
//
// Three kernels share the epilogues:
//  * gemm_kernel      16x16 tiles, bf16 or fp32 operands (fp32 through eight
//                     v_mfma_f32_16x16x4_f32 per 32-wide K slice): the float32
//                     path and the fallback for any shape.
//  * gemm_big_kernel  bf16, v_mfma_f32_32x32x16_bf16, 128x128 or 256x256
//                     block tiles with 2x2 waves of 64x64 / 128x128 and K
//                     slices of 64 double-buffered through padded LDS: the
//                     compute-bound shapes (batch >= 2).
//  * gemm_skinny_kernel  bf16, M <= 64: the weight-streaming shapes (batch 1).
//                     No LDS staging of operands: each of 8 waves streams an
//                     eighth of the K range with 32-byte loads per lane, the
//                     next 64-wide K slice in flight while the current one
//                     feeds the MFMAs, and the waves' tiles are summed through
//                     LDS.
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
// Split-K (gemm_kernel only): the K range is divided over gridDim.z; each
// block writes its partial tile and the last block to arrive adds the shares
// in split order and runs the epilogue.  The hand-off needs device-scope
// fences, which cost tens of microseconds on this part, so the bf16 kernels
// never split K.
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
// ---------------------------------------------------------------------------
struct NoPre {};

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
  __device__ __forceinline__ void ssq(int row, int group, float s) const { ssq_out[(size_t)row * np + group] = s; }
};

// Fused q/k/v projection epilogue (after the inv_rms row scale): rotate-half
// RoPE on every q head and the k head at position valid_len[b] + s for suffix
// token s of sample b (float32 cos/sin table [position][head_dim/2]).  q and k
// go to out[row][q heads | k] in the natural layout; the values go transposed
// to vt[b][d][vt_ld] (column s), the layout attention reads them in.
template <typename T>
struct EpiQkvRope {
  static constexpr bool kPaired = true, kRowScale = true, kSsq = false;
  using Pre = float2;  // (cos, sin) of the pair's angle
  T* out;
  int ldo;
  int qk_cols;  // (num_heads + 1) * head_dim
  int head_dim, S, L;
  const CallDesc* desc;
  const float* cos_t;
  const float* sin_t;
  T* vt;
  int vt_ld;
  __device__ __forceinline__ int jj(int c) const {
    const int w = c % head_dim;
    return (w >> 5) * 16 + (w & 15);
  }
  __device__ __forceinline__ Pre fetch(int row, int c) const {
    if (c >= qk_cols) return float2{0.f, 0.f};
    const int b = row / S, s = row - b * S;
    int v = desc->valid[b];
    v = v < 0 ? 0 : (v > L ? L : v);
    const size_t t = (size_t)(v + s) * (head_dim >> 1) + jj(c);
    return float2{cos_t[t], sin_t[t]};
  }
  __device__ __forceinline__ void pair(int row, int c, float x1, float x2, Pre cs) const {
    if (c < qk_cols) {
      const int half = head_dim >> 1;
      T* o = out + (size_t)row * ldo + (c / head_dim) * head_dim + jj(c);
      o[0] = from_f32<T>(x1 * cs.x - x2 * cs.y);
      o[half] = from_f32<T>(x2 * cs.x + x1 * cs.y);
    } else {
      const int b = row / S, s = row - b * S;
      T* o = vt + ((size_t)b * head_dim + (c - qk_cols)) * vt_ld + s;
      o[0] = from_f32<T>(x1);
      o[(size_t)16 * vt_ld] = from_f32<T>(x2);
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
};

// Velocity projection and Euler update (page 1, the end of denoise_step and
// the update of sample_actions), after the inv_rms row scale of the final
// norm: GEMM row r is hidden row r of the suffix, column c < A an action
// feature.  The state rows (r % S == 0) and padding columns are dropped.
// v = acc + b_out[c]; mode 0: x <- x + dt v (x from desc->x_in on the first
// step, else x_loop; written to x_loop and, on the last step, to desc->out);
// mode 1: v is written to desc->out.
struct EpiEuler {
  static constexpr bool kPaired = false, kRowScale = true, kSsq = false;
  using Pre = float;  // the current x
  float* x_loop;
  const CallDesc* desc;
  const float* b_out;
  int H, S, A;
  int from_input, write_out, mode;
  float dt;
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
    const float v = acc + b_out[col];
    if (mode == 1) {
      desc->out[i] = v;
    } else {
      const float xn = x + dt * v;
      x_loop[i] = xn;
      if (write_out) desc->out[i] = xn;
    }
    return 0.f;
  }
  __device__ __forceinline__ void ssq(int, int, float) const {}
};

// inv_rms of rows m0 .. m0+n-1 into s_inv (threads < n), from the partials.
__device__ __forceinline__ void row_scale_prologue(const GemmArgs& g, int m0, int n, float* s_inv) {
  const int t = threadIdx.x;
  if (t < n) {
    float s = 0.f;
    if (m0 + t < g.M) {
      const float* p = g.ssq_in + (size_t)(m0 + t) * g.ssq_np;
      for (int i = 0; i < g.ssq_np; ++i) s += p[i];
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
    // hand-off: the block's stores complete at the barrier, one thread publishes
    __syncthreads();
    if (tid == 0) {
      __threadfence();
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
// gemm_big_kernel: bf16, 32x32x16 MFMA, 2x2 waves, K slices of 64
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

template <int BM, int BN>
constexpr size_t big_smem_bytes() {
  return (size_t)2 * (BM + BN) * (64 + 8) * 2;
}

template <int BM, int BN, class Epi>
__global__ __launch_bounds__(256) void gemm_big_kernel(GemmArgs g, Epi epi) {
  constexpr int BK = 64, LDK = BK + 8;  // 144-byte LDS rows: conflict-free 16-byte fragment reads
  constexpr int TM = BM / 2 / 32, TN = BN / 2 / 32;
  constexpr int CPR = BK / 8;  // 16-byte chunks per row
  constexpr int AC = BM * CPR / 256, BC = BN * CPR / 256;
  constexpr int ELD = TN * 32 + 1;  // epilogue staging row (floats)
  static_assert(AC >= 1 && BC >= 1 && BM * CPR % 256 == 0 && BN * CPR % 256 == 0, "tile/thread mismatch");
  static_assert(4 * 32 * ELD * 4 <= (int)big_smem_bytes<BM, BN>(), "epilogue staging must fit");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16* As = reinterpret_cast<bf16*>(smem_raw);  // [2][BM*LDK]
  bf16* Bs = As + 2 * BM * LDK;                   // [2][BN*LDK]
  __shared__ float s_inv[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_tile = blockIdx.x, m_tile = blockIdx.y;
  const int m0 = m_tile * BM, n0 = n_tile * BN;
  const int KI = g.K / BK;
  const bf16* __restrict__ A = reinterpret_cast<const bf16*>(g.A);
  const bf16* __restrict__ W = reinterpret_cast<const bf16*>(g.W);

  // staging: thread t moves 16-byte chunks t, t+256, ... of each operand tile
  // rows past M load row M-1 (unconditional loads keep the pipeline free of
  // waits); their results are never stored
  const bf16* aptr[AC];
  int aoff[AC];
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int c = tid + i * 256, row = c / CPR, kc = (c % CPR) * 8;
    aptr[i] = A + (size_t)min(m0 + row, g.M - 1) * g.lda + kc;
    aoff[i] = row * LDK + kc;
  }
  const bf16* bptr[BC];
  int boff[BC];
#pragma unroll
  for (int i = 0; i < BC; ++i) {
    const int c = tid + i * 256, row = c / CPR, kc = (c % CPR) * 8;
    bptr[i] = W + (size_t)(n0 + row) * g.ldw + kc;
    boff[i] = row * LDK + kc;
  }
  u32x4 ra[AC], rb[BC];

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if constexpr (Epi::kRowScale) row_scale_prologue(g, m0, BM, s_inv);
#pragma unroll
  for (int i = 0; i < AC; ++i) ra[i] = *reinterpret_cast<const u32x4*>(aptr[i]);
#pragma unroll
  for (int i = 0; i < BC; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bptr[i]);
#pragma unroll
  for (int i = 0; i < AC; ++i) *reinterpret_cast<u32x4*>(&As[aoff[i]]) = ra[i];
#pragma unroll
  for (int i = 0; i < BC; ++i) *reinterpret_cast<u32x4*>(&Bs[boff[i]]) = rb[i];
  __syncthreads();
  int st = 0;
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  for (int kt = 0; kt < KI; ++kt) {
    const bool more = kt + 1 < KI;
    if (more) {
      const int ko = (kt + 1) * BK;
#pragma unroll
      for (int i = 0; i < AC; ++i) ra[i] = *reinterpret_cast<const u32x4*>(aptr[i] + ko);
#pragma unroll
      for (int i = 0; i < BC; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bptr[i] + ko);
    }
    const bf16* as = As + st * BM * LDK + (wm * TM * 32 + fr) * LDK + fk;
    const bf16* bs = Bs + st * BN * LDK + (wn * TN * 32 + fr) * LDK + fk;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(as + i * 32 * LDK + kk * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(bs + j * 32 * LDK + kk * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    // keep the stores of the next slice (and their wait on its global loads)
    // after the matrix-core work, so the loads overlap the MFMAs
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
      bf16* as_n = As + (st ^ 1) * BM * LDK;
      bf16* bs_n = Bs + (st ^ 1) * BN * LDK;
#pragma unroll
      for (int i = 0; i < AC; ++i) *reinterpret_cast<u32x4*>(&as_n[aoff[i]]) = ra[i];
#pragma unroll
      for (int i = 0; i < BC; ++i) *reinterpret_cast<u32x4*>(&bs_n[boff[i]]) = rb[i];
    }
    __syncthreads();
    st ^= 1;
  }

  // Epilogue through LDS, one 32-row strip of the wave tile at a time: the
  // strip is written in the MFMA layout (element (i, j, v) is row
  // 8 (v/4) + 4 (lane/32) + v%4, column 32 j + lane % 32 of the strip) and read
  // back row-wise, so the epilogue loops index no accumulator dynamically.
  // Lanes cover LPR items of a row and RPI rows at a time; the reads of 8 such
  // row groups are issued before their stores.
  float* strip = reinterpret_cast<float*>(smem_raw) + wave * 32 * ELD;
  const int mb = m0 + wm * TM * 32, nb = n0 + wn * TN * 32;
  constexpr int WC = TN * 32;                            // wave tile width
  constexpr int PPR = Epi::kPaired ? WC / 2 : WC;        // items per row
  constexpr int LPR = PPR < 64 ? PPR : 64;               // lanes per row
  constexpr int RPI = 64 / LPR;                          // rows per pass
  constexpr int IPL = PPR / LPR;                         // items per lane and row
  constexpr int NP = 32 / RPI;                           // passes per strip
  constexpr int GP = NP < 8 ? NP : 8;                    // passes per read group
  const int lr = lane / LPR, lc = lane % LPR;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        strip[((v >> 2) * 8 + (lane >> 5) * 4 + (v & 3)) * ELD + j * 32 + (lane & 31)] = acc[i][j][v];
    __syncthreads();
#pragma unroll
    for (int p0 = 0; p0 < NP; p0 += GP) {
      typename Epi::Pre pre[GP][IPL];
#pragma unroll
      for (int pp = 0; pp < GP; ++pp) {
        const int row = min(mb + i * 32 + (p0 + pp) * RPI + lr, g.M - 1);
#pragma unroll
        for (int q = 0; q < IPL; ++q) {
          const int it = lc + q * LPR;
          const int c = Epi::kPaired ? (it >> 4) * 32 + (it & 15) : it;
          pre[pp][q] = epi.fetch(row, nb + c);
        }
      }
#pragma unroll
      for (int pp = 0; pp < GP; ++pp) {
        const int r = (p0 + pp) * RPI + lr;
        const int row = mb + i * 32 + r;
        const bool ok = row < g.M;
        const float sc = Epi::kRowScale ? s_inv[min(row, g.M - 1) - m0] : 1.f;
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < IPL; ++q) {
          const int it = lc + q * LPR;
          if constexpr (Epi::kPaired) {
            const int c = (it >> 4) * 32 + (it & 15);
            if (ok) epi.pair(row, nb + c, sc * strip[r * ELD + c], sc * strip[r * ELD + c + 16], pre[pp][q]);
          } else {
            if (ok) ss += epi.one(row, nb + it, sc * strip[r * ELD + it], pre[pp][q]);
          }
        }
        if constexpr (Epi::kSsq) {
#pragma unroll
          for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
          if (ok && lc == 0) epi.ssq(row, nb / WC, ss);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// gemm_skinny_kernel: bf16, M <= 64 rows, BN (16/32/64) output columns per block
// ---------------------------------------------------------------------------
template <int BN, class Epi>
__global__ __launch_bounds__(512) void gemm_skinny_kernel(GemmArgs g, Epi epi) {
  constexpr int NW = 8;                         // waves; each takes 1/8 of the K range
  constexpr int TN = BN / 16, TM = 4, KS = 64;  // K super-slice: two 16x16x32 MFMA steps
  constexpr int LDR = BN + 1;
  constexpr int TPR = 512 / 64;                 // epilogue threads per row
  constexpr int CPT = BN / TPR;                 // columns per thread in the epilogue
  static_assert(!Epi::kPaired || BN >= 32, "paired epilogues need 32-column groups");
  __shared__ float red[NW][64 * LDR];
  __shared__ float s_inv[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * BN;
  const int KI = g.K / KS;
  const int wb = KI * wave / NW, we = KI * (wave + 1) / NW;
  const bf16* __restrict__ A = reinterpret_cast<const bf16*>(g.A);
  const bf16* __restrict__ W = reinterpret_cast<const bf16*>(g.W);

  if constexpr (Epi::kRowScale) row_scale_prologue(g, 0, 64, s_inv);

  // lane (l%16, l/16): row/column l%16 of each 16-tile, K elements 16*(l/16) .. +15 of a super-slice
  const int fr = lane & 15, fk = (lane >> 4) * 16;
  const bf16* wp = W + (size_t)(n0 + fr) * g.ldw + fk;
  // rows past M read row M-1 (unconditional loads); their results are never stored
  const bf16* ap[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) ap[i] = A + (size_t)min(i * 16 + fr, g.M - 1) * g.lda + fk;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // two register stages: the loads of slice k+1 are in flight while slice k feeds the MFMAs
  u32x4 wv[2][TN][2], av[2][TM][2];
  auto load = [&](int st, int k) {
    const size_t ko = (size_t)k * KS;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const u32x4* p = reinterpret_cast<const u32x4*>(wp + (size_t)j * 16 * g.ldw + ko);
      wv[st][j][0] = p[0];
      wv[st][j][1] = p[1];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const u32x4* p = reinterpret_cast<const u32x4*>(ap[i] + ko);
      av[st][i][0] = p[0];
      av[st][i][1] = p[1];
    }
  };
  auto compute = [&](int st) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[st][i][hh]),
                                                              __builtin_bit_cast(bf16x8, wv[st][j][hh]), acc[i][j],
                                                              0, 0, 0);
  };
  if (wb < we) load(0, wb);
  for (int k = wb; k < we; k += 2) {
    if (k + 1 < we) load(1, k + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    if (k + 1 < we) {
      if (k + 2 < we) load(0, k + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(1);
    }
  }

  // sum the waves' tiles
  float* r = red[wave];
#pragma unroll
  for (int i = 0; i < TM; ++i)
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
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
      if (ok && q == 0) epi.ssq(row, blockIdx.x, ss);
    }
  }
}

}  // namespace pi0x
