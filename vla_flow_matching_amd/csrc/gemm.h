// Tiled MFMA GEMM C = A * W^T for the expert's projections, with fused
// epilogues.  A is [M][K] row-major (activations), W is [N][K] row-major
// (nn.Linear layout, so both operands are contiguous along K).  K must be a
// multiple of 32 and N a multiple of the tile width; rows beyond M read as
// zero and are never written.
//
// Each 256-thread block owns a BM x BN output tile, split over 4 waves as
// WM x WN wave tiles of (BM/WM) x (BN/WN).  A and W tiles of 32 along K are
// staged through LDS (rows padded by 16 bytes), double-buffered so the global
// loads of slice k+1 are in flight while slice k feeds the matrix cores.
// With splits > 1 the K range is divided over gridDim.z blocks; each writes
// its partial tile and the last block to arrive adds the shares in split
// order (so results do not depend on arrival order) and runs the epilogue.
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
  float* partial;      // splits > 1: [tiles][splits][BM*BN] scratch
  unsigned* counters;  // splits > 1: [tiles] arrival counters, zero between launches
};

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

  __shared__ __attribute__((aligned(16))) T As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int n_tile = blockIdx.x, m_tile = blockIdx.y, split = blockIdx.z;
  const int m0 = m_tile * BM, n0 = n_tile * BN;
  const int KI = g.K / BK;
  const int kb = (int)((long)split * KI / g.splits), ke = (int)((long)(split + 1) * KI / g.splits);
  const T* __restrict__ A = reinterpret_cast<const T*>(g.A);
  const T* __restrict__ W = reinterpret_cast<const T*>(g.W);

  uint4 ra[AVT], rb[BVT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < AVT; ++i) {
      int v = tid + i * 256;
      if (v < AV) {
        int row = v / VPR, kc = (v % VPR) * VE, grow = m0 + row;
        ra[i] = grow < g.M ? *reinterpret_cast<const uint4*>(A + (size_t)grow * g.lda + kt * BK + kc)
                           : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < BVT; ++i) {
      int v = tid + i * 256;
      if (v < BV) {
        int row = v / VPR, kc = (v % VPR) * VE, grow = n0 + row;
        rb[i] = grow < g.N ? *reinterpret_cast<const uint4*>(W + (size_t)grow * g.ldw + kt * BK + kc)
                           : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < AVT; ++i) {
      int v = tid + i * 256;
      if (v < AV) *reinterpret_cast<uint4*>(&As[st][(v / VPR) * LDK + (v % VPR) * VE]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BVT; ++i) {
      int v = tid + i * 256;
      if (v < BV) *reinterpret_cast<uint4*>(&Bs[st][(v / VPR) * LDK + (v % VPR) * VE]) = rb[i];
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

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
    if (!arrive_last(&g.counters[tile], (unsigned)g.splits, tid)) return;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float s = 0.f;
          for (int z = 0; z < g.splits; ++z) s += __builtin_nontemporal_load(&P[((size_t)z * NR + (i * TN + j) * 4 + e) * 256 + tid]);
          acc[i][j][e] = s;
        }
    if (tid == 0) g.counters[tile] = 0u;
  }
  epi.template apply<TM, TN>(acc, m0 + wm * TM * 16, n0 + wn * TN * 16, lane, g.M);
}

// ---------------------------------------------------------------------------
// Epilogues.  apply() receives the wave's accumulators; element (i, j, e) is
// C[mb + 16 i + 4 (lane/16) + e][nb + 16 j + lane % 16].
// ---------------------------------------------------------------------------
#define PI0X_EPI_LOOP(...)                                              \
  _Pragma("unroll") for (int i = 0; i < TM; ++i)                          \
  _Pragma("unroll") for (int e = 0; e < 4; ++e) {                        \
    const int row = mb + i * 16 + (lane >> 4) * 4 + e;                   \
    if (row >= M) continue;                                              \
    __VA_ARGS__                                                          \
  }

// out[row][col] = act(acc + bias[col]) in TO; act = SiLU when silu != 0.
template <typename TO>
struct EpiStore {
  TO* out;
  int ldo;
  const float* bias;  // may be null
  int silu;
  template <int TM, int TN>
  __device__ __forceinline__ void apply(f32x4 (&acc)[TM][TN], int mb, int nb, int lane, int M) const {
    PI0X_EPI_LOOP(
      _Pragma("unroll") for (int j = 0; j < TN; ++j) {
        const int col = nb + j * 16 + (lane & 15);
        float v = acc[i][j][e] + (bias ? bias[col] : 0.f);
        if (silu) v = pi0x::silu(v);
        out[(size_t)row * ldo + col] = from_f32<TO>(v);
      })
  }
};

// Action rows of the suffix embedding: GEMM row r = b*H + i goes to hidden row
// b*S + 1 + i (row 0 of each sample is the state token).
struct EpiSuffixRows {
  float* h;
  int ldh, H, S;
  const float* bias;
  template <int TM, int TN>
  __device__ __forceinline__ void apply(f32x4 (&acc)[TM][TN], int mb, int nb, int lane, int M) const {
    PI0X_EPI_LOOP(
      const int hrow = (row / H) * S + 1 + row % H;
      _Pragma("unroll") for (int j = 0; j < TN; ++j) {
        const int col = nb + j * 16 + (lane & 15);
        h[(size_t)hrow * ldh + col] = acc[i][j][e] + bias[col];
      })
  }
};

// Residual update h[row][col] += acc (float32 residual stream).
struct EpiResidual {
  float* h;
  int ldh;
  template <int TM, int TN>
  __device__ __forceinline__ void apply(f32x4 (&acc)[TM][TN], int mb, int nb, int lane, int M) const {
    PI0X_EPI_LOOP(
      _Pragma("unroll") for (int j = 0; j < TN; ++j) {
        const int col = nb + j * 16 + (lane & 15);
        float* p = &h[(size_t)row * ldh + col];
        *p = *p + acc[i][j][e];
      })
  }
};

// Fused q/k/v projection epilogue.  The weight rows of every q and k head are
// stored so that output tiles come in pairs: tile 2p holds head elements
// 16p..16p+15 and tile 2p+1 holds half+16p..half+16p+15 (half = head_dim/2),
// i.e. the two halves that rotate-half RoPE mixes.  Rows are positioned at
// valid_len[b] + s for suffix token s of sample b; the rotation uses a float32
// cos/sin table [position][half].  Columns past the k head (the values) are
// stored unrotated.  Output in the natural layout [row][q heads | k | v].
template <typename T>
struct EpiQkvRope {
  T* out;
  int ldo;
  int qk_cols;  // (num_heads + 1) * head_dim
  int head_dim, S, L;
  const CallDesc* desc;
  const float* cos_t;
  const float* sin_t;
  template <int TM, int TN>
  __device__ __forceinline__ void apply(f32x4 (&acc)[TM][TN], int mb, int nb, int lane, int M) const {
    static_assert(TN % 2 == 0, "rope pairs need an even number of column tiles");
    const int half = head_dim >> 1;
    PI0X_EPI_LOOP(
      const int b = row / S, s = row - b * S;
      int v = desc->valid[b];
      v = v < 0 ? 0 : (v > L ? L : v);
      const int pos = v + s;
      _Pragma("unroll") for (int j = 0; j < TN; j += 2) {
        const int c = nb + j * 16 + (lane & 15);
        const float x1 = acc[i][j][e], x2 = acc[i][j + 1][e];
        if (c < qk_cols) {
          const int head = c / head_dim, w = c - head * head_dim;
          const int jj = (w >> 5) * 16 + (w & 15);
          const float cs = cos_t[(size_t)pos * half + jj], sn = sin_t[(size_t)pos * half + jj];
          T* o = out + (size_t)row * ldo + head * head_dim + jj;
          o[0] = from_f32<T>(x1 * cs - x2 * sn);
          o[half] = from_f32<T>(x2 * cs + x1 * sn);
        } else {
          out[(size_t)row * ldo + c] = from_f32<T>(x1);
          out[(size_t)row * ldo + c + 16] = from_f32<T>(x2);
        }
      })
  }
};

// GeGLU epilogue: weight rows interleave gate and up in blocks of 16 (tile 2p
// = gate rows 16p.., tile 2p+1 = up rows 16p..), so one lane holds gate and up
// of the same output column: out[row][16p + lane%16] = gelu_tanh(g) * u.
template <typename T>
struct EpiGeglu {
  T* out;
  int ldo;
  template <int TM, int TN>
  __device__ __forceinline__ void apply(f32x4 (&acc)[TM][TN], int mb, int nb, int lane, int M) const {
    static_assert(TN % 2 == 0, "gate/up pairs need an even number of column tiles");
    PI0X_EPI_LOOP(
      _Pragma("unroll") for (int j = 0; j < TN; j += 2) {
        const int col = ((nb + j * 16) >> 1) + (lane & 15);
        out[(size_t)row * ldo + col] = from_f32<T>(gelu_tanh(acc[i][j][e]) * acc[i][j + 1][e]);
      })
  }
};

}  // namespace pi0x
