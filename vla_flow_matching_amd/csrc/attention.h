// Grouped-query attention of the expert's suffix over [cached prefix ; suffix]
// keys with the pi0 mask (page 1, _attend and make_att_2d_masks as used by
// denoise_step): every suffix query sees the valid prefix keys j < valid_len;
// inside the suffix the state token (s = 0) sees only itself and every action
// token (s >= 1) sees the state token and all action tokens.  With causal set
// (page 3, Wall-X generate_flow_action under causal_action_attention_mask)
// suffix token s sees suffix tokens 0..s instead.
//
// Prefix pass (prefill set; page 1, _compute_layer_prefix_only under the
// prefix mask make_att_2d_masks builds from an all-zero autoregressive mask):
// the S queries per sample are the prefix tokens themselves and there are no
// suffix keys; every query sees the keys j < valid_len, which this layer's
// q/k/v epilogue has just written to the cache (desc->kv) and, transposed, to
// vtp.  Padded queries are computed like real ones (their rows are never
// read); with valid_len 0 they see no key and get a zero output.  One kv head is
// shared by all query heads, so the num_heads * S queries of a sample (query
// index qi = s*num_heads + n) form one matrix against one key/value sequence.
//
// attn_kernel: a block owns 128 queries (8 waves of 16).  Keys are staged in blocks of KB (64 for bf16, 32 for fp32): K
// row-major and V transposed ([head_dim][keys]) are copied into LDS with
// 16-byte accesses and shared by the waves, double-buffered so the global
// loads of block i+1 overlap the matrix-core work on block i.  A wave computes S^T = K Q^T, so a
// lane holds the scores of its own query (lane % 16); the online softmax runs
// in float32 in registers, in base 2 against a reference maximum that moves
// only when a score passes it by 2^8, and O^T = V^T P^T reuses those
// probabilities
// directly as the MFMA operand.  The prefix values are transposed once per
// call by transpose_v_kernel, the suffix values are written transposed by the
// q/k/v projection.  Masked keys get probability exactly 0; padded prefix keys
// are never read from the caller's cache (zeros are used instead).
//
// With splits > 1 (small batches) the key blocks of a sample are divided into
// splits; each split writes its reference maximum (log2 units), sum and
// unnormalised output and attn_combine_kernel merges them in split order.
//
// Block order: the grid is 1-D and blocks are dealt round-robin to the 8 XCDs
// (block L runs on XCD L % 8).  Work unit u = (b * splits + split) * tiles +
// tile goes to block (u / per_xcd) + 8 * (u % per_xcd), per_xcd = ceil(units
// / 8): each XCD takes a contiguous run of units, so the query tiles that read
// the same keys run together on one XCD and share them in its L2.
#pragma once

#include <type_traits>

#include "common.h"

namespace pi0x {

struct AttnArgs {
  const void* qk;  // [B*S][ldqk]: q heads at column 0, the k head at col_k
  int ldqk, col_k;
  const CallDesc* desc;
  size_t kv_k_off;  // element offset of this layer's prefix K block inside desc->kv
  const void* vtp;  // this layer's prefix V^T: [B][head_dim][Lp], zero beyond valid_len
  int Lp;
  const void* vts;  // suffix V^T: [B][head_dim][Sp], zero beyond S
  int Sp;
  int B, L, S, nh;
  void* out;  // [B*S][ldo], head n of token s at column n*head_dim
  int ldo;
  float scale;
  int causal;  // suffix mask: 0 pi0 block rule, 1 lower triangle
  int prefill;  // prefix pass: prefix keys only
  int splits, tiles;
  float* partial;  // splits > 1, per (B, tile, split, QT-tile): float32 reference maximum (log2 units) and sum [2][threads],
                   // then the unnormalised outputs in the model dtype [head_dim/16][threads][4]
};

// Per dtype: KB keys per staged block, NW waves per block, QT 16-query tiles
// per wave (NW * QT * 16 = 128 queries per block).  Two query tiles per wave
// (4 waves) halve the LDS fragment reads per query but need more than the 512
// registers a lane can hold at head_dim 256 (they spill to scratch), so both
// dtypes use 8 waves of one tile.
template <typename T> struct AttnCfg;
template <> struct AttnCfg<bf16> { static constexpr int KB = 64, NW = 8, QT = 1; };
template <> struct AttnCfg<float> { static constexpr int KB = 32, NW = 8, QT = 1; };
constexpr int kAttnQueries = 128;  // queries per block (at most)

// First 16-query tile of block `tile` when the ceil(nq / 16) tiles of a
// sample are dealt out evenly over `tiles` blocks (tiles = ceil(nq / 128), so
// no block gets more than 128 queries).
__host__ __device__ __forceinline__ int attn_wave_tile0(int tile, int nq, int tiles) {
  return (int)((long)tile * ((nq + 15) / 16) / tiles);
}

// LDS layout.  bf16 (head_dim a multiple of 64): unpadded 128-byte rows --
// K split into head_dim/64 sub-tiles [KB][64], V^T [head_dim][KB = 64] -- with
// the 16-byte chunks of row r at chunk ^ ((r / 2) % 8), so the fragment reads
// (16 rows x 4 chunks per instruction) are free of bank conflicts.  float32
// (and small head dims): rows padded by 16 bytes.
template <typename T, int DH> struct AttnLds {
  static constexpr bool kSwz = sizeof(T) == 2 && DH % 64 == 0 && AttnCfg<T>::KB == 64;
  static constexpr int VE = 16 / (int)sizeof(T);
  static constexpr int LDK = kSwz ? DH : DH + VE;  // K row (padded unless swizzled)
  static constexpr int LDV = kSwz ? AttnCfg<T>::KB : AttnCfg<T>::KB + VE;
};

template <typename T, int DH>
constexpr size_t attn_smem_bytes() {
  constexpr int KB = AttnCfg<T>::KB;
  return (size_t)2 * (KB * AttnLds<T, DH>::LDK + DH * AttnLds<T, DH>::LDV) * sizeof(T);
}

// element offset of 16-byte chunk ch (of 8 bf16) of swizzled row r (64 elements)
__device__ __forceinline__ int swz64(int r, int ch) { return r * 64 + ((ch ^ ((r >> 1) & 7)) << 3); }

// The softmax runs in base 2: scores are scaled by scale * log2(e) and the
// probabilities are 2^x (the same numbers as e^(scale * s)).  bf16 mode uses
// the hardware exp2 instruction, float32 mode libm's exp2f.
template <typename T> __device__ __forceinline__ float fexp2(float x) { return exp2f(x); }
template <> __device__ __forceinline__ float fexp2<bf16>(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLog2e = 1.4426950408889634f;
// The reference maximum of a query moves only when a score exceeds it by
// more than this (log2 units), so most key blocks skip the rescale of the
// output accumulators; in between, probabilities stay below 2^8 (exact in
// float32, and in bf16 only their 8-bit mantissa is rounded, as before).
constexpr float kRefSlack = 8.f;
// Initial reference: finite, so that x - m never meets -inf - (-inf).
constexpr float kRefInit = -3.0e38f;

// Four consecutive split-partial outputs as one access: 16 bytes of float32
// or 8 bytes of bf16 (the bf16 path keeps its unnormalised partial outputs in
// bf16, halving the split traffic; the maxima and sums stay float32).
__device__ __forceinline__ void store4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, const f32x4& v) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  *reinterpret_cast<bf16x4*>(p) = bf16x4{f2bf(v[0]), f2bf(v[1]), f2bf(v[2]), f2bf(v[3])};
}
__device__ __forceinline__ void load4(const float* p, float* v) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(p);
  v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
}
__device__ __forceinline__ void load4(const bf16* p, float* v) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
  v[0] = to_f32(x[0]); v[1] = to_f32(x[1]); v[2] = to_f32(x[2]); v[3] = to_f32(x[3]);
}

template <typename T, int DH, int NW = AttnCfg<T>::NW>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnArgs a) {
  constexpr int KB = AttnCfg<T>::KB, QT = AttnCfg<T>::QT, NT = NW * 64;
  static_assert(NW * QT * 16 <= kAttnQueries, "queries per block");
  constexpr int KT = KB / 16;   // 16-key score tiles per block
  constexpr int KS = KB / 32;   // 32-key PV steps per block
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr bool SWZ = AttnLds<T, DH>::kSwz;
  constexpr int LDK = AttnLds<T, DH>::LDK;
  constexpr int LDV = AttnLds<T, DH>::LDV;
  constexpr int NC = DH / 32, ND = DH / 16;
  // fragments per read-ahead group: a feature chunk's KT key tiles for K, 4
  // feature tiles for V^T; float32 fragments take twice the registers (the
  // head_dim 256 kernel would spill), so that path reads one ahead
  constexpr int KG = sizeof(T) == 2 ? KT : 1;
  constexpr int VG = sizeof(T) != 2 ? 1 : ND % 4 == 0 ? 4 : ND % 2 == 0 ? 2 : 1;
  constexpr int NVEC = KB * DH / VE;        // 16-byte vectors of K (and of V^T) per key block
  constexpr int KVEC = (NVEC + NT - 1) / NT;  // per thread
  constexpr bool FULL = NVEC % NT == 0;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  T* Ks = reinterpret_cast<T*>(smem_raw);  // [2][KB * LDK]
  T* Vt = Ks + 2 * KB * LDK;               // [2][DH * LDV]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4;
  const int units = a.B * a.splits * a.tiles, per_xcd = (units + 7) / 8;
  const int u = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (u >= units) return;
  const int tile = u % a.tiles, split = (u / a.tiles) % a.splits, b = u / (a.tiles * a.splits);
  const int nq = a.nh * a.S;
  // the sample's 16-query tiles are dealt out evenly over its blocks (at 408
  // queries: 6, 7, 6, 7 of 8 waves), and a wave past its block's share skips
  // the score and PV work, so no block carries more waves of work than needed
  const int wt0 = attn_wave_tile0(tile, nq, a.tiles), wt1 = attn_wave_tile0(tile + 1, nq, a.tiles);
  const bool wact = wt0 + wave * QT < wt1;
  int qs[QT], qn[QT];
  bool qok[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int wt = wt0 + wave * QT + t, qi = wt * 16 + (lane & 15);
    qok[t] = wt < wt1 && qi < nq;
    qs[t] = qok[t] ? qi / a.nh : 0;
    qn[t] = qok[t] ? qi - qs[t] * a.nh : 0;
  }

  // uniform over the block: keeps the key-block loop in scalar registers
  int valid = __builtin_amdgcn_readfirstlane(a.desc->valid[b]);
  valid = valid < 0 ? 0 : (valid > a.L ? a.L : valid);
  const T* __restrict__ qk = reinterpret_cast<const T*>(a.qk);
  const T* Kp = reinterpret_cast<const T*>(a.desc->kv) + a.kv_k_off + (size_t)b * a.L * DH;
  const T* Vtp = reinterpret_cast<const T*>(a.vtp) + (size_t)b * DH * a.Lp;
  const T* Vts = reinterpret_cast<const T*>(a.vts) + (size_t)b * DH * a.Sp;
  const T* Sq = qk + (size_t)b * a.S * a.ldqk;

  // (at least one block, so that a prefix pass with no real key still stages
  // an in-bounds block; its keys are all masked)
  const int nb_pre = a.prefill ? max((valid + KB - 1) / KB, 1) : (valid + KB - 1) / KB;
  const int nb_suf = a.prefill ? 0 : (a.S + KB - 1) / KB;
  const int nblk = nb_pre + nb_suf;
  const int blk_b = (int)((long)split * nblk / a.splits), blk_e = (int)((long)(split + 1) * nblk / a.splits);

  // staging of key block blk into registers; keys past the limit become
  // zeros when stored to LDS (masking at load time would wait on the load)
  u32x4 rk[KVEC], rv[KVEC];
  unsigned kzero = 0;
  auto gload = [&](int blk) {
    const bool pre = blk < nb_pre;
    const int base = pre ? blk * KB : (blk - nb_pre) * KB;
    const int lim = pre ? valid : a.S;
    kzero = 0;
#pragma unroll
    for (int i = 0; i < KVEC; ++i) {
      const int v = tid + i * NT, kk = v / (DH / VE), dc = v % (DH / VE), key = base + kk;
      if (!FULL && v >= NVEC) break;
      const T* src = pre ? Kp + (size_t)min(key, max(lim - 1, 0)) * DH : Sq + (size_t)min(key, lim - 1) * a.ldqk + a.col_k;
      rk[i] = gload16(src + dc * VE);
      kzero |= (key >= lim ? 1u : 0u) << i;
    }
#pragma unroll
    for (int i = 0; i < KVEC; ++i) {
      const int v = tid + i * NT, d = v / (KB / VE), kc = (v % (KB / VE)) * VE;
      if (!FULL && v >= NVEC) break;
      const T* src = pre ? Vtp + (size_t)d * a.Lp + base + kc : Vts + (size_t)d * a.Sp + base + kc;
      rv[i] = gload16(src);
    }
  };
  auto sstore = [&](int st) {
    T* ks = Ks + st * KB * LDK;
    T* vt = Vt + st * DH * LDV;
#pragma unroll
    for (int i = 0; i < KVEC; ++i) {
      const int v = tid + i * NT, kk = v / (DH / VE), dc = v % (DH / VE);
      if (!FULL && v >= NVEC) break;
      const int off = SWZ ? (dc >> 3) * (KB * 64) + swz64(kk, dc & 7) : kk * LDK + dc * VE;
      *reinterpret_cast<u32x4*>(&ks[off]) = ((kzero >> i) & 1u) ? u32x4{0u, 0u, 0u, 0u} : rk[i];
    }
#pragma unroll
    for (int i = 0; i < KVEC; ++i) {
      const int v = tid + i * NT, d = v / (KB / VE), kc = (v % (KB / VE)) * VE;
      if (!FULL && v >= NVEC) break;
      const int off = SWZ ? swz64(d, kc >> 3) : d * LDV + kc;
      *reinterpret_cast<u32x4*>(&vt[off]) = rv[i];
    }
  };

  Frag<T> qf[QT][NC];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const T* qrow = Sq + (size_t)qs[t] * a.ldqk + qn[t] * DH;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (qok[t]) load8(qf[t][c], qrow + c * 32 + g * 8);
      else
#pragma unroll
        for (int i = 0; i < 8; ++i) set_frag(qf[t][c], i, 0.f);
    }
  }
  f32x4 o[QT][ND];
#pragma unroll
  for (int t = 0; t < QT; ++t)
#pragma unroll
    for (int d = 0; d < ND; ++d) o[t][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  // reference maximum in log2 units (same on the 4 lanes of a query) and this
  // lane's share of the sum, per query tile
  const float c2 = a.scale * kLog2e;
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m_run[t] = kRefInit;
    l_run[t] = 0.f;
  }

  // unconditional (an empty split stages a block it never reads) so that
  // every path into the loop has waited for all loads issued so far
  gload(min(blk_b, nblk - 1));
  sstore(0);
  int st = 0;
  for (int blk = blk_b; blk < blk_e; ++blk) {
    const bool more = blk + 1 < blk_e;
    if (more) gload(blk + 1);
    __syncthreads();
    const T* ks = Ks + st * KB * LDK;
    const T* vt = Vt + st * DH * LDV;
    const bool pre = blk < nb_pre;
    if (wact) {
    const int base = pre ? blk * KB : (blk - nb_pre) * KB;
    const int lim = pre ? valid : a.S;

    // scores: lane holds query tile t's query (lane % 16) vs key kt*16 + 4g + e of
    // the block.  The K-dimension loop is outermost so the KT x QT accumulator
    // chains interleave; masking follows all the matrix-core work.
    f32x4 acc[QT][KT];
#pragma unroll
    for (int t = 0; t < QT; ++t)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) acc[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The fragments of read-ahead group gi+1 are read while group gi's
    // MFMAs run, so several LDS reads are in flight behind every MFMA (the
    // compiler otherwise sinks each read next to its MFMA, one in flight);
    // the scheduling barriers keep that order.  Fragment j is feature chunk
    // j / KT of key tile j % KT.
    Frag<T> kf[2][KG];
    auto kread = [&](int gi, Frag<T>* dst) {
#pragma unroll
      for (int i = 0; i < KG; ++i) {
        const int c = (gi * KG + i) / KT, row = (gi * KG + i) % KT * 16 + (lane & 15);
        load8(dst[i], &ks[SWZ ? (c >> 1) * (KB * 64) + swz64(row, (c & 1) * 4 + g) : row * LDK + c * 32 + g * 8]);
      }
    };
    kread(0, kf[0]);
#pragma unroll
    for (int gi = 0; gi < NC * KT / KG; ++gi) {
      if (gi + 1 < NC * KT / KG) kread(gi + 1, kf[(gi + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < KG; ++i) {
        const int c = (gi * KG + i) / KT, kt = (gi * KG + i) % KT;
#pragma unroll
        for (int t = 0; t < QT; ++t) mma32(kf[gi & 1][i], qf[t][c], acc[t][kt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // masks apply only to a block with a key past some query's limit: the
    // partial last prefix block and the suffix blocks (where the state token,
    // query s = 0, sees only key 0, and with causal query s sees keys 0..s)
    float sc[QT][KT][4], lmax[QT];
    if (!pre || base + KB > lim) {
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const int tlim = pre ? lim : (a.causal || qs[t] == 0) ? min(lim, qs[t] + 1) : lim;
        lmax[t] = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = base + kt * 16 + g * 4 + e;
            sc[t][kt][e] = key < tlim ? acc[t][kt][e] : -INFINITY;
            lmax[t] = fmaxf(lmax[t], sc[t][kt][e]);
          }
      }
    } else {
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        lmax[t] = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sc[t][kt][e] = acc[t][kt][e];
            lmax[t] = fmaxf(lmax[t], sc[t][kt][e]);
          }
      }
    }
    // the reference moves (with the rescale of sum and outputs by
    // 2^(old - new)) only when some lane of the wave has a score more than
    // kRefSlack above its query's reference; the new reference is the
    // query's maximum so far, taken over its 4 lanes
    bool move = false;
#pragma unroll
    for (int t = 0; t < QT; ++t) move |= lmax[t] * c2 > m_run[t] + kRefSlack;
    if (__any(move)) {
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        float r = fmaxf(lmax[t], __shfl_xor(lmax[t], 16, 64));
        r = fmaxf(r, __shfl_xor(r, 32, 64));
        const float mn = fmaxf(m_run[t], r * c2);
        const float alpha = fexp2<T>(m_run[t] - mn);
        l_run[t] *= alpha;
        m_run[t] = mn;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          o[t][d][0] *= alpha; o[t][d][1] *= alpha; o[t][d][2] *= alpha; o[t][d][3] *= alpha;
        }
      }
    }
#pragma unroll
    for (int ks2 = 0; ks2 < KS; ++ks2) {
      // probabilities of keys 32*ks2 + (i/4)*16 + 4g + i%4 as the PV operand
      // (a masked key: 2^-inf = 0)
      Frag<T> pf[QT];
#pragma unroll
      for (int t = 0; t < QT; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float e = fexp2<T>(fmaf(sc[t][2 * ks2 + i / 4][i % 4], c2, -m_run[t]));
          l_run[t] += e;
          set_frag(pf[t], i, e);
        }
      // V^T fragments in read-ahead groups of VG feature tiles, as for K;
      // keys 32 ks2 + {4g .. 4g+3, 16+4g .. 16+4g+3} are contiguous in the
      // vt_pos order
      Frag<T> vf[2][VG];
      auto vread = [&](int dg, Frag<T>* dst) {
#pragma unroll
        for (int j = 0; j < VG; ++j) {
          const int row = (dg * VG + j) * 16 + (lane & 15);
          load8(dst[j], &vt[SWZ ? swz64(row, ks2 * 4 + g) : row * LDV + ks2 * 32 + g * 8]);
        }
      };
      vread(0, vf[0]);
#pragma unroll
      for (int dg = 0; dg < ND / VG; ++dg) {
        if (dg + 1 < ND / VG) vread(dg + 1, vf[(dg + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < VG; ++j)
#pragma unroll
          for (int t = 0; t < QT; ++t) mma32(vf[dg & 1][j], pf[t], o[t][dg * VG + j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (more) sstore(st ^ 1);
    st ^= 1;
  }

  // lane holds O[q][d*16 + 4g + e] (unnormalised) of its query in each tile
  if (!wact) return;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    float l_tot = l_run[t] + __shfl_xor(l_run[t], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (a.splits > 1) {
      constexpr int NR = 2 + ND * 4;
      float* mine = a.partial + (((size_t)b * a.tiles + tile) * a.splits + split) * (QT * NR * NT) + (size_t)t * NR * NT;
      mine[tid] = m_run[t];
      mine[NT + tid] = l_tot;
      // the unnormalised outputs in the model dtype: [d-tile][thread][4]
      T* po = reinterpret_cast<T*>(mine + 2 * NT) + (size_t)tid * 4;
#pragma unroll
      for (int d = 0; d < ND; ++d) store4(po + (size_t)d * NT * 4, o[t][d]);
      continue;
    }
    if (!qok[t]) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;  // 0: a prefix-pass query with no real key
    T* orow = reinterpret_cast<T*>(a.out) + ((size_t)b * a.S + qs[t]) * a.ldo + qn[t] * DH;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int e = 0; e < 4; ++e) orow[d * 16 + g * 4 + e] = from_f32<T>(o[t][d][e] * inv);
  }
}

// Merges the split partial softmax states of attn_kernel in split order.
// Grid (CB * tiles, B, head_dim / 16) with CB = QT * NT / 128 blocks of 128
// threads per query tile: slot s = QT-tile t * NT + thread of attn_kernel (the
// query and the lanes it held there) is thread s % 128 of block CB * tile +
// s / 128, and takes 4 output features of d-tile blockIdx.z.  Small blocks
// spread the partial reads over more CUs than one block per query tile would.
template <int DH> constexpr int attn_combine_chunks() { return DH / 16; }

template <typename T, int DH, int NW = AttnCfg<T>::NW>
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  constexpr int QT = AttnCfg<T>::QT, NT = NW * 64, CB = QT * NT / 128;  // combine blocks per query tile
  constexpr int ND = DH / 16, NR = 2 + ND * 4;
  static_assert(QT * NT % 128 == 0, "whole combine blocks per attention block");
  const int slot = (int)(blockIdx.x % CB) * 128 + (int)threadIdx.x, t = slot / NT, tid = slot % NT;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4;
  const int tile = blockIdx.x / CB, b = blockIdx.y, d0 = blockIdx.z;
  const int nq = a.nh * a.S;
  const int wt = attn_wave_tile0(tile, nq, a.tiles) + wave * QT + t, qi = wt * 16 + (lane & 15);
  if (wt >= attn_wave_tile0(tile + 1, nq, a.tiles) || qi >= nq) return;
  const int qs = qi / a.nh, qn = qi - qs * a.nh;
  const float* P = a.partial + ((size_t)b * a.tiles + tile) * a.splits * (QT * NR * NT) + (size_t)t * NR * NT + tid;
  // splits in batches of ZC (4, 8 or 16, the smallest that covers the splits):
  // every load of a batch is issued before any is used (one memory round trip
  // per batch), and the running maximum carries over between batches; with
  // splits <= ZC this is the plain two-pass merge
  float m = -INFINITY, l = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  auto merge = [&](auto zc) {
    constexpr int ZC = decltype(zc)::value;
    for (int z0 = 0; z0 < a.splits; z0 += ZC) {
      float vm[ZC], vl[ZC], vo[ZC][4];
#pragma unroll
      for (int k = 0; k < ZC; ++k) {
        const float* pz = P + (size_t)min(z0 + k, a.splits - 1) * QT * NR * NT;
        vm[k] = pz[0];
        vl[k] = pz[NT];
        load4(reinterpret_cast<const T*>(pz - tid + 2 * NT) + ((size_t)d0 * NT + tid) * 4, vo[k]);
      }
      float mb = m;
#pragma unroll
      for (int k = 0; k < ZC; ++k)
        if (z0 + k < a.splits) mb = fmaxf(mb, vm[k]);
      const float s0 = (m == -INFINITY) ? 0.f : fexp2<T>(m - mb);
      l *= s0;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] *= s0;
#pragma unroll
      for (int k = 0; k < ZC; ++k) {
        if (z0 + k >= a.splits) continue;
        const float w = (vm[k] == -INFINITY) ? 0.f : fexp2<T>(vm[k] - mb);
        l += w * vl[k];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] += w * vo[k][e];
      }
      m = mb;
    }
  };
  if (a.splits <= 4) merge(std::integral_constant<int, 4>());
  else if (a.splits <= 8) merge(std::integral_constant<int, 8>());
  else merge(std::integral_constant<int, 16>());
  const float inv = l > 0.f ? 1.f / l : 0.f;
  T* orow = reinterpret_cast<T*>(a.out) + ((size_t)b * a.S + qs) * a.ldo + qn * DH;
#pragma unroll
  for (int e = 0; e < 4; ++e) orow[d0 * 16 + g * 4 + e] = from_f32<T>(o[e] * inv);
}

// Prefix values, transposed once per call: vt[l][b][d][vt_pos(key)] =
// V_l[b][key][d] for keys < valid_len[b], 0 for the rest (padded keys are not
// read).  64 keys x 64 features per block through LDS, 16 bytes per global
// access on both sides: key rows are read as vectors, and each output vector
// holds 8 (bf16) or 4 (float32) consecutive vt_pos positions of one feature,
// gathered from the LDS tile.  Lp is a multiple of 64, so a block's 64 keys
// are two whole vt_pos groups.
template <typename T>
__global__ __launch_bounds__(256) void transpose_v_kernel(const CallDesc* __restrict__ desc, int B, int L, int DH,
                                                          int Lp, T* __restrict__ vt) {
  constexpr int VE = 16 / (int)sizeof(T), KB = 64, DB = 64, LD = DB + VE;
  __shared__ __attribute__((aligned(16))) T tileb[KB * LD];
  const int k0 = blockIdx.x * KB, d0 = blockIdx.y * DB, lb = blockIdx.z;  // lb = layer * B + b
  const int layer = lb / B, b = lb - layer * B;
  int valid = desc->valid[b];
  valid = valid < 0 ? 0 : (valid > L ? L : valid);
  const T* src = reinterpret_cast<const T*>(desc->kv) + (((size_t)layer * 2 + 1) * B + b) * (size_t)L * DH;
  for (int i = threadIdx.x; i < KB * DB / VE; i += 256) {
    const int kk = i / (DB / VE), dv = (i % (DB / VE)) * VE, key = k0 + kk;
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (key < valid && d0 + dv < DH) x = gload16(src + (size_t)key * DH + d0 + dv);
    *reinterpret_cast<u32x4*>(&tileb[kk * LD + dv]) = x;
  }
  __syncthreads();
  T* dst = vt + ((size_t)lb * DH) * Lp + k0;
  for (int i = threadIdx.x; i < DB * KB / VE; i += 256) {
    const int dd = i / (KB / VE), p0 = (i % (KB / VE)) * VE;
    if (d0 + dd >= DH) continue;
    T v[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      // position p = 32 c + 8 g + 4 h + r holds key 32 c + 16 h + 4 g + r
      const int p = p0 + e;
      const int key = (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
      v[e] = tileb[key * LD + dd];
    }
    *reinterpret_cast<u32x4*>(dst + (size_t)(d0 + dd) * Lp + p0) = __builtin_bit_cast(u32x4, v);
  }
}

}  // namespace pi0x
