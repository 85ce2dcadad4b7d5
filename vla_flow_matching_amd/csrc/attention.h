// Grouped-query attention of the expert's suffix over [cached prefix ; suffix]
// keys with the pi0 mask (page 1, _attend and make_att_2d_masks as used by
// denoise_step): every suffix query sees the valid prefix keys j < valid_len;
// inside the suffix the state token (s = 0) sees only itself and every action
// token (s >= 1) sees the state token and all action tokens.  One kv head is
// shared by all query heads, so the num_heads * S queries of a sample form one
// [num_heads*S][head_dim] matrix against a single key/value sequence.
//
// Block = 4 waves = 64 queries (query index qi = s*num_heads + n), grid
// (query tiles, batch, key splits).  Keys are visited in blocks of 32: a block
// of K (row-major) and V (transposed) is staged in LDS once and used by all 4
// waves.  Each wave computes S^T = K Q^T with the matrix cores, so a lane holds
// 8 scores of its own query (lane % 16); the online softmax runs in float32
// entirely in registers, and O^T = V^T P^T reuses those 8 probabilities as the
// MFMA operand directly (no transpose through LDS).  Masked keys are skipped
// exactly: padded prefix keys are never loaded (zeros are staged) and their
// probabilities are exactly 0.
//
// With splits > 1 the key blocks of a sample are divided over gridDim.z; every
// split writes (running max, running sum, unnormalised O) and the last split
// to arrive merges them in split order.
#pragma once

#include "common.h"

namespace pi0x {

struct AttnArgs {
  const void* qkv;   // [B*S][ldqkv]: q heads at column 0, k at qk_k, v at qk_v
  int ldqkv, col_k, col_v;
  const CallDesc* desc;
  size_t kv_k_off, kv_v_off;  // element offsets of this layer's K and V blocks inside desc->kv
  int B, L, S, nh;
  void* out;  // [B*S][ldo], head n of token s at column n*head_dim
  int ldo;
  float scale;
  int splits;
  float* partial;      // splits > 1: [B*tiles][splits][(2 + DH/4) * 256]
  unsigned* counters;  // splits > 1: [B*tiles]
};

// exp for the softmax: the hardware exp2 path in bf16 mode, the accurate
// libm expf in float32 mode.
template <typename T> __device__ __forceinline__ float fexp(float x) { return expf(x); }
template <> __device__ __forceinline__ float fexp<bf16>(float x) { return __expf(x); }

template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int KB = 32;                  // keys per block
  constexpr int VE = 16 / (int)sizeof(T);  // elements per 16-byte vector
  constexpr int LDK = DH + VE;             // padded K row
  constexpr int LDV = KB + VE;             // padded V^T row
  constexpr int NC = DH / 32;              // 32-wide chunks of head_dim
  constexpr int ND = DH / 16;              // 16-wide output tiles of head_dim
  __shared__ __attribute__((aligned(16))) T Ks[KB * LDK];
  __shared__ __attribute__((aligned(16))) T Vt[DH * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int nq = a.nh * a.S;
  const int qi = tile * 64 + wave * 16 + (lane & 15);
  const bool qok = qi < nq;
  const int qs = qok ? qi / a.nh : 0, qn = qok ? qi - qs * a.nh : 0;
  const int g = lane >> 4;

  int valid = a.desc->valid[b];
  valid = valid < 0 ? 0 : (valid > a.L ? a.L : valid);
  const T* __restrict__ qkv = reinterpret_cast<const T*>(a.qkv);
  const T* __restrict__ kvb = reinterpret_cast<const T*>(a.desc->kv);
  const T* Kp = kvb + a.kv_k_off + (size_t)b * a.L * DH;
  const T* Vp = kvb + a.kv_v_off + (size_t)b * a.L * DH;
  const T* Sbase = qkv + (size_t)b * a.S * a.ldqkv;

  // this lane's query: 8 elements per 32-wide chunk, for the S^T = K Q^T operand
  Frag<T> qf[NC];
  {
    const T* qrow = Sbase + (size_t)qs * a.ldqkv + qn * DH;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (qok) load8(qf[c], qrow + c * 32 + g * 8);
      else
#pragma unroll
        for (int i = 0; i < 8; ++i) set_frag(qf[c], i, 0.f);
    }
  }

  const int nb_pre = (valid + KB - 1) / KB, nb_suf = (a.S + KB - 1) / KB;
  const int nblk = nb_pre + nb_suf;
  const int blk_b = (int)((long)split * nblk / a.splits), blk_e = (int)((long)(split + 1) * nblk / a.splits);

  f32x4 o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  for (int blk = blk_b; blk < blk_e; ++blk) {
    const bool pre = blk < nb_pre;
    const int base = pre ? blk * KB : (blk - nb_pre) * KB;  // first key of the block
    const int lim = pre ? valid : a.S;                        // keys >= lim do not exist
    // ---- stage K (row-major) and V^T ----
    constexpr int VPR = DH / VE;  // vectors per key row
#pragma unroll
    for (int it = 0; it < (KB * VPR + 255) / 256; ++it) {
      const int v = tid + it * 256;
      if (v < KB * VPR) {
        // K: chunk index fastest -> coalesced global reads, contiguous LDS rows
        const int kk = v / VPR, dc = v - kk * VPR;
        const int key = base + kk;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (key < lim) {
          const T* src = pre ? Kp + (size_t)key * DH : Sbase + (size_t)key * a.ldqkv + a.col_k;
          val = *reinterpret_cast<const uint4*>(src + dc * VE);
        }
        *reinterpret_cast<uint4*>(&Ks[kk * LDK + dc * VE]) = val;
        // V: key index fastest -> conflict-free transposed LDS writes
        const int kv2 = v % KB, dc2 = v / KB;
        const int key2 = base + kv2;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (key2 < lim) {
          const T* src = pre ? Vp + (size_t)key2 * DH : Sbase + (size_t)key2 * a.ldqkv + a.col_v;
          w = *reinterpret_cast<const uint4*>(src + dc2 * VE);
        }
        const T* wv = reinterpret_cast<const T*>(&w);
#pragma unroll
        for (int i = 0; i < VE; ++i) Vt[(dc2 * VE + i) * LDV + kv2] = wv[i];
      }
    }
    __syncthreads();

    // ---- scores: S^T tiles for keys 0..15 and 16..31 of the block ----
    f32x4 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        Frag<T> kf;
        load8(kf, &Ks[(kt * 16 + (lane & 15)) * LDK + c * 32 + g * 8]);
        mma32(kf, qf[c], st[kt]);
      }
    }
    // lane holds score of its query vs key kt*16 + 4g + e
    float p[8];
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = base + kt * 16 + g * 4 + e;
        bool vis = key < lim;
        if (!pre) vis = vis && (qs >= 1 || key == 0);
        const float s = vis ? st[kt][e] * a.scale : -INFINITY;
        p[kt * 4 + e] = s;
        bmax = fmaxf(bmax, s);
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float m_new = fmaxf(m_run, bmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : fexp<T>(m_run - m_new);
    Frag<T> pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = (p[i] == -INFINITY) ? 0.f : fexp<T>(p[i] - m_new);
      l_part = (i == 0 ? l_part * alpha : l_part) + e;
      set_frag(pf, i, e);
    }
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      o[d][0] *= alpha; o[d][1] *= alpha; o[d][2] *= alpha; o[d][3] *= alpha;
      Frag<T> vf;
      const T* vrow = &Vt[(d * 16 + (lane & 15)) * LDV];
      load4x2(vf, vrow + g * 4, vrow + 16 + g * 4);
      mma32(vf, pf, o[d]);
    }
    __syncthreads();
  }

  // lane holds O[q][d*16 + 4g + e] (unnormalised); total softmax denominator
  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (blk_b >= blk_e) { m_run = -INFINITY; l_tot = 0.f; }

  if (a.splits > 1) {
    constexpr int NR = 2 + ND * 4;
    const int wt = b * gridDim.x + tile;
    float* P = a.partial + (size_t)wt * a.splits * NR * 256;
    float* mine = P + (size_t)split * NR * 256;
    mine[tid] = m_run;
    mine[256 + tid] = l_tot;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int e = 0; e < 4; ++e) mine[(2 + d * 4 + e) * 256 + tid] = o[d][e];
    if (!arrive_last(&a.counters[wt], (unsigned)a.splits, tid)) return;
    float mz = -INFINITY;
    for (int z = 0; z < a.splits; ++z) mz = fmaxf(mz, P[(size_t)z * NR * 256 + tid]);
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_tot = 0.f;
    for (int z = 0; z < a.splits; ++z) {
      const float* pz = P + (size_t)z * NR * 256;
      const float mzz = pz[tid];
      const float w = (mzz == -INFINITY) ? 0.f : fexp<T>(mzz - mz);
      l_tot += w * pz[256 + tid];
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[d][e] += w * pz[(2 + d * 4 + e) * 256 + tid];
    }
    if (tid == 0) a.counters[wt] = 0u;
  }

  if (!qok) return;
  const float inv = 1.f / l_tot;
  T* orow = reinterpret_cast<T*>(a.out) + ((size_t)b * a.S + qs) * a.ldo + qn * DH;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[d * 16 + g * 4 + e] = from_f32<T>(o[d][e] * inv);
}

}  // namespace pi0x
