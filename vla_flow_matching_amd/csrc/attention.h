// Grouped-query attention of the expert's suffix over [cached prefix ; suffix]
// keys with the pi0 mask (page 1, _attend and make_att_2d_masks as used by
// denoise_step): every suffix query sees the valid prefix keys j < valid_len;
// inside the suffix the state token (s = 0) sees only itself and every action
// token (s >= 1) sees the state token and all action tokens.  One kv head is
// shared by all query heads, so the num_heads * S queries of a sample (query
// index qi = s*num_heads + n) form one matrix against one key/value sequence.
//
// Keys are visited in blocks of 32.  A wave computes S^T = K Q^T with the
// matrix cores, so a lane holds 8 scores of its own query (lane % 16); the
// online softmax runs in float32 in registers, and O^T = V^T P^T reuses those
// 8 probabilities directly as the MFMA operand.  V is read transposed
// ([head_dim][keys]): the prefix values are transposed once per call by
// transpose_v_kernel, the suffix values are written transposed by the q/k/v
// projection.  Masked keys get probability exactly 0; padded prefix keys are
// never read from the caller's cache (zeros are used instead).
//
// attn_kernel: 4 waves x 16 queries share each staged K / V^T block in LDS
// (large batches).  attn_small_kernel: 8 waves split the key blocks of the
// same 16 queries, load operands straight from L2, and merge their partial
// softmax states through LDS at the end (batch 1, where 64-query tiles would
// leave most of the chip idle).
#pragma once

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
};

// exp for the softmax: the hardware exp2 path in bf16 mode, libm expf in float32 mode.
template <typename T> __device__ __forceinline__ float fexp(float x) { return expf(x); }
template <> __device__ __forceinline__ float fexp<bf16>(float x) { return __expf(x); }

// Per-wave online-softmax state for 16 queries (lane % 16) and head_dim DH.
template <typename T, int DH>
struct SoftmaxState {
  static constexpr int ND = DH / 16;
  f32x4 o[ND];
  float m = -INFINITY, l = 0.f;  // running max (same on the 4 lanes of a query), this lane's share of the sum
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // st[kt][e]: score of this lane's query vs key kt*16 + 4g + e of the block (already masked to -inf).
  // Returns the probabilities as the PV operand (key order (e/4)*16 + 4g + e%4).
  __device__ __forceinline__ Frag<T> update(const float (&s)[8]) {
    float bmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) bmax = fmaxf(bmax, s[i]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float m_new = fmaxf(m, bmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : fexp<T>(m - m_new);
    Frag<T> pf;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = (s[i] == -INFINITY) ? 0.f : fexp<T>(s[i] - m_new);
      l += e;
      set_frag(pf, i, e);
    }
    m = m_new;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      o[d][0] *= alpha; o[d][1] *= alpha; o[d][2] *= alpha; o[d][3] *= alpha;
    }
    return pf;
  }
};

// Scores of one 32-key block, masked: keys >= lim do not exist; in the suffix
// (pre == false) the state query (qs == 0) only sees key 0.
__device__ __forceinline__ void mask_scores(const f32x4 (&st)[2], float scale, int base, int lim, bool pre, int qs,
                                            int g, float (&s)[8]) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = base + kt * 16 + g * 4 + e;
      bool vis = key < lim;
      if (!pre) vis = vis && (qs >= 1 || key == 0);
      s[kt * 4 + e] = vis ? st[kt][e] * scale : -INFINITY;
    }
}

template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int KB = 32;
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int LDK = DH + VE;  // padded K row
  constexpr int LDV = KB + VE;  // padded V^T row
  constexpr int NC = DH / 32, ND = DH / 16;
  __shared__ __attribute__((aligned(16))) T Ks[KB * LDK];
  __shared__ __attribute__((aligned(16))) T Vt[DH * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4;
  const int tile = blockIdx.x, b = blockIdx.y;
  const int nq = a.nh * a.S;
  const int qi = tile * 64 + wave * 16 + (lane & 15);
  const bool qok = qi < nq;
  const int qs = qok ? qi / a.nh : 0, qn = qok ? qi - qs * a.nh : 0;

  int valid = a.desc->valid[b];
  valid = valid < 0 ? 0 : (valid > a.L ? a.L : valid);
  const T* __restrict__ qk = reinterpret_cast<const T*>(a.qk);
  const T* Kp = reinterpret_cast<const T*>(a.desc->kv) + a.kv_k_off + (size_t)b * a.L * DH;
  const T* Vtp = reinterpret_cast<const T*>(a.vtp) + (size_t)b * DH * a.Lp;
  const T* Vts = reinterpret_cast<const T*>(a.vts) + (size_t)b * DH * a.Sp;
  const T* Sq = qk + (size_t)b * a.S * a.ldqk;

  Frag<T> qf[NC];
  {
    const T* qrow = Sq + (size_t)qs * a.ldqk + qn * DH;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (qok) load8(qf[c], qrow + c * 32 + g * 8);
      else
#pragma unroll
        for (int i = 0; i < 8; ++i) set_frag(qf[c], i, 0.f);
    }
  }
  const int nb_pre = (valid + KB - 1) / KB, nb_suf = (a.S + KB - 1) / KB;
  SoftmaxState<T, DH> sm;
  sm.init();

  for (int blk = 0; blk < nb_pre + nb_suf; ++blk) {
    const bool pre = blk < nb_pre;
    const int base = pre ? blk * KB : (blk - nb_pre) * KB;
    const int lim = pre ? valid : a.S;
    constexpr int KVPR = DH / VE;  // 16-byte vectors per K row
#pragma unroll
    for (int it = 0; it < (KB * KVPR + 255) / 256; ++it) {
      const int v = tid + it * 256;
      if (v < KB * KVPR) {
        const int kk = v / KVPR, dc = v - kk * KVPR, key = base + kk;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (key < lim) {
          const T* src = pre ? Kp + (size_t)key * DH : Sq + (size_t)key * a.ldqk + a.col_k;
          val = *reinterpret_cast<const uint4*>(src + dc * VE);
        }
        *reinterpret_cast<uint4*>(&Ks[kk * LDK + dc * VE]) = val;
      }
    }
    constexpr int VPR = KB / VE;  // 16-byte vectors per V^T row of the block
#pragma unroll
    for (int it = 0; it < (DH * VPR + 255) / 256; ++it) {
      const int v = tid + it * 256;
      if (v < DH * VPR) {
        const int d = v / VPR, kc = (v - d * VPR) * VE;
        const T* src = pre ? Vtp + (size_t)d * a.Lp + base + kc : Vts + (size_t)d * a.Sp + base + kc;
        *reinterpret_cast<uint4*>(&Vt[d * LDV + kc]) = *reinterpret_cast<const uint4*>(src);
      }
    }
    __syncthreads();

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
    float s[8];
    mask_scores(st, a.scale, base, lim, pre, qs, g, s);
    const Frag<T> pf = sm.update(s);
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      Frag<T> vf;
      const T* vrow = &Vt[(d * 16 + (lane & 15)) * LDV];
      load4x2(vf, vrow + g * 4, vrow + 16 + g * 4);
      mma32(vf, pf, sm.o[d]);
    }
    __syncthreads();
  }

  float l_tot = sm.l + __shfl_xor(sm.l, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (!qok) return;
  const float inv = 1.f / l_tot;
  T* orow = reinterpret_cast<T*>(a.out) + ((size_t)b * a.S + qs) * a.ldo + qn * DH;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[d * 16 + g * 4 + e] = from_f32<T>(sm.o[d][e] * inv);
}

template <typename T, int DH>
__global__ __launch_bounds__(512) void attn_small_kernel(AttnArgs a) {
  constexpr int KB = 32, NW = 8;
  constexpr int NC = DH / 32, ND = DH / 16;
  constexpr int NR = 2 + ND * 4;  // floats per lane in the merge buffer
  __shared__ float red[NW * 64 * NR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4;
  const int tile = blockIdx.x, b = blockIdx.y;
  const int nq = a.nh * a.S;
  const int qi = tile * 16 + (lane & 15);
  const bool qok = qi < nq;
  const int qs = qok ? qi / a.nh : 0, qn = qok ? qi - qs * a.nh : 0;

  int valid = a.desc->valid[b];
  valid = valid < 0 ? 0 : (valid > a.L ? a.L : valid);
  const T* __restrict__ qk = reinterpret_cast<const T*>(a.qk);
  const T* Kp = reinterpret_cast<const T*>(a.desc->kv) + a.kv_k_off + (size_t)b * a.L * DH;
  const T* Vtp = reinterpret_cast<const T*>(a.vtp) + (size_t)b * DH * a.Lp;
  const T* Vts = reinterpret_cast<const T*>(a.vts) + (size_t)b * DH * a.Sp;
  const T* Sq = qk + (size_t)b * a.S * a.ldqk;

  Frag<T> qf[NC];
  {
    const T* qrow = Sq + (size_t)qs * a.ldqk + qn * DH;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (qok) load8(qf[c], qrow + c * 32 + g * 8);
      else
#pragma unroll
        for (int i = 0; i < 8; ++i) set_frag(qf[c], i, 0.f);
    }
  }
  const int nb_pre = (valid + KB - 1) / KB, nb_suf = (a.S + KB - 1) / KB;
  SoftmaxState<T, DH> sm;
  sm.init();

  for (int blk = wave; blk < nb_pre + nb_suf; blk += NW) {
    const bool pre = blk < nb_pre;
    const int base = pre ? blk * KB : (blk - nb_pre) * KB;
    const int lim = pre ? valid : a.S;
    f32x4 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = base + kt * 16 + (lane & 15);
      const bool kok = key < lim;
      const T* krow = pre ? Kp + (size_t)key * DH : Sq + (size_t)key * a.ldqk + a.col_k;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        Frag<T> kf;
        if (kok) load8(kf, krow + c * 32 + g * 8);
        else
#pragma unroll
          for (int i = 0; i < 8; ++i) set_frag(kf, i, 0.f);
        mma32(kf, qf[c], st[kt]);
      }
    }
    float s[8];
    mask_scores(st, a.scale, base, lim, pre, qs, g, s);
    const Frag<T> pf = sm.update(s);
    const T* vbase = pre ? Vtp + base : Vts + base;
    const int vld = pre ? a.Lp : a.Sp;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      Frag<T> vf;
      const T* vrow = vbase + (size_t)(d * 16 + (lane & 15)) * vld;
      load4x2(vf, vrow + g * 4, vrow + 16 + g * 4);
      mma32(vf, pf, sm.o[d]);
    }
  }

  // merge the 8 waves' states: lane layout (q = lane % 16, g = lane / 16), O^T element d*16 + 4g + e
  float* mine = red + (wave * 64 + lane) * NR;
  mine[0] = sm.m;
  mine[1] = sm.l;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int e = 0; e < 4; ++e) mine[2 + d * 4 + e] = sm.o[d][e];
  __syncthreads();
  const int ln = tid & 63, q = ln & 15;
  const int qi2 = tile * 16 + q;
  if (qi2 >= nq) return;
  const int qs2 = qi2 / a.nh, qn2 = qi2 - qs2 * a.nh;
  float mz = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) mz = fmaxf(mz, red[(w * 64 + ln) * NR]);
  float wt[NW], lsum = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float mw = red[(w * 64 + ln) * NR];
    wt[w] = (mw == -INFINITY) ? 0.f : fexp<T>(mw - mz);
    float lw = 0.f;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) lw += red[(w * 64 + gg * 16 + q) * NR + 1];
    lsum += wt[w] * lw;
  }
  const float inv = 1.f / lsum;
  T* orow = reinterpret_cast<T*>(a.out) + ((size_t)b * a.S + qs2) * a.ldo + qn2 * DH;
  const int g2 = ln >> 4;
  for (int d = tid >> 6; d < ND; d += NW)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) acc += wt[w] * red[(w * 64 + ln) * NR + 2 + d * 4 + e];
      orow[d * 16 + g2 * 4 + e] = from_f32<T>(acc * inv);
    }
}

// Prefix values, transposed once per call: vt[l][b][d][Lp] = V_l[b][key][d] for
// keys < valid_len[b], 0 for the rest (padded keys are not read).  32 keys x 64
// features per block through LDS.
template <typename T>
__global__ __launch_bounds__(256) void transpose_v_kernel(const CallDesc* __restrict__ desc, int B, int L, int DH,
                                                          int Lp, T* __restrict__ vt) {
  __shared__ T tileb[32][64 + 1];
  const int k0 = blockIdx.x * 32, d0 = blockIdx.y * 64, lb = blockIdx.z;  // lb = layer * B + b
  const int layer = lb / B, b = lb - layer * B;
  int valid = desc->valid[b];
  valid = valid < 0 ? 0 : (valid > L ? L : valid);
  const T* src = reinterpret_cast<const T*>(desc->kv) + (((size_t)layer * 2 + 1) * B + b) * (size_t)L * DH;
  for (int i = threadIdx.x; i < 32 * 64; i += 256) {
    const int kk = i / 64, dd = i % 64, key = k0 + kk;
    tileb[kk][dd] = (key < valid && d0 + dd < DH) ? src[(size_t)key * DH + d0 + dd] : from_f32<T>(0.f);
  }
  __syncthreads();
  T* dst = vt + ((size_t)lb * DH) * Lp;
  for (int i = threadIdx.x; i < 32 * 64; i += 256) {
    const int dd = i / 32, kk = i % 32;
    if (d0 + dd < DH) dst[(size_t)(d0 + dd) * Lp + k0 + kk] = tileb[kk][dd];
  }
}

}  // namespace pi0x
