// The expert's 18-layer stack at batch 1 (page 1, _compute_layer_suffix_only
// for every layer of one denoise_step) as one persistent dataflow kernel per
// Euler step.
//
// At batch 1 the stack is weight-streaming: 51 suffix rows against 629 MB of
// weights per step.  Launching one kernel per dependent step costs a graph
// dependency (about 2-4 us) eight times per layer.  Here one launch covers all
// layers: the grid holds one block per CU, every block owns a fixed unit of
// each phase, and a unit starts as soon as the units it reads from have
// published their results -- no grid-wide barrier.
//
// Phases of one layer, with their units (W = 1024, M = 4096, 8 heads of 256):
//   Q  q/k/v + RoPE (input norm's 1/rms as a row scale): 80 units of 32
//      stored columns over the whole K, RoPE partners in one lane.
//   A  attention: (key block of 64, query tile of 64) units; each writes its
//      unnormalised output (16-byte rows: features 16 d + 4 g .. +3 of d-tiles
//      2 dp and 2 dp + 1 at element 32 dp + 8 g), running max and sum.  The
//      last key block is the suffix.
//   X  merge of the key-block partials: (query tile, 16 features) units.
//   C  o_proj: (32 output columns, one head's 256 inputs) units write
//      float32 partials; the last of the 8 units of a column group adds them
//      in head order to the residual stream (h, its bf16 copy, the rows'
//      sum-of-squares partials per 32 columns).
//   G  gate/up + GeGLU (post norm's 1/rms as a row scale): 256 units of 16
//      hidden features.
//   D  down: (32 output columns, 512 inputs) units, float32 partials, the
//      last of a column group's 8 units adds them to the residual stream.
//
// Dependencies are device-scope counters (one 128-byte line each), bumped
// once per finished unit after its stores completed and polled by the units
// that read its data.  Counters only grow within a call (zeroed before the
// first step), so a unit of layer e waits for (e + 1) x units-per-layer.
// Data that crosses blocks is written and read with agent-coherent (sc1)
// buffer accesses, so no cache writeback or invalidate is needed; the
// producer waits for its stores to complete before bumping the counter.
//
// Block roles.  Waves 0-3 compute; each owns 16 of the 64 (padded) rows of a
// unit, so no cross-wave reduction is needed.  Wave 4 streams every unit's
// weights (and the attention units' prefix key/value block) into a 152 KB
// LDS ring of 1 KB blocks (152 KB), as far ahead as the ring allows, with
// global_load_lds; its loads never sit in front of a compute wave's
// dependency polls or activation loads (vector memory returns in order per
// wave).  Ring blocks hold MFMA fragments: 64 lanes x 16 bytes, lane l the
// bf16x8 of row l % 16, reduction elements 8 (l / 16) .. +7 of a 32-wide step,
// so a compute wave reads a fragment with one conflict-free ds_read_b128.
//
// Every wait is bounded.  A wait that times out (a block that never
// arrives: the grid was not co-resident) sets an abort word in the counter
// buffer, fills the residual stream with NaN and returns; every later wait of
// the call sees the abort word and returns at once.
#pragma once

#include "common.h"

namespace pi0x {

constexpr int kB1Compute = 4;                 // compute waves
constexpr int kB1Threads = (kB1Compute + 1) * 64;
constexpr int kB1Ring = 152;                  // 1 KB blocks in the LDS ring
constexpr int kB1Spin = 1 << 22;              // polls before a wait gives up
constexpr int kB1MaxTiles = 8;                // attention query tiles of 64
constexpr int kB1MaxGroups = 64;              // 32-column groups of the width
constexpr int kB1MaxSlices = 16;              // 512-wide slices of the MLP (counter slots)
constexpr int kB1MaxParts = 8;                // K-slice partials per residual column group
constexpr int kB1MaxSplits = 24;              // attention key blocks (prefix blocks + the suffix block)
constexpr int kB1Inflight = 32;               // loader DMA blocks in flight before it waits

// counter indices (each on its own 128-byte line: index * 32 words)
enum : int {
  kCntQ = 0,
  kCntA = 1,                                  // + tile
  kCntX = kCntA + kB1MaxTiles,
  kCntC = kCntX + 1,                          // + column group
  kCntR1 = kCntC + kB1MaxGroups,
  kCntG = kCntR1 + 1,                         // + MLP slice
  kCntD = kCntG + kB1MaxSlices,               // + column group
  kCntR2 = kCntD + kB1MaxGroups,
  kCntAbort = kCntR2 + 1,
  kB1Counters = kCntAbort + 1
};
// Counters that many blocks poll exist in kB1Rep replicas on separate lines
// (replica r at word r * kB1RepStride, the stride off a power of two so the
// replicas spread over memory channels): a producer bumps every replica with
// one instruction, a block polls replica b % kB1Rep.  One hot line polled by
// every block otherwise slows every access that maps to its memory channel.
constexpr int kB1Rep = 16;
constexpr size_t kB1RepStride = (size_t)kB1Counters * 32 + 32;
constexpr size_t kB1CounterWords = kB1Rep * kB1RepStride;

struct B1Args {
  const bf16* const* lw;  // [D][4]: wqkv, wo, wgu, wdown of each layer in fragment order (b1_pack_weights_kernel)
  int D, W, M, nh, S, qd, nqkv;
  const CallDesc* desc;   // prefix K/V cache and valid length
  int L, Lp;              // padded prefix length, its 64-multiple
  const bf16* kvf;        // [D][L/64 blocks][64][512] prefix keys/values of the call in fragment order (b1_pack_kv_kernel)
  bf16* qk;               // [S][qd + 256] rotated q heads, then the rotated k
  bf16* vts;              // [256][64] suffix values transposed (vt_pos order), zero beyond S
  const float2* rope_cs;  // [S][128] (cos, sin) of every suffix row
  float* hbuf;            // [S][W] residual stream
  bf16* hb;               // [S][W] its bf16 copy
  float* ssq;             // [S][...] sum-of-squares partials of the residual rows
  int np0;                // partials per row the first layer reads (the suffix embedding's)
  bf16* o;                // [S][qd] attention output
  bf16* g;                // [S][M] GeGLU output
  float* apart;           // attention partials: [nsplit][ntile][2][64] float, then bf16 [nsplit][ntile][64][256]
  float* cpart;           // [qd/256][S][W]
  float* dpart;           // [M/512][S][W]
  unsigned* cnt;          // kB1CounterWords, zero before the first step of the call
  int step;               // Euler step of this launch
  int nsplit, ntile;      // key blocks (prefix blocks + 1 suffix block), query tiles of 64
  int causal;
  float scale;    // 1 / sqrt(head_dim)
  float rms_eps;
  unsigned long long* trace;  // kernel instantiated with tracing: [block][layer][9][4] wall-clock stamps (step 0)
};

// ---------------------------------------------------------------------------
// agent-coherent (sc1) accesses for data that crosses blocks
// ---------------------------------------------------------------------------
constexpr int kSc1 = 16;  // cache-policy bit of the buffer intrinsics: sc1 (device scope)

// A value the compiler cannot see through: descriptors and addresses built from
// it stay inside the phase that uses them instead of being hoisted out of the
// layer loop and kept live (in registers) across every phase.
template <class P>
__device__ __forceinline__ P opq(P p) {
  asm volatile("" : "+s"(p));
  return p;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t b1_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(opq(p)), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ u32x4 ld16c(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}
__device__ __forceinline__ float ld4c(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSc1));
}
__device__ __forceinline__ void st16c(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((__vector_size__(16))) unsigned, v), r,
                                         off, 0, kSc1);
}
__device__ __forceinline__ void st8c(__amdgpu_buffer_rsrc_t r, uint32_t off, uint64_t v) {
  typedef unsigned u2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, v), r, off, 0, kSc1);
}
__device__ __forceinline__ void st4c(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, off, 0, kSc1);
}
__device__ __forceinline__ void st2c(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16 v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, off, 0, kSc1);
}

__device__ __forceinline__ unsigned cnt_load(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Completion of a unit: every replica of counter c gains one (lanes 0 ..
// kB1Rep-1 of the calling wave, one instruction).
__device__ __forceinline__ void b1_signal(unsigned* cnt, int c, int lane) {
  if (lane < kB1Rep)
    __hip_atomic_fetch_add(cnt + (size_t)lane * kB1RepStride + (size_t)c * 32, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// LDS words shared by the waves of a block
struct B1Shared {
  unsigned loaded;        // ring blocks the loader has landed (monotonic)
  unsigned consumed[kB1Compute];  // ring blocks each compute wave is done with
  unsigned bar;           // compute-wave barrier arrivals
  unsigned bcast;         // (generation << 1) | last-arriver flag
  unsigned go;            // dependency waits wave 0 has seen met (the other waves wait on it)
  unsigned abort;
};

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt at their maxima)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ unsigned lds_ld(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Polls until counter c reaches target (all lanes of the wave load the same
// word).  false: the call was aborted (now or by another block).
__device__ __forceinline__ bool b1_poll(const B1Args& a, int c, unsigned target, B1Shared* sh) {
  const unsigned* p = a.cnt + (size_t)(blockIdx.x % kB1Rep) * kB1RepStride + (size_t)c * 32;
  const unsigned* ab = a.cnt + (size_t)kCntAbort * 32;
  if (cnt_load(p) >= target) return true;
  for (int i = 0; i < kB1Spin; ++i) {
    __builtin_amdgcn_s_sleep(2);
    if (cnt_load(p) >= target) return true;
    if ((i & 31) == 31 && (cnt_load(ab) != 0u || lds_ld(&sh->abort) != 0u)) {
      lds_st(&sh->abort, 1u);
      return false;
    }
  }
  __hip_atomic_store(a.cnt + (size_t)kCntAbort * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  lds_st(&sh->abort, 1u);
  return false;
}

// LDS wait used by the compute waves for the loader and each other
__device__ __forceinline__ bool b1_lds_wait(const unsigned* p, unsigned target, B1Shared* sh) {
  for (int i = 0; i < kB1Spin; ++i) {
    if (lds_ld(p) >= target) return true;
    if (lds_ld(&sh->abort) != 0u) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  lds_st(&sh->abort, 1u);
  return false;
}

// ---------------------------------------------------------------------------
// Work assignment, shared by the loader and the compute waves
// ---------------------------------------------------------------------------
struct B1Plan {
  int nQ, nA, nX, nC, nG, nD;
  int ngrp;     // 32-column groups of the width
  int nhs;      // 256-wide o_proj input slices (heads)
  int nms;      // 512-wide down input slices
};

__device__ __forceinline__ B1Plan b1_plan(const B1Args& a) {
  B1Plan p;
  p.ngrp = a.W / 32;
  p.nhs = a.qd / 256;
  p.nms = a.M / 512;
  p.nQ = a.nqkv / 32;
  p.nA = a.nsplit * a.ntile;
  p.nX = a.ntile * 16;
  p.nC = p.ngrp * p.nhs;
  p.nG = 2 * a.M / 32;
  p.nD = p.ngrp * p.nms;
  return p;
}

// attention unit u -> (split, tile): the query tiles of one key block run on
// one XCD (blocks b, b + 8, ... share an XCD), so they share the block in L2
__device__ __forceinline__ void b1_attn_unit(const B1Args& a, int u, int& split, int& tile) {
  const int x = u % 8, r = u / 8;
  tile = r % a.ntile;
  split = x + 8 * (r / a.ntile);
}
__device__ __forceinline__ int b1_attn_units_span(const B1Args& a) {  // units to scan so every (split, tile) appears
  return 8 * a.ntile * ((a.nsplit + 7) / 8);
}

// First unit of block b in a phase whose units are laid out from block off
// onwards (wrapping): u = (b - off) mod nb, then u + nb, ...  The q/k/v units
// sit on the last blocks and the attention units on the first ones, so no
// block streams both 64 KB units in one layer (the LDS ring stays ahead).
__device__ __forceinline__ int b1_first(int b, int nb, int off) { return (b - off % nb + nb) % nb; }

// ring blocks each unit takes
constexpr int kBlkQ = 64, kBlkA = 64, kBlkC = 16, kBlkG = 64, kBlkD = 32;

__device__ __forceinline__ int b1_valid(const B1Args& a) {
  int v = a.desc->valid[0];
  return v < 0 ? 0 : (v > a.L ? a.L : v);
}

// ---------------------------------------------------------------------------
// Loader wave
// ---------------------------------------------------------------------------
// 16 bytes per lane from src into LDS at byte address lds + 16 lane
// (global_load_lds_dwordx4, counted by vmcnt).  Written as an asm statement:
// the compiler does not know it writes LDS, so it does not drain the DMA queue
// (vmcnt(0)) in front of the loader's own LDS control-word accesses, which
// never touch the ring.  No result register (the data goes to LDS); the
// loader orders the ring with explicit vmcnt waits before it publishes.
__device__ __forceinline__ void b1_dma16(const bf16* src, unsigned lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory", "m0");
}

struct B1Loader {
  bf16* ring;
  B1Shared* sh;
  unsigned issued = 0;   // ring index of the next block (monotonic)
  unsigned slot = 0;     // issued % kB1Ring
  unsigned limit = 0;    // blocks that may be issued before the ring is checked again
  int inflight = 0;      // DMA instructions not yet waited for
  bool ok = true;

  __device__ __forceinline__ void publish(unsigned n) {
    asm volatile("" ::: "memory");
    lds_st(&sh->loaded, n);
  }
  __device__ __forceinline__ void publish_all() {
    wait_vmcnt<0>();
    inflight = 0;
    publish(issued);
  }
  __device__ __forceinline__ unsigned min_consumed() const {
    unsigned m = lds_ld(&sh->consumed[0]);
#pragma unroll
    for (int w = 1; w < kB1Compute; ++w) m = min(m, lds_ld(&sh->consumed[w]));
    return m;
  }
  // refresh the issue limit from the compute waves' progress; waits while the
  // ring is full (after publishing everything in flight)
  __device__ __forceinline__ bool make_room() {
    limit = min_consumed() + kB1Ring;
    if (issued < limit) return true;
    publish_all();
    for (int i = 0; i < kB1Spin; ++i) {
      __builtin_amdgcn_s_sleep(1);
      limit = min_consumed() + kB1Ring;
      if (issued < limit) return true;
      if (lds_ld(&sh->abort) != 0u) return false;
    }
    lds_st(&sh->abort, 1u);
    return false;
  }
  // n consecutive 1 KB blocks starting at src (this lane's 16 bytes at src + 8 lane)
  __device__ __forceinline__ void run(const bf16* src, int n, int lane) {
    const unsigned lds0 = (unsigned)(uintptr_t)ring;
    src += lane * 8;
    for (int i = 0; i < n && ok; ++i) {
      if (issued >= limit && !make_room()) {
        ok = false;
        return;
      }
      b1_dma16(src + (size_t)i * 512, lds0 + slot * 1024u);
      ++issued;
      slot = (slot + 1 == (unsigned)kB1Ring) ? 0u : slot + 1;
      if (++inflight >= kB1Inflight) {
        wait_vmcnt<kB1Inflight / 2>();
        inflight = kB1Inflight / 2;
        publish(issued - kB1Inflight / 2);
      }
    }
  }
  // blocks the compute waves fill or leave empty
  __device__ __forceinline__ void skip(int n) {
    for (int i = 0; i < n && ok; ++i) {
      if (issued >= limit && !make_room()) {
        ok = false;
        return;
      }
      ++issued;
      slot = (slot + 1 == (unsigned)kB1Ring) ? 0u : slot + 1;
    }
    if (ok) publish_all();
  }
  // weight tile u (32 rows) of a fragment-ordered [N][ld] matrix, columns
  // [k0, k0 + K): blocks (j, s) = (16-row half, 32-wide step), j major; each
  // half is K / 32 consecutive 1 KB blocks in memory
  __device__ __forceinline__ void weights(const bf16* wf, int ld, int u, int k0, int K, int lane) {
    const int steps = ld / 32;
    for (int j = 0; j < 2; ++j) run(wf + ((size_t)(2 * u + j) * steps + k0 / 32) * 512, K / 32, lane);
  }
};

// ---------------------------------------------------------------------------
// Compute-wave helpers
// ---------------------------------------------------------------------------
struct B1Wave {
  B1Shared* sh;
  const bf16* ring;
  int wave, lane;
  unsigned ring_pos = 0;   // ring index of the current unit's first block
  unsigned bar_gen = 0;
  unsigned wait_gen = 0;

  // dependency wait: only wave 0 polls device memory (fewer pollers on the
  // counters' lines, which the producers' atomics also need), the other
  // compute waves wait for its word in LDS
  __device__ __forceinline__ bool wait(const B1Args& a, int c, unsigned target) {
    ++wait_gen;
    if (wave == 0) {
      if (!b1_poll(a, c, target, sh)) return false;
      if (lane == 0) lds_st(&sh->go, wait_gen);
      return true;
    }
    return b1_lds_wait(&sh->go, wait_gen, sh);
  }

  __device__ __forceinline__ bool await_ring(int nblk) {
    return b1_lds_wait(&sh->loaded, ring_pos + (unsigned)nblk, sh);
  }
  __device__ __forceinline__ void release_ring(int nblk) {
    ring_pos += (unsigned)nblk;
    asm volatile("" ::: "memory");
    wait_lgkm0();  // this wave's ring reads are done
    lds_st(&sh->consumed[wave], ring_pos);
  }
  __device__ __forceinline__ bf16x8 frag(int blk) const {  // block blk of the current unit, this lane's 16 bytes
    return *reinterpret_cast<const bf16x8*>(ring + (size_t)((ring_pos + (unsigned)blk) % kB1Ring) * 512 + lane * 8);
  }
  __device__ __forceinline__ bf16* frag_w(int blk) const {
    return const_cast<bf16*>(ring) + (size_t)((ring_pos + (unsigned)blk) % kB1Ring) * 512 + lane * 8;
  }
  // all compute waves arrive (after their stores completed); returns false on abort
  __device__ __forceinline__ bool arrive_all() {
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    ++bar_gen;
    if (lane == 0) __hip_atomic_fetch_add(&sh->bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return b1_lds_wait(&sh->bar, bar_gen * kB1Compute, sh);
  }
};

// inv_rms of the 16 rows of this wave, for the row r = 4 (lane/16) + e it holds
// in the MFMA output layout: lane l sums quarter l % 4 of row l / 4's partials.
// Split in two so the partials' loads go out with the activation loads and
// are consumed after the MFMAs: b1_ssq_issue loads this lane's share (np / 4
// <= 8 partials), b1_inv_rms finishes.
struct B1Ssq {
  float v[8];
};
__device__ __forceinline__ B1Ssq b1_ssq_issue(const B1Args& a, int np, int row0, int lane) {
  const int r = row0 + (lane >> 2), q = lane & 3, per = np / 4;
  B1Ssq t;
  const auto rs = b1_rsrc(a.ssq);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    t.v[i] = (i < per && r < a.S) ? ld4c(rs, (uint32_t)(((size_t)r * np + q * per + i) * 4)) : 0.f;
  return t;
}
__device__ __forceinline__ void b1_inv_rms(const B1Args& a, const B1Ssq& t, int lane, float inv[4]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += t.v[i];
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  const float v = 1.0f / sqrtf(s / (float)a.W + a.rms_eps);
#pragma unroll
  for (int e = 0; e < 4; ++e) inv[e] = __shfl(v, (4 * (lane >> 4) + e) * 4, 64);
}

// 16 rows x K of a bf16 [S][ld] activation (columns k0 ..) as MFMA A fragments,
// rows >= S zero: frag s = row row0 + lane % 16, elements 32 s + 8 (lane/16) ..
template <int KS>
__device__ __forceinline__ void b1_load_a(const bf16* src, int ld, int k0, int row0, int S, int lane, bf16x8 (&af)[KS]) {
  const int r = row0 + (lane & 15);
  const auto rs = b1_rsrc(src);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (r < S) af[s] = __builtin_bit_cast(bf16x8, ld16c(rs, (uint32_t)(((size_t)r * ld + k0 + s * 32 + (lane >> 4) * 8) * 2)));
    else af[s] = bf16x8{};
  }
}

// 16 rows x 32 columns: acc[j] += A (KS steps) x ring blocks (j, s) of the unit
template <int KS>
__device__ __forceinline__ void b1_mma(const B1Wave& w, const bf16x8 (&af)[KS], f32x4 acc[2]) {
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const bf16x8 b0 = w.frag(s), b1 = w.frag(KS + s);
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], b0, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], b1, acc[1], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Residual reduction of one 32-column group (the last K-slice unit to arrive):
// h[row][cols] += sum over slices of part[slice][row][cols] in slice order;
// writes h, its bf16 copy and the rows' sum of squares over the group.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void b1_reduce_group(const B1Args& a, const float* part, int nslice, int grp, int tid) {
  const auto rp = b1_rsrc(part), rh = b1_rsrc(a.hbuf), rb = b1_rsrc(a.hb), rq = b1_rsrc(a.ssq);
  const size_t plane = (size_t)a.S * a.W;
  const int np = a.W / 32;
  constexpr int NT = kB1Compute * 64;
  // items (row, 4 columns): S * 8 of them, at most two per thread; every load of
  // both items is issued before any is used
  f32x4 hv[2], pv[2][kB1MaxParts];
  int row[2], c4 = tid & 7;
  bool ok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int it = tid + i * NT;
    ok[i] = it < a.S * 8;
    row[i] = ok[i] ? it >> 3 : 0;
    const uint32_t off = (uint32_t)(((size_t)row[i] * a.W + grp * 32 + c4 * 4) * 4);
    hv[i] = ok[i] ? __builtin_bit_cast(f32x4, ld16c(rh, off)) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kB1MaxParts; ++k)
      pv[i][k] = (ok[i] && k < nslice) ? __builtin_bit_cast(f32x4, ld16c(rp, (uint32_t)(off + k * plane * 4)))
                                       : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kB1MaxParts; ++k)
      if (k < nslice) sum += pv[i][k];
    const f32x4 h = hv[i] + sum;
    float ss = h[0] * h[0] + h[1] * h[1] + h[2] * h[2] + h[3] * h[3];
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    ss += __shfl_xor(ss, 4, 64);
    if (!ok[i]) continue;
    const uint32_t off = (uint32_t)(((size_t)row[i] * a.W + grp * 32 + c4 * 4) * 4);
    st16c(rh, off, __builtin_bit_cast(u32x4, h));
    const uint64_t packed = (uint64_t)__builtin_bit_cast(uint16_t, f2bf(h[0])) |
                            ((uint64_t)__builtin_bit_cast(uint16_t, f2bf(h[1])) << 16) |
                            ((uint64_t)__builtin_bit_cast(uint16_t, f2bf(h[2])) << 32) |
                            ((uint64_t)__builtin_bit_cast(uint16_t, f2bf(h[3])) << 48);
    st8c(rb, off / 2, packed);
    if (c4 == 0) st4c(rq, (uint32_t)(((size_t)row[i] * np + grp) * 4), ss);
  }
}

// On abort: the residual stream becomes NaN so the call's output is NaN.
__device__ __forceinline__ void b1_poison(const B1Args& a, int tid) {
  const auto rh = b1_rsrc(a.hbuf);
  for (int i = tid; i < a.S * a.W; i += kB1Compute * 64) st4c(rh, (uint32_t)(i * 4), __builtin_nanf(""));
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Fragment-order copies the loader streams as 1 KB contiguous blocks
// ---------------------------------------------------------------------------
// A [N][K] bf16 matrix (N % 32 == 0, K % 32 == 0), once at create: block
// (2 u + j) * (K / 32) + s holds, for lane l, the 8 elements
// W[32 u + 16 j + l % 16][32 s + 8 (l / 16) ..].
__global__ __launch_bounds__(256) void b1_pack_weights_kernel(const bf16* __restrict__ w, int N, int K,
                                                              bf16* __restrict__ wf) {
  const size_t chunks = (size_t)N * K / 8;
  const int steps = K / 32;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c % 64), s = (int)((c / 64) % steps);
    const size_t ju = c / 64 / steps;
    const size_t row = 32 * (ju / 2) + 16 * (ju % 2) + (lane & 15);
    const int col = 32 * s + 8 * (lane >> 4);
    *reinterpret_cast<u32x4*>(wf + c * 8) = *reinterpret_cast<const u32x4*>(w + row * K + col);
  }
}

// The call's prefix keys and values (batch 1), every layer, in the order the
// attention units consume them: for layer l and key block sp (64 keys), 32 key
// blocks (kt, c) -- lane l: K[64 sp + 16 kt + l % 16][32 c + 8 (l / 16) ..], the
// key clamped below valid_len -- then 32 value blocks (dd, ks) -- lane l:
// V[key][16 dd + l % 16] for the keys 64 sp + 32 ks + 16 (i / 4) + 4 (l / 16) +
// i % 4, i = 0..7 (the PV operand order of the probabilities), zero at keys >=
// valid_len.  Padded keys are never read; blocks wholly past valid_len are
// skipped (the stack never loads them).
__global__ __launch_bounds__(256) void b1_pack_kv_kernel(const CallDesc* __restrict__ desc, int L, int nsp,
                                                         bf16* __restrict__ kvf) {
  const int sp = blockIdx.x, l = blockIdx.y;
  int valid = desc->valid[0];
  valid = valid < 0 ? 0 : (valid > L ? L : valid);
  if (64 * sp >= valid) return;
  const bf16* K = reinterpret_cast<const bf16*>(desc->kv) + (size_t)l * 2 * L * 256;
  const bf16* V = K + (size_t)L * 256;
  bf16* dst = kvf + ((size_t)l * nsp + sp) * 64 * 512;
  for (int c = threadIdx.x; c < 64 * 64; c += 256) {
    const int blk = c / 64, ln = c % 64;
    if (blk < 32) {
      const int kt = blk / 8, cc = blk % 8;
      const int key = min(64 * sp + 16 * kt + (ln & 15), valid - 1);
      *reinterpret_cast<u32x4*>(dst + (size_t)c * 8) = gload16(K + (size_t)key * 256 + 32 * cc + 8 * (ln >> 4));
    } else {
      const int dd = (blk - 32) / 2, ks = (blk - 32) % 2;
      bf16x8 v;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = 64 * sp + 32 * ks + 16 * (i / 4) + 4 * (ln >> 4) + (i % 4);
        v[i] = key < valid ? V[(size_t)key * 256 + 16 * dd + (ln & 15)] : bf16(0.0f);
      }
      *reinterpret_cast<bf16x8*>(dst + (size_t)c * 8) = v;
    }
  }
}

// Trace stamps (the kernel instantiated with TR = true, first Euler step of a
// call): for block b, layer l, phase ph (Q, A, X, C, R1, G, D, R2, loader) and
// stamp k, trace[((b * D + l) * 9 + ph) * 4 + k] = device wall clock (100 MHz).
// Compute phases: k = 0 unit start, 1 dependency met, 2 weights landed,
// 3 completion published.  Loader: 0 layer start, 1 after the q/k/v unit,
// 2 after the gate/up unit, 3 after the layer.
#define B1_T(ph, k)                                                                                  \
  do {                                                                                               \
    if constexpr (TR) {                                                                              \
      if (a.step == 0 && lane == 0 && (wave == 0 || wave == kB1Compute))                             \
        a.trace[(((size_t)b * a.D + l) * 9 + (ph)) * 4 + (k)] = wall_clock64();                      \
    }                                                                                                \
  } while (0)

// The loader wave's program: every unit's blocks of every layer, in the
// order the compute waves consume them.  The ring and the control words come
// in as distinct restrict pointers, so the compiler knows the control-word
// accesses never touch what the DMA is writing and does not drain the DMA
// queue (vmcnt(0)) in front of each of them.
template <bool TR>
__device__ __forceinline__ void b1_loader(const B1Args& a, bf16* __restrict__ ring, B1Shared* __restrict__ shp,
                                          const B1Plan& p, int b, int nb, int lane, int valid, int npre, int nsp_pre,
                                          int aspan) {
  const int wave = kB1Compute;
  B1Loader ld{ring, shp};
    for (int l = 0; l < a.D && ld.ok; ++l) {
    const bf16* wqkv = a.lw[4 * l + 0];
    const bf16* wo = a.lw[4 * l + 1];
    const bf16* wgu = a.lw[4 * l + 2];
    const bf16* wdn = a.lw[4 * l + 3];
    B1_T(8, 0);
    for (int u = b1_first(b, nb, nb - p.nQ); u < p.nQ; u += nb) ld.weights(wqkv, a.W, u, 0, a.W, lane);
    B1_T(8, 1);
    for (int u = b; u < aspan; u += nb) {
      int split, tile;
      b1_attn_unit(a, u, split, tile);
      if (split >= a.nsplit) continue;
      if (split < nsp_pre && split < npre) {
        // the call's packed prefix block: 32 key fragment blocks, then 32 value blocks
        ld.run(a.kvf + ((size_t)l * nsp_pre + split) * 64 * 512, 64, lane);
      } else {
        ld.skip(kBlkA);  // suffix block (filled by the compute waves) or an empty one
      }
    }
    for (int u = b; u < p.nC; u += nb) {
      const int grp = u % p.ngrp, hs = u / p.ngrp;
      ld.weights(wo, a.qd, grp, 256 * hs, 256, lane);
    }
    for (int u = b; u < p.nG; u += nb) ld.weights(wgu, a.W, u, 0, a.W, lane);
    B1_T(8, 2);
    for (int u = b; u < p.nD; u += nb) {
      const int grp = u % p.ngrp, ms = u / p.ngrp;
      ld.weights(wdn, a.M, grp, 512 * ms, 512, lane);
    }
    B1_T(8, 3);
    }
  if (ld.ok) ld.publish_all();
}

template <bool TR>
__global__ __launch_bounds__(kB1Threads) void b1_stack_kernel(B1Args a) {
  __shared__ __attribute__((aligned(16))) bf16 ring[kB1Ring * 512];
  __shared__ B1Shared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x, nb = gridDim.x;
  if (tid == 0) {
    sh.loaded = 0;
    sh.bar = 0;
    sh.bcast = 0;
    sh.go = 0;
    sh.abort = 0;
#pragma unroll
    for (int w = 0; w < kB1Compute; ++w) sh.consumed[w] = 0;
  }
  __syncthreads();
  const B1Plan p = b1_plan(a);
  const int valid = b1_valid(a);
  const int npre = (valid + 63) / 64;          // prefix key blocks holding a valid key
  const int nsp_pre = a.nsplit - 1;            // key blocks of the padded prefix
  const int aspan = b1_attn_units_span(a);

  // ------------------------------------------------------------------ loader
  if (wave == kB1Compute) {
    b1_loader<TR>(a, ring, &sh, p, b, nb, lane, valid, npre, nsp_pre, aspan);
    return;
  }

  // ------------------------------------------------------------ compute waves
  B1Wave w{&sh, ring, wave, lane};
  // lane-derived values are rebuilt at the start of every unit (fresh_lane):
  // otherwise the compiler hoists each phase's per-lane addresses out of the
  // layer loop and keeps all of them live at once
  int lane_v = lane;
  auto fresh_lane = [&]() {
    asm volatile("" : "+v"(lane_v));
    w.lane = lane_v;
  };
  const int row0 = 16 * wave;
  auto abort_out = [&]() { b1_poison(a, tid); };
  const auto rqk = b1_rsrc(a.qk), rvts = b1_rsrc(a.vts), ro = b1_rsrc(a.o), rg = b1_rsrc(a.g);
  const int ldqk = a.qd + 256;
  const int nq = a.nh * a.S;

  for (int l = 0; l < a.D; ++l) {
    const unsigned e = (unsigned)(a.step * a.D + l);
    // ---------------------------------------------------------------- Q
    for (int u = b1_first(opq(b), nb, nb - p.nQ); u < p.nQ; u += nb) {
      fresh_lane();
      const int lane = lane_v, ctid = wave * 64 + lane_v;
      (void)ctid;
      B1_T(0, 0);
      if (!w.wait(a, kCntR2, e * p.ngrp)) return abort_out();
      B1_T(0, 1);
      bf16x8 af[32];
      b1_load_a<32>(a.hb, a.W, 0, row0, a.S, lane, af);
      const B1Ssq sq = b1_ssq_issue(a, l == 0 ? a.np0 : p.ngrp, row0, lane);
      // the RoPE angles of this lane's rows (or nothing for the value columns)
      const int cq = 32 * u + (lane & 15);
      float2 rcs[4];
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int row = min(row0 + 4 * (lane >> 4) + e4, a.S - 1);
        const int wc = cq % 256, jj = (wc >> 5) * 16 + (wc & 15);
        rcs[e4] = cq < a.qd + 256 ? a.rope_cs[(size_t)row * 128 + jj] : float2{1.f, 0.f};
      }
      if (!w.await_ring(kBlkQ)) return abort_out();
      B1_T(0, 2);
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      b1_mma<32>(w, af, acc);
      w.release_ring(kBlkQ);
      float inv[4];
      b1_inv_rms(a, sq, lane, inv);
      const int c = cq;  // stored column of acc[0]; acc[1] is c + 16
      const int qkc = a.qd + 256;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int row = row0 + 4 * (lane >> 4) + e4;
        if (row >= a.S) continue;
        const float x1 = acc[0][e4] * inv[e4], x2 = acc[1][e4] * inv[e4];
        if (c < qkc) {
          const int head = c / 256, wc = c % 256, jj = (wc >> 5) * 16 + (wc & 15);
          const float2 cs = rcs[e4];
          const size_t o1 = (size_t)row * ldqk + head * 256 + jj;
          st2c(rqk, (uint32_t)(o1 * 2), f2bf(x1 * cs.x - x2 * cs.y));
          st2c(rqk, (uint32_t)((o1 + 128) * 2), f2bf(x2 * cs.x + x1 * cs.y));
        } else {
          const int d = c - qkc;
          st2c(rvts, (uint32_t)(((size_t)d * 64 + vt_pos(row)) * 2), f2bf(x1));
          st2c(rvts, (uint32_t)(((size_t)(d + 16) * 64 + vt_pos(row)) * 2), f2bf(x2));
        }
      }
      if (!w.arrive_all()) return abort_out();
      if (wave == 0) b1_signal(a.cnt, kCntQ, lane);
      B1_T(0, 3);
    }
    // ---------------------------------------------------------------- A
    for (int u = opq(b); u < aspan; u += nb) {
      fresh_lane();
      const int lane = lane_v, ctid = wave * 64 + lane_v;
      (void)ctid;
      int split, tile;
      b1_attn_unit(a, u, split, tile);
      if (split >= a.nsplit) continue;
      const bool suffix = split == nsp_pre;
      const bool empty = !suffix && split >= npre;
      B1_T(1, 0);
      if (!w.wait(a, kCntQ, (e + 1) * p.nQ)) return abort_out();
      B1_T(1, 1);
      // one 16-query tile per wave (query qi = 64 tile + 16 wave + lane % 16);
      // its q fragments are requested before anything else waits
      const int qi = 64 * tile + 16 * wave + (lane & 15);
      const bool qok = qi < nq;
      const int qs = qok ? qi / a.nh : 0, qn = qok ? qi % a.nh : 0;
      bf16x8 qf[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        qf[c] = (qok && !empty) ? __builtin_bit_cast(bf16x8, ld16c(rqk, (uint32_t)(((size_t)qs * ldqk + qn * 256 + c * 32 +
                                                                                    (lane >> 4) * 8) * 2)))
                                : bf16x8{};
      if (!w.await_ring(kBlkA)) return abort_out();
      B1_T(1, 2);
      if (suffix) {
        // stage the suffix keys (rows >= S zero) and values (V^T, zero beyond S) in the unit's blocks
        // (every load of the wave's 16 blocks is issued before the first LDS write)
        u32x4 sv[64 / kB1Compute];
#pragma unroll
        for (int j = 0; j < 64 / kB1Compute; ++j) {
          const int i = wave + j * kB1Compute;
          sv[j] = u32x4{0u, 0u, 0u, 0u};
          if (i < 32) {
            const int kt = i / 8, c = i % 8, key = 16 * kt + (lane & 15);
            if (key < a.S) sv[j] = ld16c(rqk, (uint32_t)(((size_t)key * ldqk + a.qd + c * 32 + (lane >> 4) * 8) * 2));
          } else {
            const int dd = (i - 32) / 2, ks = (i - 32) % 2;
            sv[j] = ld16c(rvts, (uint32_t)(((size_t)(16 * dd + (lane & 15)) * 64 + 32 * ks + (lane >> 4) * 8) * 2));
          }
        }
#pragma unroll
        for (int j = 0; j < 64 / kB1Compute; ++j) *reinterpret_cast<u32x4*>(w.frag_w(wave + j * kB1Compute)) = sv[j];
        wait_lgkm0();
        if (!w.arrive_all()) return abort_out();
      }
      float m_run = -INFINITY, l_run = 0.f;
      f32x4 oacc[16];
#pragma unroll
      for (int d = 0; d < 16; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (!empty) {
        f32x4 sacc[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w.frag(kt * 8 + c), qf[c], sacc[kt], 0, 0, 0);
        // mask and softmax over this key block: lane holds keys 16 kt + 4 (lane/16) + e of its query
        const int g4 = (lane >> 4) * 4;
        const int lim = !suffix ? valid - 64 * split : ((a.causal || qs == 0) ? min(a.S, qs + 1) : a.S);
        float sc[4][4];
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const float v = kt * 16 + g4 + e4 < lim ? sacc[kt][e4] * a.scale : -INFINITY;
            sc[kt][e4] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        m_run = mx;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 pf;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = sc[2 * ks + i / 4][i % 4];
            const float ev = (x == -INFINITY) ? 0.f : __expf(x - m_run);
            l_run += ev;
            pf[i] = f2bf(ev);
          }
#pragma unroll
          for (int d = 0; d < 16; ++d)
            oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w.frag(32 + d * 2 + ks), pf, oacc[d], 0, 0, 0);
        }
      }
      w.release_ring(kBlkA);
      // partial state of (split, tile): max and sum per query (float [ub][2][64]),
      // unnormalised outputs in bf16 ([ub][64][256] after the float part)
      const size_t ub = (size_t)split * a.ntile + tile;
      const auto rap = b1_rsrc(a.apart);
      const size_t obase = (size_t)a.nsplit * a.ntile * 128 * 4;
      float lt = l_run + __shfl_xor(l_run, 16, 64);
      lt += __shfl_xor(lt, 32, 64);
      const int q = 16 * wave + (lane & 15);
      if ((lane >> 4) == 0) {
        st4c(rap, (uint32_t)((ub * 128 + q) * 4), m_run);
        st4c(rap, (uint32_t)((ub * 128 + 64 + q) * 4), lt);
      }
      // features 16 d + 4 g + e (g = lane / 16) of d-tiles d = 2 dp and 2 dp + 1
      // as one 16-byte store at element 32 dp + 8 g of the query's row
#pragma unroll
      for (int dp = 0; dp < 8; ++dp) {
        bf16x8 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r[e] = f2bf(oacc[2 * dp][e]);
          r[4 + e] = f2bf(oacc[2 * dp + 1][e]);
        }
        st16c(rap, (uint32_t)(obase + ((ub * 64 + q) * 256 + dp * 32 + (lane >> 4) * 8) * 2), __builtin_bit_cast(u32x4, r));
      }
      if (!w.arrive_all()) return abort_out();
      if (wave == 0) b1_signal(a.cnt, (kCntA + tile), lane);
      B1_T(1, 3);
    }
    // ---------------------------------------------------------------- X
    for (int u = b1_first(opq(b), nb, aspan); u < p.nX; u += nb) {
      fresh_lane();
      const int lane = lane_v, ctid = wave * 64 + lane_v;
      (void)ctid;
      const int tile = u / 16, dc = u % 16;
      B1_T(2, 0);
      if (!w.wait(a, kCntA + tile, (e + 1) * a.nsplit)) return abort_out();
      B1_T(2, 1);
      // thread: query q of the tile, features 16 dc + 4 part .. +3
      const int q = ctid >> 2, part = ctid & 3;
      const int qi = 64 * tile + q;
      const auto rap = b1_rsrc(a.apart);
      const size_t obase = (size_t)a.nsplit * a.ntile * 128 * 4;
      if (qi < nq) {
        // splits in chunks of 8: a chunk's states are requested before any is
        // used, and the running maximum carries over between chunks (split order)
        typedef unsigned u2 __attribute__((ext_vector_type(2)));
        constexpr int CH = 8;
        float m = -INFINITY, lsum = 0.f, acc4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < a.nsplit; s0 += CH) {
          float ms[CH], ls[CH];
          u2 raw[CH];
#pragma unroll
          for (int k = 0; k < CH; ++k) {
            const size_t ub = (size_t)min(s0 + k, a.nsplit - 1) * a.ntile + tile;
            ms[k] = ld4c(rap, (uint32_t)((ub * 128 + q) * 4));
            ls[k] = ld4c(rap, (uint32_t)((ub * 128 + 64 + q) * 4));
            raw[k] = __builtin_bit_cast(
                u2, __builtin_amdgcn_raw_buffer_load_b64(
                      rap, (uint32_t)(obase + ((ub * 64 + q) * 256 + (dc >> 1) * 32 + part * 8 + (dc & 1) * 4) * 2), 0,
                      kSc1));
          }
          float mb = m;
#pragma unroll
          for (int k = 0; k < CH; ++k)
            if (s0 + k < a.nsplit) mb = fmaxf(mb, ms[k]);
          const float s_old = (m == -INFINITY) ? 0.f : __expf(m - mb);
          lsum *= s_old;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc4[i] *= s_old;
#pragma unroll
          for (int k = 0; k < CH; ++k) {
            if (s0 + k >= a.nsplit || ms[k] == -INFINITY) continue;
            const float wgt = __expf(ms[k] - mb);
            lsum += ls[k] * wgt;
            acc4[0] += __builtin_bit_cast(float, raw[k][0] << 16) * wgt;
            acc4[1] += __builtin_bit_cast(float, raw[k][0] & 0xffff0000u) * wgt;
            acc4[2] += __builtin_bit_cast(float, raw[k][1] << 16) * wgt;
            acc4[3] += __builtin_bit_cast(float, raw[k][1] & 0xffff0000u) * wgt;
          }
          m = mb;
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        const uint64_t packed = (uint64_t)__builtin_bit_cast(uint16_t, f2bf(acc4[0] * inv)) |
                                ((uint64_t)__builtin_bit_cast(uint16_t, f2bf(acc4[1] * inv)) << 16) |
                                ((uint64_t)__builtin_bit_cast(uint16_t, f2bf(acc4[2] * inv)) << 32) |
                                ((uint64_t)__builtin_bit_cast(uint16_t, f2bf(acc4[3] * inv)) << 48);
        const int s = qi / a.nh, n = qi % a.nh;
        st8c(ro, (uint32_t)(((size_t)s * a.qd + n * 256 + dc * 16 + part * 4) * 2), packed);
      }
      if (!w.arrive_all()) return abort_out();
      if (wave == 0) b1_signal(a.cnt, kCntX, lane);
      B1_T(2, 3);
    }
    // ---------------------------------------------------------------- C
    for (int u = opq(b); u < p.nC; u += nb) {
      fresh_lane();
      const int lane = lane_v, ctid = wave * 64 + lane_v;
      (void)ctid;
      const int grp = u % p.ngrp, hs = u / p.ngrp;
      B1_T(3, 0);
      if (!w.wait(a, kCntX, (e + 1) * p.nX)) return abort_out();
      B1_T(3, 1);
      bf16x8 af[8];
      b1_load_a<8>(a.o, a.qd, 256 * hs, row0, a.S, lane, af);
      if (!w.await_ring(kBlkC)) return abort_out();
      B1_T(3, 2);
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      b1_mma<8>(w, af, acc);
      w.release_ring(kBlkC);
      const auto rp = b1_rsrc(a.cpart);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int row = row0 + 4 * (lane >> 4) + e4;
          if (row < a.S)
            st4c(rp, (uint32_t)((((size_t)hs * a.S + row) * a.W + 32 * grp + 16 * j + (lane & 15)) * 4), acc[j][e4]);
        }
      if (!w.arrive_all()) return abort_out();
      if (wave == 0) {
        unsigned last = 0;
        if (lane == 0) {
          const unsigned old = __hip_atomic_fetch_add(a.cnt + (size_t)(kCntC + grp) * 32, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
          last = (old + 1u == (e + 1) * (unsigned)p.nhs) ? 1u : 0u;
          lds_st(&sh.bcast, (w.bar_gen << 1) | last);
        }
      }
      if (!b1_lds_wait(&sh.bcast, w.bar_gen << 1, &sh)) return abort_out();
      B1_T(3, 3);
      if ((lds_ld(&sh.bcast) & 1u) != 0u) {
        B1_T(4, 0);
        b1_reduce_group(a, a.cpart, p.nhs, grp, ctid);
        if (!w.arrive_all()) return abort_out();
        if (wave == 0) b1_signal(a.cnt, kCntR1, lane);
        B1_T(4, 3);
      }
    }
    // ---------------------------------------------------------------- G
    for (int u = opq(b); u < p.nG; u += nb) {
      fresh_lane();
      const int lane = lane_v, ctid = wave * 64 + lane_v;
      (void)ctid;
      B1_T(5, 0);
      if (!w.wait(a, kCntR1, (e + 1) * p.ngrp)) return abort_out();
      B1_T(5, 1);
      bf16x8 af[32];
      b1_load_a<32>(a.hb, a.W, 0, row0, a.S, lane, af);
      const B1Ssq sq = b1_ssq_issue(a, p.ngrp, row0, lane);
      if (!w.await_ring(kBlkG)) return abort_out();
      B1_T(5, 2);
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      b1_mma<32>(w, af, acc);
      w.release_ring(kBlkG);
      float inv[4];
      b1_inv_rms(a, sq, lane, inv);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int row = row0 + 4 * (lane >> 4) + e4;
        if (row >= a.S) continue;
        const float gt = acc[0][e4] * inv[e4], up = acc[1][e4] * inv[e4];
        st2c(rg, (uint32_t)(((size_t)row * a.M + 16 * u + (lane & 15)) * 2), f2bf(gelu_tanh_fast<bf16>(gt) * up));
      }
      if (!w.arrive_all()) return abort_out();
      if (wave == 0) b1_signal(a.cnt, kCntG + (16 * u) / 512, lane);
      B1_T(5, 3);
    }
    // ---------------------------------------------------------------- D
    for (int u = opq(b); u < p.nD; u += nb) {
      fresh_lane();
      const int lane = lane_v, ctid = wave * 64 + lane_v;
      (void)ctid;
      const int grp = u % p.ngrp, ms = u / p.ngrp;
      B1_T(6, 0);
      if (!w.wait(a, kCntG + ms, (e + 1) * 32u)) return abort_out();
      B1_T(6, 1);
      bf16x8 af[16];
      b1_load_a<16>(a.g, a.M, 512 * ms, row0, a.S, lane, af);
      if (!w.await_ring(kBlkD)) return abort_out();
      B1_T(6, 2);
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      b1_mma<16>(w, af, acc);
      w.release_ring(kBlkD);
      const auto rp = b1_rsrc(a.dpart);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int row = row0 + 4 * (lane >> 4) + e4;
          if (row < a.S)
            st4c(rp, (uint32_t)((((size_t)ms * a.S + row) * a.W + 32 * grp + 16 * j + (lane & 15)) * 4), acc[j][e4]);
        }
      if (!w.arrive_all()) return abort_out();
      if (wave == 0) {
        if (lane == 0) {
          const unsigned old = __hip_atomic_fetch_add(a.cnt + (size_t)(kCntD + grp) * 32, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
          const unsigned last = (old + 1u == (e + 1) * (unsigned)p.nms) ? 1u : 0u;
          lds_st(&sh.bcast, (w.bar_gen << 1) | last);
        }
      }
      if (!b1_lds_wait(&sh.bcast, w.bar_gen << 1, &sh)) return abort_out();
      B1_T(6, 3);
      if ((lds_ld(&sh.bcast) & 1u) != 0u) {
        B1_T(7, 0);
        b1_reduce_group(a, a.dpart, p.nms, grp, ctid);
        if (!w.arrive_all()) return abort_out();
        if (wave == 0) b1_signal(a.cnt, kCntR2, lane);
        B1_T(7, 3);
      }
    }
  }
}

#undef B1_T

}  // namespace pi0x
