// Shared device-side types and helpers for the pi0x kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pi0x {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
// 16 raw bytes as a native vector (HIP's uint4 struct copies through memory)
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// Per-call arguments that change between calls without re-recording the
// captured graph.  A one-thread kernel writes this struct on the caller's
// stream right before the graph replays; every kernel reads its pointers here.
struct CallDesc {
  const void* kv;        // prefix K/V, [depth][2][B][L][head_dim], model dtype
  const int32_t* valid;  // [B] valid prefix lengths
  const float* state;    // [B][state_dim]
  const float* x_in;     // denoise: the noise (x at t = 1); single step: x_t.  [B][H][A]
  float* out;            // denoise: the actions; single step: the velocity.  [B][H][A]
  float t;               // single step: the time value
  const float* dof_mask;  // first-step padding blend (NULL: none), [B][H][A]
  const float* padding;   // the padding action of that blend, [B][H][A]
  // prefix pass: the embeddings [B][L][width] (model dtype) and the cache it
  // writes, [depth][2][B][L][head_dim] (kv points at the same cache)
  const void* emb;
  void* kv_out;
};

// Boundary normalization statistics (page 1, _build_norm_buffers /
// _apply_norm), set by pi0x_set_normalization and read by the kernels on
// every call.  mode 0: none; 1: mean/std; 2: min/max.  Only the first count
// features are transformed; the rest pass through.  Host-prepared float32:
//   state  (forward):  mean/std  (s - a) / d         with d = std + 1e-8
//                      min/max   2 (s - a) / d - 1   with d = max(max - min, 1e-8)
//   action (inverse):  mean/std  x d + a             with d = std
//                      min/max   (x + 1) / 2 d + a   with d = max(max - min, 1e-8)
constexpr int kNormMaxDim = 64;
struct NormDev {
  int state_mode, state_count, action_mode, action_count;
  float sa[kNormMaxDim], sd[kNormMaxDim];
  float aa[kNormMaxDim], ad[kNormMaxDim];
};

__device__ __forceinline__ float norm_state(const NormDev* n, int j, float x) {
  if (n->state_mode == 0 || j >= n->state_count) return x;
  if (n->state_mode == 1) return (x - n->sa[j]) / n->sd[j];
  return 2.0f * (x - n->sa[j]) / n->sd[j] - 1.0f;
}
__device__ __forceinline__ float unnorm_action(const NormDev* n, int j, float x) {
  if (n->action_mode == 0 || j >= n->action_count) return x;
  if (n->action_mode == 1) return x * n->ad[j] + n->aa[j];
  return (x + 1.0f) * 0.5f * n->ad[j] + n->aa[j];
}

// 16-byte load through a global-address-space pointer.  Pointers read from
// memory (the call descriptor) are generic to the compiler; generic loads
// also count against the LDS counter, so a later LDS wait would stall on them.
__device__ __forceinline__ u32x4 gload16(const void* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(
      (const __attribute__((address_space(1))) void*)p);
}

// float -> bfloat16, round to nearest even (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ bf16 f2bf(float f) { return (bf16)f; }

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float f) { return f2bf(f); }

__device__ __forceinline__ float to_f32(float f) { return f; }
__device__ __forceinline__ float to_f32(bf16 b) {
  return __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// ---------------------------------------------------------------------------
// MFMA fragments.  A "k32 fragment" is what one lane contributes to a 16x16
// output tile for a 32-wide slice of the reduction dimension: lane l covers
// row/column (l % 16) and the 8 reduction indices 8*(l/16) .. 8*(l/16)+7.
// bf16 issues one v_mfma_f32_16x16x32_bf16; fp32 issues eight
// v_mfma_f32_16x16x4_f32, the i-th taking reduction index 8*(l/16)+i (the
// two operands only have to agree on which index each lane supplies).
// Output tile layout (both): lane l holds rows 4*(l/16)+e, e = 0..3, of
// column l % 16.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mma32(const Frag<bf16>& a, const Frag<bf16>& b, f32x4& c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma32(const Frag<float>& a, const Frag<float>& b, f32x4& c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], c, 0, 0, 0);
}

// 8 consecutive elements
__device__ __forceinline__ void load8(Frag<bf16>& f, const bf16* p) { f.v = *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void load8(Frag<float>& f, const float* p) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// 4 + 4 consecutive elements from two places
__device__ __forceinline__ void load4x2(Frag<bf16>& f, const bf16* p0, const bf16* p1) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}
__device__ __forceinline__ void load4x2(Frag<float>& f, const float* p0, const float* p1) {
  float4 a = *reinterpret_cast<const float4*>(p0);
  float4 b = *reinterpret_cast<const float4*>(p1);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ void set_frag(Frag<bf16>& f, int i, float x) { f.v[i] = f2bf(x); }
__device__ __forceinline__ void set_frag(Frag<float>& f, int i, float x) { f.v[i] = x; }

// 8 consecutive floats from memory (two 16-byte loads) / to memory as T
// (one 16-byte store for bf16, two for float32).  Pointers 16-byte aligned.
__device__ __forceinline__ void load8f(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<float4*>(p + 4) = float4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = f2bf(v[i]);
  *reinterpret_cast<bf16x8*>(p) = r;
}

// Key order of the transposed values (V^T) within every group of 32 keys:
// key k = 16 h + 4 g + e (h < 2, g < 4, e < 4) is stored at 8 g + 4 h + e, so
// the 8 keys one lane contributes to a 16x16x32 PV MFMA (4 g .. 4 g + 3 and
// 16 + 4 g .. 16 + 4 g + 3) are contiguous: one 16-byte read.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4):
// lane l of the wave writes dst + 16 l bytes, dst wave-uniform.  Counted by
// vmcnt like any other vector-memory load.
__device__ __forceinline__ void lds_dma16(const bf16* src, bf16* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// s_waitcnt with only the vector-memory counter limited to N (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the LDS ring.  __syncthreads() would also wait for
// every outstanding global load (its fence covers the DMA writes), draining
// the prefetch; the ring orders its DMA with explicit vmcnt waits instead, and
// the empty asm statements only keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Orders one wave's LDS accesses across lanes: a wave's LDS instructions
// execute in program order, so only the compiler has to be kept from moving
// loads and stores across this point.
__device__ __forceinline__ void wave_lds_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// tanh-GELU through the identity 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)):
// gelu(x) = x / (1 + exp(-2 sqrt(2/pi) (x + 0.044715 x^3))).  The bf16 path
// uses the hardware exp2 and reciprocal (its result is rounded to bf16), the
// float32 path libm expf and an IEEE division.
template <typename T>
__device__ __forceinline__ float gelu_tanh_fast(float x) {
  const float u = -1.5957691216057308f * (x + 0.044715f * x * x * x);  // -2 sqrt(2/pi) (...)
  if (sizeof(T) == 2) return x * __builtin_amdgcn_rcpf(1.0f + __expf(u));  // v_rcp_f32 (1 ulp)
  return x / (1.0f + expf(u));
}

}  // namespace pi0x
