// Shared device helpers for the gfx950 (CDNA4) MLA kernels.
//
// Matrix-core convention used by every kernel: an MFMA "fragment" is the 8 values of
// the contraction index k that one lane feeds to one MFMA k-step.
//   bf16: one v_mfma_f32_{16x16x32,32x32x16}_bf16; lane l holds k = 8*(l/W) + [0..7]
//         (W = 16 or 32, the tile width).
//   fp32: eight v_mfma_f32_{16x16x4,32x32x2}f32; instruction j consumes the lane's j-th
//         value, i.e. k = 8*(l/W) + j.  Because the A and B operands use the same
//         lane -> k map, the contraction over k is identical to the bf16 one (the sum
//         over k does not depend on the order of its terms), so one kernel source
//         serves both element types.
// Accumulator (C/D) layouts are the hardware's:
//   16x16: lane l owns column l%16 and rows 4*(l/16) + i, i = 0..3;
//   32x32: lane l owns column l%32 and rows 8*(i/4) + 4*(l/32) + (i%4), i = 0..15.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace mla {

// f(integral_constant<LO + i>) for i in the sequence, in order, fully unrolled
template <int LO, typename F, int... I>
__device__ __forceinline__ void unroll_from(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, LO + I>{}), ...);
}

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Element conversion (fp32 -> bf16 rounds to nearest even on gfx950)
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

// ---------------------------------------------------------------------------
// 8-element fragments
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

template <typename T> __device__ __forceinline__ Frag<T> frag_zero();
template <> __device__ __forceinline__ Frag<bf16> frag_zero<bf16>() {
  Frag<bf16> f;
  f.v = (bf16x8){0, 0, 0, 0, 0, 0, 0, 0};
  return f;
}
template <> __device__ __forceinline__ Frag<float> frag_zero<float>() {
  Frag<float> f;
  f.lo = (f32x4){0.f, 0.f, 0.f, 0.f};
  f.hi = f.lo;
  return f;
}

// Fragment from 8 fp32 values (rounded for bf16).
template <typename T> __device__ __forceinline__ Frag<T> frag_from_f32(const float* v);
template <> __device__ __forceinline__ Frag<bf16> frag_from_f32<bf16>(const float* v) {
  Frag<bf16> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = (bf16)v[j];
  return f;
}
template <> __device__ __forceinline__ Frag<float> frag_from_f32<float>(const float* v) {
  Frag<float> f;
  f.lo = (f32x4){v[0], v[1], v[2], v[3]};
  f.hi = (f32x4){v[4], v[5], v[6], v[7]};
  return f;
}

// Contiguous 8-element fragment load from LDS or global memory (16-B aligned for bf16,
// 32-B aligned... 16-B aligned halves for fp32).
template <typename T> __device__ __forceinline__ Frag<T> frag_load(const T* p);
template <> __device__ __forceinline__ Frag<bf16> frag_load<bf16>(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
template <> __device__ __forceinline__ Frag<float> frag_load<float>(const float* p) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f;
}

// Two 4-element runs (k slots 0..3 from p0, 4..7 from p1).
template <typename T> __device__ __forceinline__ Frag<T> frag_load_2x4(const T* p0, const T* p1);
template <> __device__ __forceinline__ Frag<bf16> frag_load_2x4<bf16>(const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  Frag<bf16> f;
  f.v = (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}
template <> __device__ __forceinline__ Frag<float> frag_load_2x4<float>(const float* p0, const float* p1) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p0);
  f.hi = *reinterpret_cast<const f32x4*>(p1);
  return f;
}

// ---------------------------------------------------------------------------
// MFMA k-steps
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mma16(const Frag<bf16>& a, const Frag<bf16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ f32x16 mma32(const Frag<bf16>& a, const Frag<bf16>& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32(const Frag<float>& a, const Frag<float>& b, f32x16 c) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[0], b.lo[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[1], b.lo[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[2], b.lo[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[3], b.lo[3], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[0], b.hi[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[1], b.hi[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[2], b.hi[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[3], b.hi[3], c, 0, 0, 0);
  return c;
}

// ---------------------------------------------------------------------------
// 8-element chunks moved between global memory, registers and LDS
// ---------------------------------------------------------------------------
template <typename T> struct Chunk;
template <> struct Chunk<bf16> { uint4 a; };
template <> struct Chunk<float> { uint4 a, b; };

template <typename T> __device__ __forceinline__ void chunk_zero(Chunk<T>& c);
template <> __device__ __forceinline__ void chunk_zero<bf16>(Chunk<bf16>& c) { c.a = make_uint4(0, 0, 0, 0); }
template <> __device__ __forceinline__ void chunk_zero<float>(Chunk<float>& c) {
  c.a = make_uint4(0, 0, 0, 0);
  c.b = c.a;
}

// Vector load of 8 contiguous elements (address 16-B aligned).
template <typename T> __device__ __forceinline__ void chunk_load(Chunk<T>& c, const T* p);
template <> __device__ __forceinline__ void chunk_load<bf16>(Chunk<bf16>& c, const bf16* p) {
  c.a = *reinterpret_cast<const uint4*>(p);
}
template <> __device__ __forceinline__ void chunk_load<float>(Chunk<float>& c, const float* p) {
  c.a = *reinterpret_cast<const uint4*>(p);
  c.b = *reinterpret_cast<const uint4*>(p + 4);
}

// Element-wise load of the first n (< 8 allowed) elements, rest zero.
template <typename T> __device__ __forceinline__ void chunk_load_partial(Chunk<T>& c, const T* p, int n) {
  T v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (j < n) ? p[j] : from_f32<T>(0.f);
  __builtin_memcpy(&c, v, sizeof(v));
}

template <typename T> __device__ __forceinline__ void chunk_store(T* p, const Chunk<T>& c);
template <> __device__ __forceinline__ void chunk_store<bf16>(bf16* p, const Chunk<bf16>& c) {
  *reinterpret_cast<uint4*>(p) = c.a;
}
template <> __device__ __forceinline__ void chunk_store<float>(float* p, const Chunk<float>& c) {
  *reinterpret_cast<uint4*>(p) = c.a;
  *reinterpret_cast<uint4*>(p + 4) = c.b;
}

template <typename T> __device__ __forceinline__ T chunk_elem(const Chunk<T>& c, int j) {
  T v[8];
  __builtin_memcpy(v, &c, sizeof(v));
  return v[j];
}

// Scatter the chunk's 8 elements down a column: p[j * stride] = elem j.
template <typename T> __device__ __forceinline__ void chunk_store_column(T* p, int stride, const Chunk<T>& c) {
  T v[8];
  __builtin_memcpy(v, &c, sizeof(v));
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j * stride] = v[j];
}

// ---------------------------------------------------------------------------
// Misc
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max32(float v) {
  // max with the lane 32 apart (the other half of a 32x32 accumulator column)
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float wave_sum32(float v) { return v + __shfl_xor(v, 32); }

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int round_up(int a, int b) { return cdiv(a, b) * b; }

// Dropout draws: SplitMix64 (Steele, Lea, Flood, OOPSLA 2014) used as a counter-based
// generator.  One draw serves the four attention weights (query i, keys 4 j4 .. 4 j4 + 3) of
// head stream zh = b H + h: the generator's output n + 1 from state seed, n = zh 2^38 +
// i 2^18 + j4, i.e. the state seed + (n + 1) gamma through the output function (two
// xor-shift-multiply steps, a final xor-shift).  Key 4 j4 + e uses bits 16 e .. 16 e + 15 and
// is kept when they are >= thr = floor(p 2^16).
constexpr uint64_t kSplitmixGamma = 0x9E3779B97F4A7C15ull;
// the generator's output function applied to a state
__device__ __forceinline__ uint64_t splitmix_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
// the state of draw n: linear in n, so kernels that walk the counters step it by additions
__device__ __forceinline__ uint64_t splitmix_state(uint64_t seed, uint64_t n) {
  return seed + (n + 1ull) * kSplitmixGamma;
}
__device__ __forceinline__ uint64_t dropout_draw(uint64_t seed, uint64_t n) {
  return splitmix_mix(splitmix_state(seed, n));
}
__device__ __forceinline__ uint64_t dropout_counter4(int zh, int i, int j4) {
  return ((uint64_t)(uint32_t)zh << 38) + ((uint64_t)(uint32_t)i << 18) + (uint64_t)(uint32_t)j4;
}
// Keep bits of the four weights (query i, keys 4 j4 .. 4 j4 + 3): bit e for key 4 j4 + e.
__device__ __forceinline__ unsigned dropout_keep4(uint64_t seed, uint32_t thr, int j4, int i, int zh) {
  const uint64_t r = dropout_draw(seed, dropout_counter4(zh, i, j4));
  unsigned bits = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) bits |= ((uint32_t)(r >> (16 * e)) & 0xFFFFu) >= thr ? (1u << e) : 0u;
  return bits;
}

// Rotation angle pos * theta in double, reduced to [-pi, pi] before the fp32 sin/cos,
// so that large positions keep fp32 accuracy in the rotation.
__device__ __forceinline__ void rope_sincos(int pos, float inv_freq_hi, float inv_freq_lo,
                                            float* s, float* c) {
  double a = (double)pos * ((double)inv_freq_hi + (double)inv_freq_lo);
  const double two_pi = 6.283185307179586476925286766559;
  a = a - two_pi * rint(a * (1.0 / two_pi));   // a multiply: a double division is ~10x the work
  sincosf((float)a, s, c);
}

}  // namespace mla
