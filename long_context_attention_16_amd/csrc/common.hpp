// Device helpers shared by the kernels of the compressed-attention library.
// gfx950 (CDNA4) only: wave64, MFMA, 160 KB LDS per CU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kRopeDims = 64;        // rotated dims: the last 64 of each head
constexpr int kRopePairs = kRopeDims / 2;

// ---------------------------------------------------------------- bf16 / f32
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// Round-to-nearest-even f32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Element access by storage type: float (f32) or uint16_t (bf16 bits).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ---------------------------------------------------------------- RoPE
// RoPE frequency of rotated pair i in revolutions per position:
// 10000^(-i/32) / (2*pi), evaluated in double at compile time.
constexpr double cexp_small(double x) {  // e^x for |x| <= 0.2 (Taylor, 24 terms)
  double term = 1.0, sum = 1.0;
  for (int k = 1; k < 24; ++k) { term *= x / k; sum += term; }
  return sum;
}
constexpr double cexp(double x) {  // e^x for -16 <= x <= 0: e^(x/128)^128
  double y = cexp_small(x / 128.0);
  for (int k = 0; k < 7; ++k) y *= y;
  return y;
}
constexpr double kLn10000 = 9.210340371976184;
constexpr double kTwoPi = 6.283185307179586476925;
constexpr double rope_rev(int i) { return cexp(-(double)i / 32.0 * kLn10000) / kTwoPi; }
__constant__ const double kRopeRev[32] = {
    rope_rev(0),  rope_rev(1),  rope_rev(2),  rope_rev(3),  rope_rev(4),  rope_rev(5),  rope_rev(6),
    rope_rev(7),  rope_rev(8),  rope_rev(9),  rope_rev(10), rope_rev(11), rope_rev(12), rope_rev(13),
    rope_rev(14), rope_rev(15), rope_rev(16), rope_rev(17), rope_rev(18), rope_rev(19), rope_rev(20),
    rope_rev(21), rope_rev(22), rope_rev(23), rope_rev(24), rope_rev(25), rope_rev(26), rope_rev(27),
    rope_rev(28), rope_rev(29), rope_rev(30), rope_rev(31)};

// cos/sin of position p times the frequency of pair i. The angle is reduced
// to a fraction of a revolution in double (exact to ~1e-11 rad for positions
// up to 2^20), then evaluated in float on [-pi, pi].
__device__ __forceinline__ void rope_cos_sin_f(int64_t p, double rev, float* c, float* s) {
  const double a = (double)p * rev;
  const float r = (float)(a - rint(a));
  const float x = r * 6.2831853071795865f;
  *s = sinf(x);
  *c = cosf(x);
}
__device__ __forceinline__ void rope_cos_sin(int64_t p, int i, float* c, float* s) {
  rope_cos_sin_f(p, kRopeRev[i], c, s);
}

// Absolute position of query row 0 of sequence b: `bound` for every
// sequence, or q_pos[b] clamped into [0, bound] when per-sequence positions
// are given (q_pos != nullptr; bound is then their upper bound, which sized
// the grid and the workspace).
__device__ __forceinline__ int64_t seq_pos(const int64_t* q_pos, int64_t bound, int b) {
  if (q_pos == nullptr) return bound;
  const int64_t v = q_pos[b];
  return v < 0 ? 0 : (v > bound ? bound : v);
}

// max(x, 0) as one integer max on the bit pattern: a float's sign bit makes
// every negative value (and -0) a negative int32, so they become +0 and
// everything else passes unchanged. fmaxf on a value the compiler cannot
// prove quiet costs an extra canonicalizing max in IEEE mode.
__device__ __forceinline__ float relu_bits(float x) {
  const int v = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(float, v > 0 ? v : 0);
}

// ---------------------------------------------------------------- top-k keys
// Order-preserving map of a finite float to uint32 (larger float -> larger
// key); -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) == 0) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Key of a score rounded to bfloat16 (nearest even), as a 32-bit key whose
// low 16 bits are zero: `key >> 16` orders the same way, so a selection can
// run on 16-bit keys and hand on `key16 << 16`.
__device__ __forceinline__ uint32_t score_key_bf16(float f) {
  return score_key(bf16_bits_to_f32(f32_to_bf16_bits(f))) & 0xFFFF0000u;
}

// Row stride, in elements, of a score matrix: N_cap for f32; for bf16 N_cap
// rounded up to even, so a 4-byte store of two neighbouring entries never
// crosses into the next row.
__host__ __device__ inline int64_t score_stride(int64_t N_cap, int sbf) { return sbf ? (N_cap + 1) & ~(int64_t)1 : N_cap; }

// 32-bit word a lane stores for its score v: the f32 bits, or for bf16 scores
// the pair (its entry, the next lane's entry), which the even lane of each
// pair stores (lanes 2i and 2i+1 hold neighbouring entries of one row). The
// lanes swap values with one DPP move (quad_perm [1,0,3,2]); every lane
// executes it.
__device__ __forceinline__ uint32_t score_word(float v, int sbf) {
  if (!sbf) return __builtin_bit_cast(uint32_t, v);
  const int nb = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false);
  return (uint32_t)f32_to_bf16_bits(v) | ((uint32_t)f32_to_bf16_bits(__builtin_bit_cast(float, nb)) << 16);
}

}  // namespace csa
