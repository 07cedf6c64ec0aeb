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
// Frequency of rotated pair i (0..31): 10000^(-i/32), in double.
__device__ __forceinline__ double rope_inv_freq(int i) {
  // log2(10000) = 13.287712379549449
  return exp2(-(double)i * (13.287712379549449 / 32.0));
}
// cos/sin of p * theta with the product and the reduction mod 2*pi in double,
// so positions up to 2^20 keep full float accuracy.
__device__ __forceinline__ void rope_cos_sin(int64_t p, double theta, float* c, float* s) {
  const double two_pi = 6.283185307179586476925;
  double a = (double)p * theta;
  double k = rint(a * (1.0 / two_pi));
  double r = fma(-k, two_pi, a);
  // second term of 2*pi (Cody-Waite) keeps the reduced angle exact to ~1e-16
  r = fma(-k, 2.4492935982947064e-16, r);
  float rf = (float)r;
  *s = sinf(rf);
  *c = cosf(rf);
}

// ---------------------------------------------------------------- top-k keys
// Order-preserving map of a finite float to uint32 (larger float -> larger
// key); -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) == 0) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace csa
