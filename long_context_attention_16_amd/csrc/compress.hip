// K1 — KV compressor.
//
// Fold every m raw tokens' K and V into one compressed entry (CSA m = 4, HCA
// m' = 128): source "DeepSeek V4 重磅開源！…" (InfoQ), section 混合注意力機制.
// The pages give no folding rule; the one computed here is a softmax-gated
// weighted sum with one scalar gate per token, g_s = <w_gate, K_raw[s]>, the
// same weights for K and V, and RoPE applied to the folded key at the
// position of the block's last token.
//
// Design: one wavefront per block, one pass over the block's rows. Each lane
// owns D/64 contiguous channels, so every row is one fully coalesced wave
// load. The softmax is evaluated online (running max and rescaled sums), so K
// and V are read from HBM exactly once; the kernel is a pure streaming kernel
// bound by HBM bandwidth.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

template <typename T, int VEC> struct RowIO;
template <> struct RowIO<float, 2> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    float2 x = *reinterpret_cast<const float2*>(p); v[0] = x.x; v[1] = x.y;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  }
};
template <> struct RowIO<float, 8> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};
template <> struct RowIO<uint16_t, 2> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
    uint32_t x = *reinterpret_cast<const uint32_t*>(p);
    v[0] = bf16_bits_to_f32((uint16_t)(x & 0xFFFF)); v[1] = bf16_bits_to_f32((uint16_t)(x >> 16));
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
    *reinterpret_cast<uint32_t*>(p) = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
  }
};
template <> struct RowIO<uint16_t, 8> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
    uint4 x = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32((uint16_t)(w[i] & 0xFFFF));
      v[2 * i + 1] = bf16_bits_to_f32((uint16_t)(w[i] >> 16));
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_bits(v[2 * i]) | ((uint32_t)f32_to_bf16_bits(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

constexpr int kCompressWaves = 4;

template <typename T, int VEC>
__global__ __launch_bounds__(kCompressWaves * kWave) void compress_kernel(
    int B, int T_, int m, int64_t pos0, int nb, const T* __restrict__ k_raw,
    const T* __restrict__ v_raw, const float* __restrict__ w_gate, T* __restrict__ k_c,
    T* __restrict__ v_c, int64_t N_cap) {
  constexpr int D = VEC * kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t blk = (int64_t)blockIdx.x * kCompressWaves + threadIdx.x / kWave;
  if (blk >= (int64_t)B * nb) return;
  const int b = (int)(blk / nb);
  const int i = (int)(blk % nb);
  const int c0 = lane * VEC;

  float wg[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) wg[e] = w_gate[c0 + e];

  const int64_t row0 = (int64_t)b * T_ + (int64_t)i * m;
  const T* kp = k_raw + row0 * D + c0;
  const T* vp = v_raw + row0 * D + c0;

  float ak[VEC], av[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) { ak[e] = 0.f; av[e] = 0.f; }
  float run_max = -INFINITY, run_sum = 0.f;

  for (int s = 0; s < m; ++s) {
    float kv[VEC], vv[VEC];
    RowIO<T, VEC>::load(kp + (int64_t)s * D, kv);
    RowIO<T, VEC>::load(vp + (int64_t)s * D, vv);
    float g = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) g = fmaf(wg[e], kv[e], g);
    g = wave_sum(g);
    const float nmax = fmaxf(run_max, g);
    const float scale = __expf(run_max - nmax);   // 0 on the first row
    const float p = __expf(g - nmax);
    run_sum = fmaf(run_sum, scale, p);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      ak[e] = fmaf(ak[e], scale, p * kv[e]);
      av[e] = fmaf(av[e], scale, p * vv[e]);
    }
    run_max = nmax;
  }
  const float inv = 1.0f / run_sum;
#pragma unroll
  for (int e = 0; e < VEC; ++e) { ak[e] *= inv; av[e] *= inv; }

  // RoPE on the folded key at the block's last position.
  const int64_t j = pos0 / m + i;
  const int64_t p = j * m + m - 1;
  if (c0 >= D - kRopeDims) {
#pragma unroll
    for (int e = 0; e < VEC; e += 2) {
      const int pair = (c0 + e - (D - kRopeDims)) / 2;
      float cs, sn;
      rope_cos_sin(p, pair, &cs, &sn);
      const float x0 = ak[e], x1 = ak[e + 1];
      ak[e] = x0 * cs - x1 * sn;
      ak[e + 1] = x0 * sn + x1 * cs;
    }
  }
  const int64_t orow = (int64_t)b * N_cap + j;
  RowIO<T, VEC>::store(k_c + orow * D + c0, ak);
  RowIO<T, VEC>::store(v_c + orow * D + c0, av);
}

int launch_compress(int B, int T_, int D, int m, int64_t pos0, int kv_dtype, const void* k_raw,
                    const void* v_raw, const float* w_gate, void* k_c, void* v_c, int64_t N_cap,
                    hipStream_t stream) {
  const int nb = T_ / m;
  const int64_t total = (int64_t)B * nb;
  if (total == 0) return 0;
  const dim3 grid((unsigned)((total + kCompressWaves - 1) / kCompressWaves));
  const dim3 block(kCompressWaves * kWave);
#define CSA_LAUNCH_COMPRESS(TT, VV)                                                          \
  hipLaunchKernelGGL((compress_kernel<TT, VV>), grid, block, 0, stream, B, T_, m, pos0, nb, \
                     (const TT*)k_raw, (const TT*)v_raw, w_gate, (TT*)k_c, (TT*)v_c, N_cap)
  if (kv_dtype == 0) {
    if (D == 128) CSA_LAUNCH_COMPRESS(float, 2); else CSA_LAUNCH_COMPRESS(float, 8);
  } else {
    if (D == 128) CSA_LAUNCH_COMPRESS(uint16_t, 2); else CSA_LAUNCH_COMPRESS(uint16_t, 8);
  }
#undef CSA_LAUNCH_COMPRESS
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
