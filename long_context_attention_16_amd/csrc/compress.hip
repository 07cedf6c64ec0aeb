// K1 — KV compressor.
//
// Fold every m raw tokens' K and V into one compressed entry (CSA m = 4, HCA
// m' = 128): source "DeepSeek V4 重磅開源！…" (InfoQ), section 混合注意力機制.
// The pages give no folding rule; the one computed here is a softmax-gated
// weighted sum with one scalar gate per token, g_s = <w_gate, K_raw[s]>, the
// same weights for K and V, and RoPE applied to the folded key at the
// position of the block's last token.
//
// Design: one wavefront per block, one pass over the block's rows. For
// D = 512 each lane owns 8 contiguous channels, so every row is one fully
// coalesced 1 KB wave load (D = 128: see compress_d128_kernel). The softmax is evaluated online (running max and rescaled sums), so K
// and V are read from HBM exactly once; the kernel is a pure streaming kernel
// bound by HBM bandwidth.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

template <typename T, int VEC> struct RowIO;
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

  // One row of the online softmax fold (rows in order, so the result does
  // not depend on how many rows are loaded ahead).
  auto fold = [&](const float (&kv)[VEC], const float (&vv)[VEC]) {
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
  };
  // Rows four at a time: their loads are all issued before the first fold,
  // so a long block (m' = 128) keeps four rows per wave in flight instead of
  // one round trip per row.
  constexpr int kAhead = 4;
  int s = 0;
  for (; s + kAhead <= m; s += kAhead) {
    float kv[kAhead][VEC], vv[kAhead][VEC];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      RowIO<T, VEC>::load(kp + (int64_t)(s + u) * D, kv[u]);
      RowIO<T, VEC>::load(vp + (int64_t)(s + u) * D, vv[u]);
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) fold(kv[u], vv[u]);
  }
  for (; s < m; ++s) {
    float kv[VEC], vv[VEC];
    RowIO<T, VEC>::load(kp + (int64_t)s * D, kv);
    RowIO<T, VEC>::load(vp + (int64_t)s * D, vv);
    fold(kv, vv);
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

// D = 128: a row is 256 bytes (bf16), too short for one 16-byte load per lane
// of a wave, so a wave folds four blocks at once: the 16-lane group g = l / 16
// owns block 4w + g, lane l channels 8(l % 16) .. 8(l % 16) + 7. A wave load
// then reads one row of each of the four blocks (1 KB); gates are reduced
// inside each 16-lane group and every group runs its own online softmax.
constexpr int kD128BlocksPerWave = 4;
template <typename T>
__global__ __launch_bounds__(kCompressWaves * kWave) void compress_d128_kernel(
    int B, int T_, int m, int64_t pos0, int nb, const T* __restrict__ k_raw, const T* __restrict__ v_raw,
    const float* __restrict__ w_gate, T* __restrict__ k_c, T* __restrict__ v_c, int64_t N_cap) {
  constexpr int D = 128, VEC = 8;
  const int lane = threadIdx.x % kWave;
  const int64_t wv = (int64_t)blockIdx.x * kCompressWaves + threadIdx.x / kWave;
  const int64_t blk = wv * kD128BlocksPerWave + lane / 16;
  const bool live = blk < (int64_t)B * nb;
  // dead groups (past the last block) fold block 0 and store nothing
  const int b = live ? (int)(blk / nb) : 0;
  const int i = live ? (int)(blk % nb) : 0;
  const int c0 = (lane % 16) * VEC;

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
  auto fold = [&](const float (&kv)[VEC], const float (&vv)[VEC]) {
    float g = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) g = fmaf(wg[e], kv[e], g);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) g += __shfl_xor(g, o, kWave);  // sum over the group's 16 lanes
    const float nmax = fmaxf(run_max, g);
    const float scale = __expf(run_max - nmax);  // 0 on the first row
    const float p = __expf(g - nmax);
    run_sum = fmaf(run_sum, scale, p);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      ak[e] = fmaf(ak[e], scale, p * kv[e]);
      av[e] = fmaf(av[e], scale, p * vv[e]);
    }
    run_max = nmax;
  };
  constexpr int kAhead = 4;  // rows loaded before the first of them is folded
  int s = 0;
  for (; s + kAhead <= m; s += kAhead) {
    float kv[kAhead][VEC], vv[kAhead][VEC];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      RowIO<T, VEC>::load(kp + (int64_t)(s + u) * D, kv[u]);
      RowIO<T, VEC>::load(vp + (int64_t)(s + u) * D, vv[u]);
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) fold(kv[u], vv[u]);
  }
  for (; s < m; ++s) {
    float kv[VEC], vv[VEC];
    RowIO<T, VEC>::load(kp + (int64_t)s * D, kv);
    RowIO<T, VEC>::load(vp + (int64_t)s * D, vv);
    fold(kv, vv);
  }
  const float inv = 1.0f / run_sum;
#pragma unroll
  for (int e = 0; e < VEC; ++e) { ak[e] *= inv; av[e] *= inv; }
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
  if (!live) return;
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
  if (D == 128) {
    const int64_t waves = (total + kD128BlocksPerWave - 1) / kD128BlocksPerWave;
    const dim3 grid((unsigned)((waves + kCompressWaves - 1) / kCompressWaves));
    if (kv_dtype == 0)
      hipLaunchKernelGGL((compress_d128_kernel<float>), grid, block, 0, stream, B, T_, m, pos0, nb,
                         (const float*)k_raw, (const float*)v_raw, w_gate, (float*)k_c, (float*)v_c, N_cap);
    else
      hipLaunchKernelGGL((compress_d128_kernel<uint16_t>), grid, block, 0, stream, B, T_, m, pos0, nb,
                         (const uint16_t*)k_raw, (const uint16_t*)v_raw, w_gate, (uint16_t*)k_c, (uint16_t*)v_c,
                         N_cap);
  } else if (kv_dtype == 0) {
    CSA_LAUNCH_COMPRESS(float, 8);
  } else {
    CSA_LAUNCH_COMPRESS(uint16_t, 8);
  }
#undef CSA_LAUNCH_COMPRESS
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
