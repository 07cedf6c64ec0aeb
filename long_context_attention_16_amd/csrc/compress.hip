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

template <> struct RowIO<float, 2> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    const float2 a = *reinterpret_cast<const float2*>(p);
    v[0] = a.x; v[1] = a.y;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  }
};
template <> struct RowIO<uint16_t, 2> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    v[0] = bf16_bits_to_f32((uint16_t)(w & 0xFFFF));
    v[1] = bf16_bits_to_f32((uint16_t)(w >> 16));
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
    *reinterpret_cast<uint32_t*>(p) = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
  }
};

// e4m3fn code of x: round to nearest even on the grid of x's binary exponent
// (3 mantissa bits; the subnormal step 2^-9 below 2^-6), every magnitude
// above 448 saturating to 448; the sign bit is x's.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  int e;
  frexpf(a, &e);                                  // a = f * 2^e, f in [0.5, 1)
  const int ge = a < 0.015625f ? -6 : e - 1;      // grid exponent
  const float q = rintf(ldexpf(a, 3 - ge));       // multiples of 2^(ge - 3), 0 .. 16
  // q in [8, 16] for a normal grid (16 carries into the next exponent),
  // [0, 8] on the subnormal grid; both map to 8 * ge + 48 + q
  return sign | (uint32_t)(8 * ge + 48 + (int)q);
}

// e2m1 code of x (already divided by its scale): nearest of 0, 0.5, 1, 1.5,
// 2, 3, 4, 6, ties to the even code, saturating at 6; the sign bit is x's.
// The thresholds are the midpoints, each strict or not by the tie rule.
__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
  const float a = fabsf(x);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.f);
  return c | ((__builtin_bit_cast(uint32_t, x) >> 28) & 0x8u);
}

// Stores the folded indexer-key pair (x0, x1), channels c and c + 1 of
// compressed row orow, in format fmt: f32, bf16 (nearest even), e4m3fn, or
// MXFP4 (two e2m1 codes in one byte plus the e8m0 scale of the 32-element
// block, floor(log2 amax) - 2 + 127 clamped to 0..254, 0 for an all-zero
// block). For MXFP4 the 16 pairs of a block are held by the 16 lanes of one
// aligned 16-lane group, which reduce its amax together: every lane of the
// group calls this (fmt is uniform); st says whether this lane stores.
__device__ __forceinline__ void store_index_key(int fmt, void* ki_c, uint8_t* ki_sc, int64_t orow, int d_i, int c,
                                                float x0, float x1, bool st) {
  if (fmt == 0) {
    if (st) *reinterpret_cast<float2*>((float*)ki_c + orow * d_i + c) = make_float2(x0, x1);
  } else if (fmt == 1) {
    if (st)
      *reinterpret_cast<uint32_t*>((uint16_t*)ki_c + orow * d_i + c) =
          (uint32_t)f32_to_bf16_bits(x0) | ((uint32_t)f32_to_bf16_bits(x1) << 16);
  } else if (fmt == 2) {
    if (st)
      *reinterpret_cast<uint16_t*>((uint8_t*)ki_c + orow * d_i + c) =
          (uint16_t)(f32_to_e4m3(x0) | (f32_to_e4m3(x1) << 8));
  } else {
    float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    int e;
    frexpf(amax, &e);
    const int code = amax > 0.f ? min(max(e + 124, 0), 254) : 0;
    const float y0 = ldexpf(x0, 127 - code), y1 = ldexpf(x1, 127 - code);
    if (st) {
      ((uint8_t*)ki_c)[orow * (d_i / 2) + c / 2] = (uint8_t)(f32_to_e2m1(y0) | (f32_to_e2m1(y1) << 4));
      if (c % 32 == 0) ki_sc[orow * (d_i / 32) + c / 32] = (uint8_t)code;
    }
  }
}

// Optional indexer-key fold of the batch compressor: raw rows [B, T, d_i]
// in the KV dtype, folded rows [B, N_cap, d_i] in idx_fmt (d_i = 0: none).
struct IndexKeyFold {
  int d_i, idx_fmt;
  const void* ki_raw;
  void* ki_c;
  uint8_t* ki_sc;
};

constexpr int kCompressWaves = 4;

template <typename T, int VEC>
__global__ __launch_bounds__(kCompressWaves * kWave) void compress_kernel(
    int B, int T_, int m, int64_t pos0, int nb, const T* __restrict__ k_raw,
    const T* __restrict__ v_raw, const float* __restrict__ w_gate, T* __restrict__ k_c,
    T* __restrict__ v_c, int64_t N_cap, IndexKeyFold ik) {
  constexpr int D = VEC * kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t blk = (int64_t)blockIdx.x * kCompressWaves + threadIdx.x / kWave;
  if (blk >= (int64_t)B * nb) return;
  const int b = (int)(blk / nb);
  const int i = (int)(blk % nb);
  const int c0 = lane * VEC;
  const bool xl = lane < ik.d_i / 2;  // lane folds indexer-key channels 2 lane, 2 lane + 1

  float wg[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) wg[e] = w_gate[c0 + e];

  const int64_t row0 = (int64_t)b * T_ + (int64_t)i * m;
  const T* kp = k_raw + row0 * D + c0;
  const T* vp = v_raw + row0 * D + c0;
  const T* xp = (const T*)ik.ki_raw + row0 * ik.d_i + 2 * lane;

  float ak[VEC], av[VEC], ax[2] = {0.f, 0.f};
#pragma unroll
  for (int e = 0; e < VEC; ++e) { ak[e] = 0.f; av[e] = 0.f; }
  float run_max = -INFINITY, run_sum = 0.f;

  // One row of the online softmax fold (rows in order, so the result does
  // not depend on how many rows are loaded ahead).
  auto fold = [&](const float (&kv)[VEC], const float (&vv)[VEC], const float (&xv)[2]) {
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
    ax[0] = fmaf(ax[0], scale, p * xv[0]);
    ax[1] = fmaf(ax[1], scale, p * xv[1]);
    run_max = nmax;
  };
  // Rows four at a time: their loads are all issued before the first fold,
  // so a long block (m' = 128) keeps four rows per wave in flight instead of
  // one round trip per row.
  constexpr int kAhead = 4;
  int s = 0;
  for (; s + kAhead <= m; s += kAhead) {
    float kv[kAhead][VEC], vv[kAhead][VEC], xv[kAhead][2];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      RowIO<T, VEC>::load(kp + (int64_t)(s + u) * D, kv[u]);
      RowIO<T, VEC>::load(vp + (int64_t)(s + u) * D, vv[u]);
      xv[u][0] = 0.f; xv[u][1] = 0.f;
      if (xl) RowIO<T, 2>::load(xp + (int64_t)(s + u) * ik.d_i, xv[u]);
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) fold(kv[u], vv[u], xv[u]);
  }
  for (; s < m; ++s) {
    float kv[VEC], vv[VEC], xv[2] = {0.f, 0.f};
    RowIO<T, VEC>::load(kp + (int64_t)s * D, kv);
    RowIO<T, VEC>::load(vp + (int64_t)s * D, vv);
    if (xl) RowIO<T, 2>::load(xp + (int64_t)s * ik.d_i, xv);
    fold(kv, vv, xv);
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
  // the indexer key: the same weights, unrotated, in the indexer's format
  if (ik.d_i > 0) store_index_key(ik.idx_fmt, ik.ki_c, ik.ki_sc, orow, ik.d_i, 2 * lane, ax[0] * inv, ax[1] * inv, xl);
}

// D = 128: a row is 256 bytes (bf16), too short for one 16-byte load per lane
// of a wave, so a wave folds four blocks at once: the 16-lane group g = l / 16
// owns block 4w + g, lane l channels 8(l % 16) .. 8(l % 16) + 7. A wave load
// then reads one row of each of the four blocks (1 KB); gates are reduced
// inside each 16-lane group and every group runs its own online softmax.
// The indexer key (d_i = 32, 64 or 128) is folded by the same group: lane l
// owns the channel pairs 32 r + 2 (l % 16), +1 for r < d_i / 32, so each
// 32-element block of the key lies in one group (MXFP4's scale block).
constexpr int kD128BlocksPerWave = 4;
constexpr int kXPairs = 4;  // indexer-key channel pairs per lane at d_i = 128
template <typename T>
__global__ __launch_bounds__(kCompressWaves * kWave) void compress_d128_kernel(
    int B, int T_, int m, int64_t pos0, int nb, const T* __restrict__ k_raw, const T* __restrict__ v_raw,
    const float* __restrict__ w_gate, T* __restrict__ k_c, T* __restrict__ v_c, int64_t N_cap, IndexKeyFold ik) {
  constexpr int D = 128, VEC = 8;
  const int lane = threadIdx.x % kWave;
  const int64_t wv = (int64_t)blockIdx.x * kCompressWaves + threadIdx.x / kWave;
  const int64_t blk = wv * kD128BlocksPerWave + lane / 16;
  const bool live = blk < (int64_t)B * nb;
  // dead groups (past the last block) fold block 0 and store nothing
  const int b = live ? (int)(blk / nb) : 0;
  const int i = live ? (int)(blk % nb) : 0;
  const int c0 = (lane % 16) * VEC;
  const int nxp = ik.d_i / 32;  // channel pairs per lane (uniform)

  float wg[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) wg[e] = w_gate[c0 + e];
  const int64_t row0 = (int64_t)b * T_ + (int64_t)i * m;
  const T* kp = k_raw + row0 * D + c0;
  const T* vp = v_raw + row0 * D + c0;
  const T* xp = (const T*)ik.ki_raw + row0 * ik.d_i + 2 * (lane % 16);
  float ak[VEC], av[VEC], ax[kXPairs][2];
#pragma unroll
  for (int e = 0; e < VEC; ++e) { ak[e] = 0.f; av[e] = 0.f; }
#pragma unroll
  for (int r = 0; r < kXPairs; ++r) { ax[r][0] = 0.f; ax[r][1] = 0.f; }
  float run_max = -INFINITY, run_sum = 0.f;
  auto fold = [&](const float (&kv)[VEC], const float (&vv)[VEC], const float (&xv)[kXPairs][2]) {
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
#pragma unroll
    for (int r = 0; r < kXPairs; ++r) {
      ax[r][0] = fmaf(ax[r][0], scale, p * xv[r][0]);
      ax[r][1] = fmaf(ax[r][1], scale, p * xv[r][1]);
    }
    run_max = nmax;
  };
  auto load_x = [&](int64_t s_, float (&xv)[kXPairs][2]) {
#pragma unroll
    for (int r = 0; r < kXPairs; ++r) {
      xv[r][0] = 0.f; xv[r][1] = 0.f;
      if (r < nxp) RowIO<T, 2>::load(xp + s_ * ik.d_i + 32 * r, xv[r]);
    }
  };
  constexpr int kAhead = 4;  // rows loaded before the first of them is folded
  int s = 0;
  for (; s + kAhead <= m; s += kAhead) {
    float kv[kAhead][VEC], vv[kAhead][VEC], xv[kAhead][kXPairs][2];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      RowIO<T, VEC>::load(kp + (int64_t)(s + u) * D, kv[u]);
      RowIO<T, VEC>::load(vp + (int64_t)(s + u) * D, vv[u]);
      load_x(s + u, xv[u]);
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) fold(kv[u], vv[u], xv[u]);
  }
  for (; s < m; ++s) {
    float kv[VEC], vv[VEC], xv[kXPairs][2];
    RowIO<T, VEC>::load(kp + (int64_t)s * D, kv);
    RowIO<T, VEC>::load(vp + (int64_t)s * D, vv);
    load_x(s, xv);
    fold(kv, vv, xv);
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
  const int64_t orow = (int64_t)b * N_cap + j;
  // every lane of a group reaches the MXFP4 amax reduction (live is uniform
  // per group)
#pragma unroll
  for (int r = 0; r < kXPairs; ++r)
    if (r < nxp)
      store_index_key(ik.idx_fmt, ik.ki_c, ik.ki_sc, orow, ik.d_i, 32 * r + 2 * (lane % 16), ax[r][0] * inv,
                      ax[r][1] * inv, live);
  if (!live) return;
  RowIO<T, VEC>::store(k_c + orow * D + c0, ak);
  RowIO<T, VEC>::store(v_c + orow * D + c0, av);
}

// ------------------------------------------------------------ state append
//
// One decode step of the state cache: the token at position t = pos[b] of
// each sequence enters slot t % R of the sequence's ring of raw rows (K, V
// and the indexer's raw key); when it completes a block (t + 1 a multiple of
// m) the block's m rows are folded into entry j = (t + 1) / m - 1 exactly as
// compress_kernel folds a block (same online softmax, RoPE at position t),
// and the indexer key is folded with the same weights, unrotated, and stored
// in the indexer's format. Source: "DeepSeek V4 重磅開源！…" (InfoQ), section
// 框架層優化 (a state cache of window tokens and not-yet-compressed tokens,
// kept apart from the compressed KV cache), and section 混合注意力機制 (an
// entry exists once its block is complete).
//
// One wave per sequence: lane l owns channels VEC*l .. VEC*l + VEC - 1 of
// the K and V rows (VEC = D / 64) and channels 2l, 2l + 1 of the indexer key
// (lanes l < d_i / 2). The token's own row is folded from registers, not
// read back from the ring.

struct StateArgs {
  int B, m, R, d_i, idx_fmt;
  int64_t N_cap;
  const int64_t* pos;
  const void *k_new, *v_new, *ki_new;
  const float* w_gate;
  void *k_ring, *v_ring, *ki_ring, *k_c, *v_c, *ki_c;
  uint8_t* ki_sc;
};

constexpr int kAppendWaves = 4;

template <typename T, int VEC>
__global__ __launch_bounds__(kAppendWaves * kWave) void state_append_kernel(StateArgs a) {
  constexpr int D = VEC * kWave;
  const int lane = threadIdx.x % kWave;
  const int b = blockIdx.x * kAppendWaves + threadIdx.x / kWave;
  if (b >= a.B) return;
  const int64_t t = a.pos[b];
  if (t < 0) return;  // an inactive slot of the batch
  const int c0 = lane * VEC;
  const bool xl = lane < a.d_i / 2;  // lane holds indexer-key channels
  const T* kn_p = (const T*)a.k_new + (int64_t)b * D + c0;
  const T* vn_p = (const T*)a.v_new + (int64_t)b * D + c0;
  const int64_t slot_t = t % a.R;
  T* kr = (T*)a.k_ring + (int64_t)b * a.R * D + c0;
  T* vr = (T*)a.v_ring + (int64_t)b * a.R * D + c0;
  T* xr = (T*)a.ki_ring + (int64_t)b * a.R * a.d_i + 2 * lane;
  float kn[VEC], vn[VEC], xn[2] = {0.f, 0.f};
  RowIO<T, VEC>::load(kn_p, kn);
  RowIO<T, VEC>::load(vn_p, vn);
  if (xl) RowIO<T, 2>::load((const T*)a.ki_new + (int64_t)b * a.d_i + 2 * lane, xn);
  RowIO<T, VEC>::store(kr + slot_t * D, kn);
  RowIO<T, VEC>::store(vr + slot_t * D, vn);
  if (xl) RowIO<T, 2>::store(xr + slot_t * a.d_i, xn);

  const int m = a.m;
  if ((t + 1) % m != 0) return;  // no block completed
  const int64_t j = (t + 1) / m - 1;
  if (j >= a.N_cap) return;

  float wg[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) wg[e] = a.w_gate[c0 + e];
  float ak[VEC], av[VEC], ax[2] = {0.f, 0.f};
#pragma unroll
  for (int e = 0; e < VEC; ++e) { ak[e] = 0.f; av[e] = 0.f; }
  float run_max = -INFINITY, run_sum = 0.f;
  auto fold = [&](const float (&kv)[VEC], const float (&vv)[VEC], const float (&xv)[2]) {
    float g = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) g = fmaf(wg[e], kv[e], g);
    g = wave_sum(g);
    const float nmax = fmaxf(run_max, g);
    const float scale = __expf(run_max - nmax);  // 0 on the first row
    const float p = __expf(g - nmax);
    run_sum = fmaf(run_sum, scale, p);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      ak[e] = fmaf(ak[e], scale, p * kv[e]);
      av[e] = fmaf(av[e], scale, p * vv[e]);
    }
    ax[0] = fmaf(ax[0], scale, p * xv[0]);
    ax[1] = fmaf(ax[1], scale, p * xv[1]);
    run_max = nmax;
  };
  // rows t - m + 1 .. t - 1 from the ring in batches of four, all four
  // loaded before the first is folded (one round trip for m = 4); the rows of
  // a batch past the block read a valid slot and are not folded. Then the
  // new row.
  int64_t slot = (t - m + 1) % a.R;
  auto next = [&](int64_t sl) { return sl + 1 == a.R ? (int64_t)0 : sl + 1; };
  constexpr int kAhead = 4;
  for (int s = 0; s < m - 1; s += kAhead) {
    const int cnt = min(kAhead, m - 1 - s);
    float kv[kAhead][VEC], vv[kAhead][VEC], xv[kAhead][2];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      RowIO<T, VEC>::load(kr + slot * D, kv[u]);
      RowIO<T, VEC>::load(vr + slot * D, vv[u]);
      xv[u][0] = 0.f; xv[u][1] = 0.f;
      if (xl) RowIO<T, 2>::load(xr + slot * a.d_i, xv[u]);
      slot = next(slot);
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u)
      if (u < cnt) fold(kv[u], vv[u], xv[u]);
  }
  fold(kn, vn, xn);
  const float inv = 1.0f / run_sum;
#pragma unroll
  for (int e = 0; e < VEC; ++e) { ak[e] *= inv; av[e] *= inv; }
  ax[0] *= inv;
  ax[1] *= inv;
  if (c0 >= D - kRopeDims) {  // RoPE on the folded key at the block's last position t
#pragma unroll
    for (int e = 0; e < VEC; e += 2) {
      const int pair = (c0 + e - (D - kRopeDims)) / 2;
      float cs, sn;
      rope_cos_sin(t, pair, &cs, &sn);
      const float x0 = ak[e], x1 = ak[e + 1];
      ak[e] = x0 * cs - x1 * sn;
      ak[e + 1] = x0 * sn + x1 * cs;
    }
  }
  const int64_t orow = (int64_t)b * a.N_cap + j;
  RowIO<T, VEC>::store((T*)a.k_c + orow * D + c0, ak);
  RowIO<T, VEC>::store((T*)a.v_c + orow * D + c0, av);
  if (a.d_i == 0) return;
  // the indexer key in its storage format
  store_index_key(a.idx_fmt, a.ki_c, a.ki_sc, orow, a.d_i, 2 * lane, ax[0], ax[1], xl);
}

int launch_state_append(int B, int D, int m, int R, int kv_dtype, const int64_t* pos, const void* k_new,
                        const void* v_new, const float* w_gate, void* k_ring, void* v_ring, void* k_c, void* v_c,
                        int64_t N_cap, int d_i, int idx_fmt, const void* ki_new, void* ki_ring, void* ki_c,
                        uint8_t* ki_c_scale, hipStream_t stream) {
  if (B == 0) return 0;
  StateArgs a{};
  a.B = B; a.m = m; a.R = R; a.d_i = d_i; a.idx_fmt = idx_fmt; a.N_cap = N_cap; a.pos = pos;
  a.k_new = k_new; a.v_new = v_new; a.ki_new = ki_new; a.w_gate = w_gate;
  a.k_ring = k_ring; a.v_ring = v_ring; a.ki_ring = ki_ring; a.k_c = k_c; a.v_c = v_c; a.ki_c = ki_c;
  a.ki_sc = ki_c_scale;
  const dim3 grid((unsigned)((B + kAppendWaves - 1) / kAppendWaves)), block(kAppendWaves * kWave);
  if (kv_dtype == 0) {
    if (D == 128) hipLaunchKernelGGL((state_append_kernel<float, 2>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((state_append_kernel<float, 8>), grid, block, 0, stream, a);
  } else {
    if (D == 128) hipLaunchKernelGGL((state_append_kernel<uint16_t, 2>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((state_append_kernel<uint16_t, 8>), grid, block, 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

int launch_compress(int B, int T_, int D, int m, int64_t pos0, int kv_dtype, const void* k_raw,
                    const void* v_raw, const float* w_gate, void* k_c, void* v_c, int64_t N_cap, int d_i,
                    int idx_fmt, const void* ki_raw, void* ki_c, uint8_t* ki_c_scale, hipStream_t stream) {
  const int nb = T_ / m;
  const int64_t total = (int64_t)B * nb;
  if (total == 0) return 0;
  IndexKeyFold ik{d_i, idx_fmt, ki_raw, ki_c, ki_c_scale};
  const dim3 grid((unsigned)((total + kCompressWaves - 1) / kCompressWaves));
  const dim3 block(kCompressWaves * kWave);
#define CSA_LAUNCH_COMPRESS(TT, VV)                                                          \
  hipLaunchKernelGGL((compress_kernel<TT, VV>), grid, block, 0, stream, B, T_, m, pos0, nb, \
                     (const TT*)k_raw, (const TT*)v_raw, w_gate, (TT*)k_c, (TT*)v_c, N_cap, ik)
  if (D == 128) {
    const int64_t waves = (total + kD128BlocksPerWave - 1) / kD128BlocksPerWave;
    const dim3 grid((unsigned)((waves + kCompressWaves - 1) / kCompressWaves));
    if (kv_dtype == 0)
      hipLaunchKernelGGL((compress_d128_kernel<float>), grid, block, 0, stream, B, T_, m, pos0, nb,
                         (const float*)k_raw, (const float*)v_raw, w_gate, (float*)k_c, (float*)v_c, N_cap, ik);
    else
      hipLaunchKernelGGL((compress_d128_kernel<uint16_t>), grid, block, 0, stream, B, T_, m, pos0, nb,
                         (const uint16_t*)k_raw, (const uint16_t*)v_raw, w_gate, (uint16_t*)k_c, (uint16_t*)v_c,
                         N_cap, ik);
  } else if (kv_dtype == 0) {
    CSA_LAUNCH_COMPRESS(float, 8);
  } else {
    CSA_LAUNCH_COMPRESS(uint16_t, 8);
  }
#undef CSA_LAUNCH_COMPRESS
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
