// K4 / K5 — compressed attention with sliding window and attention sink.
//
// Source: "DeepSeek V4 重磅開源！…" (InfoQ), section 混合注意力機制: CSA attends
// the k compressed entries chosen per query, HCA attends every compressed
// entry (m' = 128) densely; both rotate only the last 64 dims (RoPE), add a
// sliding-window branch over raw recent tokens, and carry an attention sink so
// a query's weights may add up to less than one. Form taken (the pages give
// no formula): one softmax over compressed rows and window rows
// s = max(0, t-W+1) .. t, logits <RoPE(q, t), key> / sqrt(D), and a per-head
// sink logit that joins only the denominator.
//
// Design (MQA: one KV head shared by H query heads):
//  * one workgroup per (query, split of its source list); NW = ceil(H/16)
//    waves, wave w owning heads 16w .. 16w+15;
//  * 32 source rows per tile are gathered (CSA: rows named by idx; HCA:
//    consecutive rows; window: raw rows, rotated while staged) into LDS. K is
//    kept row-major; V is stored transposed with its rows permuted so that a
//    lane's 8 PV k-values are one 16-byte LDS read;
//  * S^T = K Q^T and O^T = V^T P^T on MFMA 16x16 (bf16: 16x16x32; f32:
//    16x16x4), so a lane's accumulators all belong to one head and the online
//    softmax rescale is one multiply per register;
//  * the split count depends only on the query's own source count, never on
//    the batch, so results are batch-invariant and deterministic; a separate
//    combine kernel merges the splits in a fixed order.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Chunk;  // one 16-byte chunk of a row
template <> struct Chunk<uint16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const uint4& r, float* v) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32((uint16_t)(w[i] & 0xFFFF));
      v[2 * i + 1] = bf16_bits_to_f32((uint16_t)(w[i] >> 16));
    }
  }
  static __device__ __forceinline__ uint4 pack(const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_bits(v[2 * i]) | ((uint32_t)f32_to_bf16_bits(v[2 * i + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct Chunk<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(const uint4& r, float* v) {
    v[0] = __builtin_bit_cast(float, r.x); v[1] = __builtin_bit_cast(float, r.y);
    v[2] = __builtin_bit_cast(float, r.z); v[3] = __builtin_bit_cast(float, r.w);
  }
  static __device__ __forceinline__ uint4 pack(const float* v) {
    return make_uint4(__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                      __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3]));
  }
};

// Rotate the pairs of a 16-byte chunk starting at dim d0 (RoPE at position pos).
template <typename T, int D>
__device__ __forceinline__ uint4 rope_chunk(uint4 raw, int d0, int64_t pos) {
  if (d0 < D - kRopeDims) return raw;
  float v[Chunk<T>::N];
  Chunk<T>::unpack(raw, v);
#pragma unroll
  for (int e = 0; e < Chunk<T>::N; e += 2) {
    const int pair = (d0 + e - (D - kRopeDims)) / 2;
    float c, s;
    rope_cos_sin(pos, rope_inv_freq(pair), &c, &s);
    const float x0 = v[e], x1 = v[e + 1];
    v[e] = x0 * c - x1 * s;
    v[e + 1] = x0 * s + x1 * c;
  }
  return Chunk<T>::pack(v);
}

template <typename T, int D, int NW, bool HCA>
__global__ __launch_bounds__(NW * kWave) void attn_kernel(AttnArgs p) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int NT = NW * kWave;
  constexpr int KSTR = D + (BF ? 8 : 4);  // K row stride (elements)
  constexpr int VTSTR = 36;               // bf16 V^T row stride: 32 rows + 4 pad
  constexpr int VSTR = D + 4;             // f32 V row stride
  constexpr int EPC = Chunk<T>::N;
  constexpr int CPR = D / EPC;
  __shared__ __attribute__((aligned(16))) T Ks[32 * KSTR];
  __shared__ __attribute__((aligned(16))) T Vs[BF ? D * VTSTR : 32 * VSTR];
  __shared__ int64_t row_off[32];
  __shared__ int64_t row_pos[32];
  __shared__ int row_kind[32];  // 0: no row (masked), 1: compressed entry, 2: raw window row

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int g = lane / 16, l16 = lane % 16;
  const int qrow = blockIdx.x / p.nsplit_max;
  const int split = blockIdx.x % p.nsplit_max;
  const int b = qrow / p.Lq, i = qrow % p.Lq;
  const int64_t t = p.q_pos0 + i;
  const int n_c = HCA ? (int)((t + 1) / p.m) : p.topk;
  const int64_t lo = t - p.W + 1 > 0 ? t - p.W + 1 : 0;
  const int n_w = p.W > 0 ? (int)(t - lo + 1) : 0;
  const int S = n_c + p.W;
  const int CH = attn_split_rows(S);
  const int nsplit = attn_nsplit(S);
  if (split >= nsplit) return;
  const int s0 = split * CH;
  const int s1 = min(S, s0 + CH);

  const int h = wave * 16 + l16;
  const bool hok = h < p.H;
  const T* qbase = (const T*)p.q + ((int64_t)qrow * p.H + (hok ? h : 0)) * D;

  // Q fragments (B operand of S^T = K Q^T), rotated at t.
  typedef typename std::conditional<BF, bf16x8, float>::type QFrag;
  constexpr int QN = BF ? D / 32 : D / 4;
  QFrag qf[QN];
  if constexpr (BF) {
#pragma unroll
    for (int s = 0; s < QN; ++s) {
      const int d0 = 32 * s + 8 * g;
      uint4 raw = hok ? *reinterpret_cast<const uint4*>(qbase + d0) : make_uint4(0, 0, 0, 0);
      raw = rope_chunk<T, D>(raw, d0, t);
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  } else {
#pragma unroll
    for (int u = 0; u < D / 8; ++u) {
      const int d0 = 8 * u + 2 * g;
      float2 x = hok ? *reinterpret_cast<const float2*>(qbase + d0) : make_float2(0.f, 0.f);
      if (d0 >= D - kRopeDims) {
        float c, s;
        rope_cos_sin(t, rope_inv_freq((d0 - (D - kRopeDims)) / 2), &c, &s);
        const float x0 = x.x, x1 = x.y;
        x.x = x0 * c - x1 * s;
        x.y = x0 * s + x1 * c;
      }
      qf[2 * u] = x.x;
      qf[2 * u + 1] = x.y;
    }
  }

  const float cscale = kLog2e / sqrtf((float)D);
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const T* kc = (const T*)p.k_c;
  const T* vc = (const T*)p.v_c;
  const T* kr = (const T*)p.k_raw;
  const T* vr = (const T*)p.v_raw;

  for (int ts = s0; ts < s1; ts += 32) {
    if (tid < 32) {
      const int sp = ts + tid;
      int kind = 0;
      int64_t off = 0, pos = 0;
      if (sp < s1) {
        if (sp < n_c) {
          const int64_t j = HCA ? (int64_t)sp : (int64_t)p.idx[(int64_t)qrow * p.topk + sp];
          if (j >= 0 && j < p.N_cap) { kind = 1; off = ((int64_t)b * p.N_cap + j) * D; }
        } else {
          const int w = sp - n_c;
          if (w < n_w) {
            kind = 2;
            pos = lo + w;
            off = ((int64_t)b * p.T_raw + (pos - p.raw_pos0)) * D;
          }
        }
      }
      row_kind[tid] = kind;
      row_off[tid] = off;
      row_pos[tid] = pos;
    }
    __syncthreads();

    for (int c = tid; c < 32 * CPR; c += NT) {
      const int r = c / CPR;
      const int d0 = (c % CPR) * EPC;
      const int kind = row_kind[r];
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (kind) {
        const int64_t off = row_off[r] + d0;
        kv = *reinterpret_cast<const uint4*>((kind == 1 ? kc : kr) + off);
        vv = *reinterpret_cast<const uint4*>((kind == 1 ? vc : vr) + off);
        if (kind == 2) kv = rope_chunk<T, D>(kv, d0, row_pos[r]);
      }
      *reinterpret_cast<uint4*>(&Ks[r * KSTR + d0]) = kv;
      if constexpr (BF) {
        const int pr = 8 * ((r % 16) / 4) + 4 * (r / 16) + (r % 4);
        const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          Vs[(d0 + e) * VTSTR + pr] = (uint16_t)((e & 1) ? (w[e / 2] >> 16) : (w[e / 2] & 0xFFFF));
      } else {
        *reinterpret_cast<uint4*>(&Vs[r * VSTR + d0]) = vv;
      }
    }
    __syncthreads();

    // S^T tiles: rows 16*rt + (4g + r), column = head.
    f32x4 sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const T* krow = &Ks[(16 * rt + l16) * KSTR];
      if constexpr (BF) {
#pragma unroll
        for (int s = 0; s < QN; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 32 * s + 8 * g);
          sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sacc[rt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int u = 0; u < D / 8; ++u) {
          const float2 kk = *reinterpret_cast<const float2*>(krow + 8 * u + 2 * g);
          sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.x, qf[2 * u], sacc[rt], 0, 0, 0);
          sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.y, qf[2 * u + 1], sacc[rt], 0, 0, 0);
        }
      }
    }
    float x[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = row_kind[16 * rt + 4 * g + r] != 0;
        x[rt][r] = ok ? sacc[rt][r] * cscale : -INFINITY;
        tmax = fmaxf(tmax, x[rt][r]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[rt][r] = none ? 0.f : exp2f(x[rt][r] - m_new);
        psum += x[rt][r];
      }
    psum += __shfl_xor(psum, 16, kWave);
    psum += __shfl_xor(psum, 32, kWave);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] *= alpha;

    if constexpr (BF) {
      const float pv[8] = {x[0][0], x[0][1], x[0][2], x[0][3], x[1][0], x[1][1], x[1][2], x[1][3]};
      const bf16x8 pf = __builtin_bit_cast(bf16x8, Chunk<uint16_t>::pack(pv));
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&Vs[(16 * dt + l16) * VTSTR + 8 * g]);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[dt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float* vrow = reinterpret_cast<const float*>(&Vs[(16 * rt + 4 * g + r) * VSTR]);
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt)
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * dt + l16], x[rt][r], acc[dt], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  if (!hok) return;
  if (nsplit == 1) {
    const float z2 = p.sink ? p.sink[h] * kLog2e : -INFINITY;
    const float M = fmaxf(z2, m_run);
    float f = 0.f, lse2 = -INFINITY;
    if (M != -INFINITY) {
      const float den = exp2f(z2 - M) + l_run * exp2f(m_run - M);
      f = exp2f(m_run - M) / den;
      lse2 = M + log2f(den);
    }
    T* orow = (T*)p.out + ((int64_t)qrow * p.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int d = 16 * dt + 4 * g;
      if constexpr (BF) {
        const uint32_t lo2 = (uint32_t)f32_to_bf16_bits(acc[dt][0] * f) | ((uint32_t)f32_to_bf16_bits(acc[dt][1] * f) << 16);
        const uint32_t hi2 = (uint32_t)f32_to_bf16_bits(acc[dt][2] * f) | ((uint32_t)f32_to_bf16_bits(acc[dt][3] * f) << 16);
        *reinterpret_cast<uint2*>(orow + d) = make_uint2(lo2, hi2);
      } else {
        *reinterpret_cast<float4*>(orow + d) = make_float4(acc[dt][0] * f, acc[dt][1] * f, acc[dt][2] * f, acc[dt][3] * f);
      }
    }
    if (p.lse && g == 0) p.lse[(int64_t)qrow * p.H + h] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  } else {
    const int64_t slot = ((int64_t)qrow * p.nsplit_max + split) * p.H + h;
    float* po = p.ws_o + slot * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (g == 0) *reinterpret_cast<float2*>(p.ws_ml + slot * 2) = make_float2(m_run, l_run);
  }
}

// Merge the splits of one (query, head): fixed split order.
template <typename T, int D, bool HCA>
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs p) {
  const int qrow = blockIdx.x / p.H;
  const int h = blockIdx.x % p.H;
  const int i = qrow % p.Lq;
  const int64_t t = p.q_pos0 + i;
  const int n_c = HCA ? (int)((t + 1) / p.m) : p.topk;
  const int nsplit = attn_nsplit(n_c + p.W);
  if (nsplit == 1) return;
  const int64_t slot0 = ((int64_t)qrow * p.nsplit_max) * p.H + h;
  const float z2 = p.sink ? p.sink[h] * kLog2e : -INFINITY;
  float M = z2;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, p.ws_ml[(slot0 + (int64_t)s * p.H) * 2]);
  float den = 0.f;
  if (M != -INFINITY) {
    den = exp2f(z2 - M);
    for (int s = 0; s < nsplit; ++s) {
      const float2 ml = *reinterpret_cast<const float2*>(p.ws_ml + (slot0 + (int64_t)s * p.H) * 2);
      den += ml.y * exp2f(ml.x - M);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  T* orow = (T*)p.out + ((int64_t)qrow * p.H + h) * D;
  for (int d = threadIdx.x * 4; d < D; d += 128 * 4) {
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
      for (int s = 0; s < nsplit; ++s) {
        const int64_t slot = slot0 + (int64_t)s * p.H;
        const float ms = p.ws_ml[slot * 2];
        const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - M) * inv;
        const float4 v = *reinterpret_cast<const float4*>(p.ws_o + slot * D + d);
        o[0] = fmaf(wgt, v.x, o[0]); o[1] = fmaf(wgt, v.y, o[1]);
        o[2] = fmaf(wgt, v.z, o[2]); o[3] = fmaf(wgt, v.w, o[3]);
      }
    }
    if constexpr (sizeof(T) == 2) {
      const uint32_t lo2 = (uint32_t)f32_to_bf16_bits(o[0]) | ((uint32_t)f32_to_bf16_bits(o[1]) << 16);
      const uint32_t hi2 = (uint32_t)f32_to_bf16_bits(o[2]) | ((uint32_t)f32_to_bf16_bits(o[3]) << 16);
      *reinterpret_cast<uint2*>(orow + d) = make_uint2(lo2, hi2);
    } else {
      *reinterpret_cast<float4*>(orow + d) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
  if (p.lse && threadIdx.x == 0)
    p.lse[(int64_t)qrow * p.H + h] = M == -INFINITY ? -INFINITY : (M + log2f(den)) * kLn2;
}

template <typename T, int D, bool HCA>
static void launch_attn_t(const AttnArgs& a, hipStream_t st) {
  const int nw = (a.H + 15) / 16;
  const dim3 grid((unsigned)((int64_t)a.B * a.Lq * a.nsplit_max));
#define CSA_ATTN_NW(N) hipLaunchKernelGGL((attn_kernel<T, D, N, HCA>), grid, dim3(N * kWave), 0, st, a)
  if (nw == 1) CSA_ATTN_NW(1);
  else if (nw == 2) CSA_ATTN_NW(2);
  else if (nw <= 4) CSA_ATTN_NW(4);
  else CSA_ATTN_NW(8);
#undef CSA_ATTN_NW
  if (a.nsplit_max > 1)
    hipLaunchKernelGGL((attn_combine_kernel<T, D, HCA>), dim3((unsigned)((int64_t)a.B * a.Lq * a.H)),
                       dim3(128), 0, st, a);
}

int launch_attn(const AttnArgs& a, int kv_dtype, bool hca, hipStream_t st) {
  if ((int64_t)a.B * a.Lq == 0) return 0;
#define CSA_ATTN_D(TT, HH) \
  if (a.D == 128) launch_attn_t<TT, 128, HH>(a, st); else launch_attn_t<TT, 512, HH>(a, st)
  if (kv_dtype == 0) {
    if (hca) { CSA_ATTN_D(float, true); } else { CSA_ATTN_D(float, false); }
  } else {
    if (hca) { CSA_ATTN_D(uint16_t, true); } else { CSA_ATTN_D(uint16_t, false); }
  }
#undef CSA_ATTN_D
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
