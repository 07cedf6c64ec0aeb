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
//  * one workgroup per (query, split of its source list), two waves per
//    group of 16 heads: both compute the group's scores, each accumulates the
//    output for one half of D (halving the accumulator registers so that two
//    waves fit per SIMD);
//  * 32 source rows per tile go straight from HBM into LDS (CSA: rows named
//    by idx; HCA: consecutive rows; window: raw rows, then rotated in LDS),
//    double-buffered so the next tile's loads fly while this one is used;
//    V stays row-major and is read with the LDS transpose instruction;
//  * S^T = K Q^T and O^T = V^T P^T on MFMA 16x16 (bf16: 16x16x32; f32:
//    16x16x4), so a lane's accumulators all belong to one head and the online
//    softmax rescale is one multiply per register;
//  * the split count depends only on the query's own source count, never on
//    the batch, so results are batch-invariant and deterministic; a separate
//    combine kernel merges the splits in a fixed order (bf16 inputs keep
//    their split partials in bf16, halving that traffic).
#include "common.hpp"
#include "launch.hpp"
#include "attn_tile.hpp"

namespace csa {

template <typename T, int D>
struct AttnState {
  static constexpr bool BF = sizeof(T) == 2;
  typedef typename std::conditional<BF, bf16x8, float>::type QFrag;
  static constexpr int QN = BF ? D / 32 : D / 4;
  QFrag qf[QN];
  f32x4 acc[D / 32];  // this wave's half of D
  float m_run, l_run;
};

// bf16 tile for the pair of waves that shares a group of 16 heads: each
// wave computes S^T = K Q^T for its own 16 of the tile's 32 rows only, the
// pair swaps its row maxima and then its probabilities (bf16, the precision
// P enters the MFMA with anyway) through LDS, and each wave accumulates
// O^T += V^T P^T over all 32 rows for its half of D. Each wave's l_run sums
// its own rows; the pair adds them once at the end.
template <int D>
__device__ __forceinline__ void compute_tile_bf(AttnState<uint16_t, D>& st, const uint8_t* Ks, const uint8_t* Vs,
                                                const int* kind, float cscale, int dh, float* xm_own,
                                                const float* xm_oth, uint2* xp_own, const uint2* xp_oth) {
  constexpr int ROWB = D * 2;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, l16 = lane % 16;
  const int rt = dh;  // this wave's rows 16dh .. 16dh+15
  f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int QN = D / 32;
  constexpr int KB = QN < 8 ? QN : 8;  // k-steps per batch of fragment reads
#pragma unroll
  for (int s0 = 0; s0 < QN; s0 += KB) {
    uint4 kf[KB];
#pragma unroll
    for (int s = 0; s < KB; ++s)
      kf[s] = *reinterpret_cast<const uint4*>(Ks + lds_pos<ROWB, k_line<uint16_t, D>()>(16 * rt + l16,
                                                                                        (32 * (s0 + s) + 8 * g) * 2));
#pragma unroll
    for (int s = 0; s < KB; ++s)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[s]), st.qf[s0 + s], sacc, 0, 0, 0);
  }
  float x[4];
  float tm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool ok = kind[16 * rt + 4 * g + r] != 0;
    x[r] = ok ? sacc[r] * cscale : -INFINITY;
    tm = fmaxf(tm, x[r]);
  }
  tm = fmaxf(tm, __shfl_xor(tm, 16, kWave));
  tm = fmaxf(tm, __shfl_xor(tm, 32, kWave));
  if (g == 0) xm_own[l16] = tm;
  attn_lds_barrier();
  const float tmax = fmaxf(tm, xm_oth[l16]);
  const float m_new = fmaxf(st.m_run, tmax);
  const bool none = m_new == -INFINITY;
  const float alpha = none ? 1.f : exp2f(st.m_run - m_new);
  float e[4];
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    e[r] = none ? 0.f : exp2f(x[r] - m_new);
    psum += e[r];
  }
  psum += __shfl_xor(psum, 16, kWave);
  psum += __shfl_xor(psum, 32, kWave);
  st.l_run = st.l_run * alpha + psum;
  st.m_run = m_new;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.acc[dt] *= alpha;
  const uint2 mine = make_uint2((uint32_t)f32_to_bf16_bits(e[0]) | ((uint32_t)f32_to_bf16_bits(e[1]) << 16),
                                (uint32_t)f32_to_bf16_bits(e[2]) | ((uint32_t)f32_to_bf16_bits(e[3]) << 16));
  xp_own[lane] = mine;
  attn_lds_barrier();
  const uint2 oth = xp_oth[lane];  // the partner's lane with the same head and row offset
  const uint2 t0 = rt == 0 ? mine : oth, t1 = rt == 0 ? oth : mine;
  const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(t0.x, t0.y, t1.x, t1.y));

  const int dt0 = dh * (D / 32);  // first d-tile of this wave's half
  // transposed LDS reads: lane (l16, g) gets column d of rows 4g..4g+3 and 16+4g..16+4g+3
  const int j4 = l16 / 4, jm = l16 % 4;
  const int off_a = lds_pos<ROWB>(4 * g + j4, jm * 8) + dt0 * 32;
  int off_b = lds_pos<ROWB>(16 + 4 * g + j4, jm * 8) + dt0 * 32;
  // Opaque to the compiler: folded into the first base as one large
  // immediate, some of these reads lose their LDS alias information, and
  // the compiler then waits for every copy in flight (the next tile's
  // prefetch) before them.
  __asm__ volatile("" : "+v"(off_b));
  constexpr int DB = D / 32 < 8 ? D / 32 : 8;  // d-tiles per batch of reads
#pragma unroll
  for (int d0 = 0; d0 < D / 32; d0 += DB) {
    v4i16 lo4[DB], hi4[DB];
#pragma unroll
    for (int q = 0; q < DB; ++q) {
      lo4[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(Vs + off_a + (d0 + q) * 32));
      hi4[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(Vs + off_b + (d0 + q) * 32));
    }
#pragma unroll
    for (int q = 0; q < DB; ++q) {
      const short8_t vv = {lo4[q][0], lo4[q][1], lo4[q][2], lo4[q][3], hi4[q][0], hi4[q][1], hi4[q][2], hi4[q][3]};
      st.acc[d0 + q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf, st.acc[d0 + q], 0, 0, 0);
    }
  }
}

// S^T = K Q^T, online softmax, O^T += V^T P^T for one tile in LDS.
template <typename T, int D>
__device__ __forceinline__ void compute_tile(AttnState<T, D>& st, const uint8_t* Ks, const uint8_t* Vs,
                                             const int* kind, float cscale, int dh) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int ROWB = D * (int)sizeof(T);
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, l16 = lane % 16;
  f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  if constexpr (BF) {
    constexpr int QN = D / 32;
    constexpr int KB = QN < 8 ? QN : 8;  // k-steps per batch of fragment reads
#pragma unroll
    for (int s0 = 0; s0 < QN; s0 += KB) {
      uint4 kf[2][KB];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int s = 0; s < KB; ++s)
          kf[rt][s] = *reinterpret_cast<const uint4*>(Ks + lds_pos<ROWB, k_line<T, D>()>(16 * rt + l16, (32 * (s0 + s) + 8 * g) * 2));
#pragma unroll
      for (int s = 0; s < KB; ++s)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[rt][s]), st.qf[s0 + s],
                                                              sacc[rt], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int u = 0; u < D / 8; ++u)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float2 kk = *reinterpret_cast<const float2*>(Ks + lds_pos<ROWB, k_line<T, D>()>(16 * rt + l16, (8 * u + 2 * g) * 4));
        sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.x, st.qf[2 * u], sacc[rt], 0, 0, 0);
        sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.y, st.qf[2 * u + 1], sacc[rt], 0, 0, 0);
      }
  }
  float x[2][4];
  float tmax = -INFINITY;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = kind[16 * rt + 4 * g + r] != 0;
      x[rt][r] = ok ? sacc[rt][r] * cscale : -INFINITY;
      tmax = fmaxf(tmax, x[rt][r]);
    }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
  const float m_new = fmaxf(st.m_run, tmax);
  const bool none = m_new == -INFINITY;
  const float alpha = none ? 1.f : exp2f(st.m_run - m_new);
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
  st.l_run = st.l_run * alpha + psum;
  st.m_run = m_new;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.acc[dt] *= alpha;

  const int dt0 = dh * (D / 32);  // first d-tile of this wave's half
  if constexpr (BF) {
    const float pv[8] = {x[0][0], x[0][1], x[0][2], x[0][3], x[1][0], x[1][1], x[1][2], x[1][3]};
    const bf16x8 pf = __builtin_bit_cast(bf16x8, Chunk<uint16_t>::pack(pv));
    // transposed LDS reads: lane (l16, g) gets column d of rows 4g..4g+3 and 16+4g..16+4g+3
    const int j4 = l16 / 4, jm = l16 % 4;
    const int off_a = lds_pos<ROWB>(4 * g + j4, jm * 8) + dt0 * 32;
    int off_b = lds_pos<ROWB>(16 + 4 * g + j4, jm * 8) + dt0 * 32;
    // Opaque to the compiler: folded into the first base as one large
    // immediate, some of these reads lose their LDS alias information, and
    // the compiler then waits for every copy in flight (the next tile's
    // prefetch) before them.
    __asm__ volatile("" : "+v"(off_b));
    constexpr int DB = D / 32 < 8 ? D / 32 : 8;  // d-tiles per batch of reads
#pragma unroll
    for (int d0 = 0; d0 < D / 32; d0 += DB) {
      v4i16 lo4[DB], hi4[DB];
#pragma unroll
      for (int q = 0; q < DB; ++q) {
        lo4[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(Vs + off_a + (d0 + q) * 32));
        hi4[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(Vs + off_b + (d0 + q) * 32));
      }
#pragma unroll
      for (int q = 0; q < DB; ++q) {
        const short8_t vv = {lo4[q][0], lo4[q][1], lo4[q][2], lo4[q][3], hi4[q][0], hi4[q][1], hi4[q][2], hi4[q][3]};
        st.acc[d0 + q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf, st.acc[d0 + q], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vr_ = 16 * rt + 4 * g + r;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const float v = *reinterpret_cast<const float*>(Vs + lds_pos<ROWB>(vr_, 4 * (16 * (dt0 + dt) + l16)));
          st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, x[rt][r], st.acc[dt], 0, 0, 0);
        }
      }
  }
}


template <typename T, int D, int NW, bool HCA>
__global__ __launch_bounds__(NW * kWave) void attn_kernel(AttnArgs p) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int NT = NW * kWave;
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int NL = 32 * ROWB / 1024;   // lines per tile
  constexpr bool DBUF = attn_double_buffered<T, D>(NW);
  constexpr int NBUF = DBUF ? 2 : 1;
  constexpr int LOADS = 2 * NL / NW;     // vector-memory ops per wave per tile
  __shared__ __attribute__((aligned(16))) uint8_t Ks0[NL * k_line<T, D>()];
  __shared__ __attribute__((aligned(16))) uint8_t Vs0[NL * kLineB];
  __shared__ __attribute__((aligned(16))) uint8_t Ks1[DBUF ? NL * k_line<T, D>() : 16];
  __shared__ __attribute__((aligned(16))) uint8_t Vs1[DBUF ? NL * kLineB : 16];
  __shared__ int kind[NBUF][32];
  __shared__ int64_t rpos[NBUF][32];
  __shared__ float qcos[kRopePairs], qsin[kRopePairs];
  __shared__ int sidx[HCA ? 1 : kMaxSplitRows];
  // bf16: the wave pairs' exchange of row maxima / final sums and of P
  __shared__ float xch_m[BF ? NW : 1][16];
  __shared__ uint2 xch_p[BF ? NW : 1][kWave];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int g = lane / 16, l16 = lane % 16;
  const int qrow = blockIdx.x / p.nsplit_max;
  const int split = blockIdx.x % p.nsplit_max;
  SplitInfo si;
  si.b = qrow / p.Lq;
  const int i = qrow % p.Lq;
  si.t = seq_pos(p.q_pos, p.q_pos0, si.b) + i;
  si.n_c = HCA ? (int)((si.t + 1) / p.m) : p.topk;
  si.lo = si.t - p.W + 1 > 0 ? si.t - p.W + 1 : 0;
  si.row_lo = attn_raw_row(p, si.lo);
  si.n_w = p.W > 0 ? (int)(si.t - si.lo + 1) : 0;
  const int S = si.n_c + p.W;
  const int CH = attn_split_rows(S);
  const int nsplit = attn_nsplit(S);
  if (split >= nsplit) return;
  si.s0 = split * CH;
  si.s1 = min(S, si.s0 + CH);
  const int ntiles = (si.s1 - si.s0 + 31) / 32;

  // Prologue: the split's idx slots, the query's RoPE table; first tiles' loads.
  if constexpr (!HCA) {
    for (int r = tid; r < si.s1 - si.s0; r += NT) {
      const int sp = si.s0 + r;
      sidx[r] = sp < si.n_c ? p.idx[(int64_t)qrow * p.topk + sp] : -1;
    }
  }
  const double rev = kRopeRev[tid % kRopePairs];
  if (tid < kRopePairs) rope_cos_sin_f(si.t, rev, &qcos[tid], &qsin[tid]);
  __syncthreads();
  // wave = (head group of 16, half of D): both halves compute the same S for
  // their heads; each accumulates O for its own half of D
  const int dh = wave & 1;
  const int h = (wave >> 1) * 16 + l16;
  const bool hok = h < p.H;
  const T* qbase = (const T*)p.q + ((int64_t)qrow * p.H + (hok ? h : 0)) * D;
  AttnState<T, D> st;
  // Q loads first: vmcnt completes in order, so waiting for them later does
  // not wait for the tile loads issued after them.
  constexpr int QL = BF ? D / 32 : D / 8;
  typedef typename std::conditional<BF, uint4, float2>::type QRaw;
  QRaw qraw[QL];
#pragma unroll
  for (int s = 0; s < QL; ++s)
    qraw[s] = *reinterpret_cast<const QRaw*>(qbase + (BF ? 32 * s + 8 * g : 8 * s + 2 * g));
  // Copies are issued for every tile slot of the ring, also past the split's
  // last tile (their rows are masked: row 0, which stays cached), so every
  // path through the loop has the same memory-counter state and the
  // compiler's own wait analysis adds no waits.
  issue_tile<T, D, NW, HCA>(p, si, sidx, si.s0, Ks0, Vs0, kind[0], rpos[0]);
  if (DBUF) issue_tile<T, D, NW, HCA>(p, si, sidx, si.s0 + 32, Ks1, Vs1, kind[NBUF - 1], rpos[NBUF - 1]);
  if constexpr (BF) {
#pragma unroll
    for (int s = 0; s < QL; ++s) {
      const int d0 = 32 * s + 8 * g;
      uint4 raw = hok ? qraw[s] : make_uint4(0, 0, 0, 0);
      if (d0 >= D - kRopeDims) {
        float v[8];
        Chunk<uint16_t>::unpack(raw, v);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int pr = (d0 + e - (D - kRopeDims)) / 2;
          const float c = qcos[pr], sn = qsin[pr], x0 = v[e], x1 = v[e + 1];
          v[e] = x0 * c - x1 * sn;
          v[e + 1] = x0 * sn + x1 * c;
        }
        raw = Chunk<uint16_t>::pack(v);
      }
      st.qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  } else {
#pragma unroll
    for (int u = 0; u < QL; ++u) {
      const int d0 = 8 * u + 2 * g;
      float2 x = hok ? qraw[u] : make_float2(0.f, 0.f);
      if (d0 >= D - kRopeDims) {
        const int pr = (d0 - (D - kRopeDims)) / 2;
        const float c = qcos[pr], sn = qsin[pr], x0 = x.x, x1 = x.y;
        x.x = x0 * c - x1 * sn;
        x.y = x0 * sn + x1 * c;
      }
      st.qf[2 * u] = x.x;
      st.qf[2 * u + 1] = x.y;
    }
  }
  attn_lds_barrier();  // row kinds/positions of the first tiles are visible
  st.m_run = -INFINITY;
  st.l_run = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float cscale = kLog2e / sqrtf((float)D);

  // One tile: wait for its loads, rotate window rows in LDS (cos/sin
  // evaluated in place: no table, so more workgroups fit per CU), compute,
  // then reuse the buffer for the tile two ahead.
  auto step = [&](int tt, uint8_t* Kb, uint8_t* Vb, int bi) {
    const int ts = si.s0 + 32 * tt;
    const bool win = si.n_w > 0 && ts + 32 > si.n_c;
    // kind/rpos of this buffer were written by issue_tile before a barrier.
    // This tile's copies: everything issued after them is the next tile's.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(DBUF ? LOADS : 0));
    attn_lds_barrier();
    if (win) {
      rope_rows_lds_direct<T, D>(Kb, kind[bi], rpos[bi], rev, NT);
      attn_lds_barrier();
    }
    if constexpr (BF)
      compute_tile_bf<D>(st, Kb, Vb, kind[bi], cscale, dh, xch_m[wave], xch_m[wave ^ 1], xch_p[wave],
                         xch_p[wave ^ 1]);
    else
      compute_tile<T, D>(st, Kb, Vb, kind[bi], cscale, dh);
    attn_lds_barrier();
    issue_tile<T, D, NW, HCA>(p, si, sidx, si.s0 + 32 * (tt + NBUF), Kb, Vb, kind[bi], rpos[bi]);
  };
  for (int tt = 0; tt < ntiles; tt += NBUF) {
    step(tt, Ks0, Vs0, 0);
    if (DBUF && tt + 1 < ntiles) step(tt + 1, Ks1, Vs1, NBUF - 1);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS outlives the workgroup
  if constexpr (BF) {  // each wave of a pair summed its own rows: add the partner's
    if (g == 0) xch_m[wave][l16] = st.l_run;
    attn_lds_barrier();
    st.l_run += xch_m[wave ^ 1][l16];
  }

  if (!hok) return;
  if (nsplit == 1) {
    const float z2 = p.sink ? p.sink[h] * kLog2e : -INFINITY;
    const float M = fmaxf(z2, st.m_run);
    float f = 0.f, lse2 = -INFINITY;
    if (M != -INFINITY) {
      const float den = exp2f(z2 - M) + st.l_run * exp2f(st.m_run - M);
      f = exp2f(st.m_run - M) / den;
      lse2 = M + log2f(den);
    }
    T* orow = (T*)p.out + ((int64_t)qrow * p.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int d = 16 * (dh * (D / 32) + dt) + 4 * g;
      if constexpr (BF) {
        const uint32_t lo2 = (uint32_t)f32_to_bf16_bits(st.acc[dt][0] * f) | ((uint32_t)f32_to_bf16_bits(st.acc[dt][1] * f) << 16);
        const uint32_t hi2 = (uint32_t)f32_to_bf16_bits(st.acc[dt][2] * f) | ((uint32_t)f32_to_bf16_bits(st.acc[dt][3] * f) << 16);
        *reinterpret_cast<uint2*>(orow + d) = make_uint2(lo2, hi2);
      } else {
        *reinterpret_cast<float4*>(orow + d) = make_float4(st.acc[dt][0] * f, st.acc[dt][1] * f, st.acc[dt][2] * f, st.acc[dt][3] * f);
      }
    }
    if (p.lse && g == 0 && dh == 0) p.lse[(int64_t)qrow * p.H + h] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  } else {
    const int64_t slot = ((int64_t)qrow * p.nsplit_max + split) * p.H + h;
    T* po = (T*)p.ws_o + slot * D + dh * (D / 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      if constexpr (BF) {
        const uint32_t lo2 = (uint32_t)f32_to_bf16_bits(st.acc[dt][0]) | ((uint32_t)f32_to_bf16_bits(st.acc[dt][1]) << 16);
        const uint32_t hi2 = (uint32_t)f32_to_bf16_bits(st.acc[dt][2]) | ((uint32_t)f32_to_bf16_bits(st.acc[dt][3]) << 16);
        *reinterpret_cast<uint2*>(po + 16 * dt + 4 * g) = make_uint2(lo2, hi2);
      } else {
        *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) = make_float4(st.acc[dt][0], st.acc[dt][1], st.acc[dt][2], st.acc[dt][3]);
      }
    }
    if (g == 0 && dh == 0) *reinterpret_cast<float2*>(p.ws_ml + slot * 2) = make_float2(st.m_run, st.l_run);
  }
}

// Merge the splits of one (query, head) in a fixed split order. A thread
// owns 16 bytes of the output row (8 bf16 or 4 f32 values) and keeps all the
// row's split statistics in registers (at most kMaxSplits: a split holds at
// least S/16 rows), so its loads of the split partials are independent and
// issued together rather than one dependent round trip per split.
constexpr int kMaxSplits = 16;
constexpr int kCombThreads = 64;  // small workgroups: at decode sizes they still cover every CU
template <typename T, int D, bool HCA>
__global__ __launch_bounds__(kCombThreads) void attn_combine_kernel(AttnArgs p) {
  constexpr int VPT = 16 / (int)sizeof(T);  // values per thread
  constexpr int TPH = D / VPT;              // threads per (query, head) row (32 to 128)
  const int64_t gt = (int64_t)blockIdx.x * kCombThreads + threadIdx.x;
  const int64_t row = gt / TPH;
  if (row >= (int64_t)p.B * p.Lq * p.H) return;
  const int64_t qrow = row / p.H;
  const int h = (int)(row % p.H);
  const int i = (int)(qrow % p.Lq);
  const int64_t t = seq_pos(p.q_pos, p.q_pos0, (int)(qrow / p.Lq)) + i;
  const int n_c = HCA ? (int)((t + 1) / p.m) : p.topk;
  const int nsplit = attn_nsplit(n_c + p.W);
  if (nsplit == 1) return;
  const int64_t slot0 = (qrow * p.nsplit_max) * p.H + h;
  const float z2 = p.sink ? p.sink[h] * kLog2e : -INFINITY;
  float2 ml[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    ml[s] = s < nsplit ? *reinterpret_cast<const float2*>(p.ws_ml + (slot0 + (int64_t)s * p.H) * 2)
                       : make_float2(-INFINITY, 0.f);
  const int d = (int)(gt % TPH) * VPT;
  uint4 raw[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    raw[s] = s < nsplit ? *reinterpret_cast<const uint4*>((const T*)p.ws_o + (slot0 + (int64_t)s * p.H) * D + d)
                        : make_uint4(0, 0, 0, 0);
  float M = z2;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) M = fmaxf(M, ml[s].x);
  float den = 0.f;
  float wgt[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) wgt[s] = 0.f;
  if (M != -INFINITY) {
    den = exp2f(z2 - M);
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      wgt[s] = ml[s].x == -INFINITY ? 0.f : exp2f(ml[s].x - M);
      den += ml[s].y * wgt[s];
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float o[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) o[v] = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    float x[VPT];
    Chunk<T>::unpack(raw[s], x);
    const float w = wgt[s] * inv;
#pragma unroll
    for (int v = 0; v < VPT; ++v) o[v] = fmaf(w, x[v], o[v]);
  }
  *reinterpret_cast<uint4*>((T*)p.out + (qrow * p.H + h) * D + d) = Chunk<T>::pack(o);
  if (p.lse && gt % TPH == 0)
    p.lse[qrow * p.H + h] = M == -INFINITY ? -INFINITY : (M + log2f(den)) * kLn2;
}

template <typename T, int D, bool HCA>
static void launch_attn_t(const AttnArgs& a, hipStream_t st) {
  const int hg = (a.H + 15) / 16;  // head groups; two waves (halves of D) per group
  const dim3 grid((unsigned)((int64_t)a.B * a.Lq * a.nsplit_max));
#define CSA_ATTN_NW(N) hipLaunchKernelGGL((attn_kernel<T, D, N, HCA>), grid, dim3(N * kWave), 0, st, a)
  if (hg == 1) CSA_ATTN_NW(2);
  else if (hg == 2) CSA_ATTN_NW(4);
  else if (hg <= 4) CSA_ATTN_NW(8);
  else CSA_ATTN_NW(16);
#undef CSA_ATTN_NW
  if (a.nsplit_max > 1)
    hipLaunchKernelGGL((attn_combine_kernel<T, D, HCA>),
                       dim3((unsigned)(((int64_t)a.B * a.Lq * a.H * D * sizeof(T) / 16 + kCombThreads - 1) /
                                       kCombThreads)),
                       dim3(kCombThreads), 0, st, a);
}

int launch_attn(const AttnArgs& a, int kv_dtype, bool hca, hipStream_t st) {
  if ((int64_t)a.B * a.Lq == 0) return 0;
  if (a.nsplit_max > kMaxSplits) return 1;  // cannot happen: a split holds at least S/16 rows
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
