// Device code of the two-launch CSA attention for many heads (one shared KV
// head of dim 512 in bf16, H a multiple of 16): phase A (logits of all heads
// against a chunk of 64 source rows) and phase B (P V over all rows for one
// 64- or 32-wide slice of D), as work-unit bodies with their LDS in structs (a
// kernel can then overlay them with other work in one LDS buffer).
//
// Source: "DeepSeek V4 重磅開源！…" (InfoQ), section 混合注意力機制 (the
// selected compressed entries plus a sliding window over raw tokens, RoPE on
// the last 64 dims, an attention sink).
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace csa {
namespace dec {

constexpr int kDecD = 512;           // head dim of this path
constexpr int kArows = 64;           // source rows per phase-A chunk
constexpr int kAtiles = kArows / 16;   // 16-row MFMA tiles of a chunk
constexpr int kCtiles = kArows / 32;   // 32-row phase-B tiles of a chunk
constexpr int kAline = 1024 + 16;    // LDS bytes per K row: 260 words, 4 mod 32, so the 16-byte fragment
                                     // reads of 8 consecutive rows hit 8 disjoint groups of 4 banks
constexpr int kBrowsMax = 640;       // V rows staged at once by phase B
constexpr int kBrowsNarrow = 1152;   // ... when its workgroups are few (one per CU)
constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLn2D = 0.6931471805599453f;

// Workgroup barrier for LDS data: waits for this wave's LDS operations only
// (not for its outstanding global loads or global-to-LDS copies, which
// __syncthreads' fence would drain, the counter being in order), then
// s_barrier; the memory clobber keeps the compiler from moving accesses
// across it. Copied rows are waited for explicitly (vmcnt) where needed.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef short v4i16d __attribute__((ext_vector_type(4)));
typedef short short8d __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16d lds_v4i16d;

// Source of slot sp of query row qrow: 0 = masked (reads row 0 of the
// compressed cache, which is finite), 1 = compressed entry, 2 = window row at
// absolute position *pos. *src = element offset of the row.
// The idx slot of a source slot, read unconditionally (clamped into the
// list; a list of length 0 reads the first q element instead and ignores it),
// so the lookup is one load with no branch around it.
__device__ __forceinline__ const int32_t* idx_slot(const AttnArgs& p, int qrow, int sp) {
  return p.topk > 0 ? p.idx + (int64_t)qrow * p.topk + min(sp, p.topk - 1) : (const int32_t*)p.q;
}

// Source of slot sp given its idx value j (idx_slot).
__device__ __forceinline__ int dec_source(const AttnArgs& p, int b, int64_t lo, int64_t row_lo, int n_w, int sp,
                                          int32_t jv, int64_t* src, int64_t* pos) {
  const int64_t j = p.topk > 0 ? (int64_t)jv : -1;
  const int w = sp - p.topk;
  const bool comp = sp < p.topk && j >= 0 && j < p.N_cap;
  const bool win = sp >= p.topk && w < n_w;
  *pos = win ? lo + w : 0;
  *src = comp ? ((int64_t)b * p.N_cap + j) * kDecD
       : win ? ((int64_t)b * p.T_raw + attn_window_row(p, row_lo, w)) * kDecD
             : (int64_t)b * p.N_cap * kDecD;
  return comp ? 1 : win ? 2 : 0;
}

struct DecQuery {
  int b, n_w;
  int64_t t, lo, row_lo;  // row_lo: raw row of window position lo
};

__device__ __forceinline__ DecQuery dec_query(const AttnArgs& p, int qrow) {
  DecQuery d;
  d.b = qrow / p.Lq;
  d.t = seq_pos(p.q_pos, p.q_pos0, d.b) + qrow % p.Lq;
  d.lo = d.t - p.W + 1 > 0 ? d.t - p.W + 1 : 0;
  d.n_w = p.W > 0 ? (int)(d.t - d.lo + 1) : 0;
  d.row_lo = attn_raw_row(p, d.lo);
  return d;
}

// LDS of a phase-A work unit.
struct DecAShared {
  __attribute__((aligned(16))) uint8_t Ks[kArows * kAline];
  int kind[kArows];
  int64_t rpos[kArows];
  const uint8_t* rsrc[kArows];
  float qcos[kRopePairs], qsin[kRopePairs];
};

// Phase A: logits of all heads of query row qrow against its chunk c of 64
// source rows (NW waves of 16 heads; extra waves of the workgroup, if any,
// only join the barriers).
template <int NW>
__device__ __forceinline__ void dec_a_body(DecAShared& L, const AttnArgs& p, const int qrow, const int c,
                                           const int nchunk, const int spad, uint16_t* __restrict__ pp,
                                           float* __restrict__ ml, int64_t* __restrict__ rowsrc) {
  constexpr int QS = kDecD / 32;  // k-steps of 32 dims
  uint8_t* Ks = L.Ks;
  int* kind = L.kind;
  int64_t* rpos = L.rpos;
  const uint8_t** rsrc = L.rsrc;
  float* qcos = L.qcos;
  float* qsin = L.qsin;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int g = lane / 16, l16 = lane % 16;
  const DecQuery dq = dec_query(p, qrow);
  const int r0 = c * kArows;
  const int h = wave * 16 + l16;  // H == 16 * NW

  // The chunk's row sources first (one slot per thread, all lookups in
  // flight together), then this wave's Q fragments: vector-memory operations
  // complete in order, so the barrier below waits for the lookups alone and
  // the Q loads overlap the row copies, which are issued once every source
  // is known.
  // Chunk c holds the sources r * nchunk + c (r < 64), so the window rows
  // (the last sources) spread over all chunks and so does their RoPE work.
  const int su = (tid % kArows) * nchunk + c;
  // Every thread reads one idx slot and the RoPE frequency of pair tid % 32
  // (the only pair it ever rotates), unconditionally, before the Q loads.
  const int32_t jv = *idx_slot(p, qrow, su);
  const double rev = kRopeRev[tid % kRopePairs];
  const uint16_t* qb = (const uint16_t*)p.q + ((int64_t)qrow * p.H + h) * kDecD;
  uint4 qraw[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) qraw[s] = *reinterpret_cast<const uint4*>(qb + 32 * s + 8 * g);
  int64_t src, pos;
  const int kd = dec_source(p, dq.b, dq.lo, dq.row_lo, dq.n_w, su, jv, &src, &pos);
  if (tid < kRopePairs) rope_cos_sin_f(dq.t, rev, &qcos[tid], &qsin[tid]);
  if (tid < kArows) {
    kind[tid] = kd;
    rpos[tid] = pos;
    rsrc[tid] = (const uint8_t*)(kd == 2 ? p.k_raw : p.k_c) + src * 2;
  }
  lds_barrier();
  // K rows of the chunk straight into LDS: wave w copies rows w, w + NW, ...
  for (int r = wave; r < kArows; r += NW)
    __builtin_amdgcn_global_load_lds((const void*)(rsrc[r] + lane * 16),
                                     (__attribute__((address_space(3))) void*)(Ks + r * kAline), 16, 0, 0);
  bf16x8 qf[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    const int d0 = 32 * s + 8 * g;
    uint4 raw = qraw[s];
    if (d0 >= kDecD - kRopeDims) {
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pr = (d0 + 2 * e - (kDecD - kRopeDims)) / 2;
        const float x0 = bf16_bits_to_f32((uint16_t)(w[e] & 0xFFFF)), x1 = bf16_bits_to_f32((uint16_t)(w[e] >> 16));
        const float cs = qcos[pr], sn = qsin[pr];
        o[e] = (uint32_t)f32_to_bf16_bits(x0 * cs - x1 * sn) | ((uint32_t)f32_to_bf16_bits(x0 * sn + x1 * cs) << 16);
      }
      raw = make_uint4(o[0], o[1], o[2], o[3]);
    }
    qf[s] = __builtin_bit_cast(bf16x8, raw);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's K row copies have landed
  lds_barrier();
  // RoPE of the window rows, in LDS (pairs of the last 64 dims). Thread tid
  // rotates pair tid % 32 of rows r0' = tid / 32, r0' + R, r0' + 2R, ...
  // (R = threads / 32); those rows hold sources R * nchunk apart, which in
  // the window are positions R * nchunk apart, so their angles are stepped
  // by one complex multiply each from two evaluations.
  {
    constexpr int R = NW * kWave / kRopePairs;
    const int pr = tid % kRopePairs;
    const int64_t step = (int64_t)R * nchunk;  // position step between rows r and r + R
    float cs = 1.f, sn = 0.f, cd = 1.f, sd = 0.f;
    bool have = false, have_d = false;
    for (int r = tid / kRopePairs; r < kArows; r += R) {
      if (kind[r] != 2) { have = false; continue; }
      if (!have) {  // first window row of this thread (or after a gap): evaluate
        rope_cos_sin_f(rpos[r], rev, &cs, &sn);
        if (!have_d) { rope_cos_sin_f(step, rev, &cd, &sd); have_d = true; }
      } else {
        const float c2 = cs * cd - sn * sd, s2 = sn * cd + cs * sd;
        cs = c2;
        sn = s2;
      }
      have = r + R < kArows && kind[r + R] == 2 && rpos[r + R] == rpos[r] + step;
      uint32_t* wp = reinterpret_cast<uint32_t*>(Ks + r * kAline + (kDecD - kRopeDims + 2 * pr) * 2);
      const uint32_t v = *wp;
      const float x0 = bf16_bits_to_f32((uint16_t)(v & 0xFFFF)), x1 = bf16_bits_to_f32((uint16_t)(v >> 16));
      *wp = (uint32_t)f32_to_bf16_bits(x0 * cs - x1 * sn) | ((uint32_t)f32_to_bf16_bits(x0 * sn + x1 * cs) << 16);
    }
  }
  lds_barrier();

  // S^T = K Q^T: kAtiles 16-row tiles; lane (head l16, g) gets rows 4g..4g+3.
  f32x4 sacc[kAtiles];
#pragma unroll
  for (int rt = 0; rt < kAtiles; ++rt) sacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s0 = 0; s0 < QS; s0 += 4) {
    uint4 kf[kAtiles][4];
#pragma unroll
    for (int rt = 0; rt < kAtiles; ++rt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[rt][s] = *reinterpret_cast<const uint4*>(Ks + (16 * rt + l16) * kAline + (32 * (s0 + s) + 8 * g) * 2);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int rt = 0; rt < kAtiles; ++rt)
        sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[rt][s]), qf[s0 + s],
                                                            sacc[rt], 0, 0, 0);
  }
  const float cscale = kLog2eD / sqrtf((float)kDecD);
  float x[kAtiles][4];
  float mx = -INFINITY;
#pragma unroll
  for (int rt = 0; rt < kAtiles; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[rt][r] = kind[16 * rt + 4 * g + r] ? sacc[rt][r] * cscale : -INFINITY;
      mx = fmaxf(mx, x[rt][r]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
  float sum = 0.f;
  uint16_t* prow = pp + ((int64_t)qrow * p.H + h) * spad + r0;
#pragma unroll
  for (int rt = 0; rt < kAtiles; ++rt) {
    float e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      e[r] = mx == -INFINITY ? 0.f : exp2f(x[rt][r] - mx);
      sum += e[r];
    }
    const uint32_t lo2 = (uint32_t)f32_to_bf16_bits(e[0]) | ((uint32_t)f32_to_bf16_bits(e[1]) << 16);
    const uint32_t hi2 = (uint32_t)f32_to_bf16_bits(e[2]) | ((uint32_t)f32_to_bf16_bits(e[3]) << 16);
    *reinterpret_cast<uint2*>(prow + 16 * rt + 4 * g) = make_uint2(lo2, hi2);
  }
  sum += __shfl_xor(sum, 16, kWave);
  sum += __shfl_xor(sum, 32, kWave);
  if (g == 0) *reinterpret_cast<float2*>(ml + (((int64_t)qrow * nchunk + c) * p.H + h) * 2) = make_float2(mx, sum);
  // for phase B: each slot's row in elements, of the compressed cache (>= 0)
  // or of the raw rows (one's complement)
  if (tid < kArows) rowsrc[(int64_t)qrow * spad + r0 + tid] = kd == 2 ? ~src : src;
}

// Phase B: O[:, slice] = sum over all rows of P_r V_r[slice], with
// P_r = P'_r * 2^(m_c - M) / den for the chunk c holding row r. Every
// dependent lookup (chunk statistics, row sources) is made by all threads at
// once into LDS before the copies that need them are issued.
constexpr int kMaxChunks = (2048 + 256 + kArows - 1) / kArows;  // k <= 2048, W <= 256

// LDS of a phase-B work unit staging BR rows at once.
// Phase B's D slice: 64 dims (128 bytes of a row) when a call has enough
// query rows to fill the chip with 8 slices each, else 32 (16 slices, twice
// the workgroups). Each output element is the same MFMA sum either way (an
// MFMA's sum for one element does not depend on the other elements of its
// block), so the choice never changes a bit of the result.
template <int NW, int BR, int DSL> struct DecBShared {
  static constexpr int H = 16 * NW;
  __attribute__((aligned(16))) uint8_t Vs[BR * DSL * 2];
  float2 mls[kMaxChunks * H];
  const uint8_t* vsrc[BR];
  float fsc[BR / kArows][H];
  float Mh[H], denh[H];
};

// Phase B of query row qrow, D slice sl, staging BR source rows at a time.
template <int NW, int BR, int DSL>
__device__ __forceinline__ void dec_b_body(DecBShared<NW, BR, DSL>& L, const AttnArgs& p, const int qrow, const int sl,
                                           const int nchunk, const int spad, const uint16_t* __restrict__ pp,
                                           const float* __restrict__ ml, const int64_t* __restrict__ rowsrc) {
  constexpr int H = 16 * NW;
  constexpr int NT = NW * kWave;
  constexpr int kBrows = BR;
  constexpr int kBtiles = kBrows / 32;
  constexpr int kFc = kBrows / kArows;  // chunks per staged block
  constexpr int kStatIt = (kMaxChunks * H + NT - 1) / NT;
  constexpr int kSrcIt = (kBrows + NT - 1) / NT;
  uint8_t* Vs = L.Vs;
  float2* mls = L.mls;
  const uint8_t** vsrc = L.vsrc;
  auto& fsc = L.fsc;
  float* Mh = L.Mh;
  float* denh = L.denh;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int g = lane / 16, l16 = lane % 16;
  const int h = wave * 16 + l16;
  const uint16_t* prow = pp + ((int64_t)qrow * H + h) * spad;

  // Row sources of the first block (written by phase A), the chunk
  // statistics of the query (nchunk x H pairs) and this thread's sink logit
  // (H = NT / 4 heads, one per thread): unconditional loads, all in flight
  // together, each consumed at once into LDS so none is deferred to a later
  // use.
  const int64_t* rs = rowsrc + (int64_t)qrow * spad;
  constexpr int kDsl = DSL;
  constexpr int RPC = 1024 / (kDsl * 2);  // rows per wave copy (16-byte lanes)
  constexpr int CPR = kDsl * 2 / 16;      // 16-byte chunks per row slice
  const uint8_t* vbase = (const uint8_t*)p.v_c + sl * kDsl * 2;
  const uint8_t* rbase = (const uint8_t*)p.v_raw + sl * kDsl * 2;
  auto put_sources = [&](int rb, int nrows) {
    int64_t e[kSrcIt];
#pragma unroll
    for (int it = 0; it < kSrcIt; ++it) e[it] = rs[rb + min(tid + it * NT, nrows - 1)];
#pragma unroll
    for (int it = 0; it < kSrcIt; ++it)
      if (tid + it * NT < nrows) vsrc[tid + it * NT] = e[it] >= 0 ? vbase + e[it] * 2 : rbase + (~e[it]) * 2;
  };
  // V slices of a block into LDS: each wave copy moves RPC rows of 2*DSL
  // bytes, stored XOR-swizzled so that the transposed reads below are
  // conflict-free: 128-byte rows (one row spans every bank) take chunk
  // position = chunk ^ 2 (r % 4); 64-byte rows (four rows share the banks,
  // and a half-wave's reads would put rows r and r + 8 on the same banks)
  // take chunk ^ 2 ((r / 8) % 2), which sends r + 8 to the other half.
  // Lane l of the copy, which lands at chunk position l % CPR of row
  // L*RPC + l/CPR, fetches the global chunk that belongs there.
  // A fixed trip count (rows past nrows re-copy the last row into slots
  // that are never read): a loop with a data-dependent count would make the
  // compiler drain every load in flight (the P' fragments) before it.
  auto copy_block = [&](int nrows) {
#pragma unroll
    for (int u = 0; u < (kBrows / RPC + NW - 1) / NW; ++u) {
      const int L_ = wave + NW * u;
      if ((kBrows / RPC) % NW != 0 && L_ >= kBrows / RPC) break;  // wave-uniform
      const int r = L_ * RPC + lane / CPR;
      const int swz = DSL == 64 ? 2 * (r % 4) : 2 * ((r / 8) % 2);
      __builtin_amdgcn_global_load_lds((const void*)(vsrc[min(r, nrows - 1)] + (((lane % CPR) ^ swz) * 16)),
                                       (__attribute__((address_space(3))) void*)(Vs + L_ * 1024), 16, 0, 0);
    }
  };
  // This lane's P' fragments of the first block (rows 32t + 8g .. +7 of head
  // h, the MFMA's B operand as they are): independent of everything else, so
  // issued first and in flight with the lookups and the copies.
  uint4 pf[kBtiles];
  auto load_pf = [&](int rb, int nrows) {
#pragma unroll
    for (int t = 0; t < kBtiles; ++t)
      pf[t] = *reinterpret_cast<const uint4*>(prow + rb + min(32 * t, nrows - 32) + 8 * g);
  };
  load_pf(0, min(kBrows, spad));
  const float2* mlq = reinterpret_cast<const float2*>(ml) + (int64_t)qrow * nchunk * H;
  float2 mv[kStatIt];
#pragma unroll
  for (int it = 0; it < kStatIt; ++it) mv[it] = mlq[min(tid + it * NT, nchunk * H - 1)];
  const float zraw = *(p.sink ? p.sink + tid % H : (const float*)p.q);
  put_sources(0, min(kBrows, spad));
#pragma unroll
  for (int it = 0; it < kStatIt; ++it)
    if (tid + it * NT < nchunk * H) mls[tid + it * NT] = mv[it];
  const float z2 = p.sink ? zraw * kLog2eD : -INFINITY;

  f32x4 acc[kDsl / 16];
#pragma unroll
  for (int dt = 0; dt < kDsl / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int rb = 0; rb < spad; rb += kBrows) {
    const int nrows = min(kBrows, spad - rb);  // a multiple of 64
    if (rb > 0) {
      lds_barrier();  // every wave is done with the previous block's Vs, vsrc and fsc
      put_sources(rb, nrows);
    }
    lds_barrier();  // vsrc (and, first block, mls)
    copy_block(nrows);
    if (rb == 0) {
      // Per head (one per thread): M = max(sink, chunk maxima), den = sink
      // term + rescaled chunk sums; LDS only, while the copies fly.
      if (tid < H) {
        float M = z2;
        for (int c = 0; c < nchunk; ++c) M = fmaxf(M, mls[c * H + tid].x);
        float den = 0.f;
        if (M != -INFINITY) {
          den = exp2f(z2 - M);
          for (int c = 0; c < nchunk; ++c) {
            const float2 v = mls[c * H + tid];
            if (v.x != -INFINITY) den += v.y * exp2f(v.x - M);
          }
        }
        Mh[tid] = M;
        denh[tid] = den;
      }
      lds_barrier();  // Mh, denh
    }
    // Per (chunk of the block, head): the factor 2^(m_c - M) / den.
    for (int e = tid; e < kFc * H; e += NT) {
      const int c = e / H, hh = e % H;
      const int cg = rb / kArows + c;
      float f = 0.f;
      if (cg < nchunk) {
        const float m = mls[cg * H + hh].x;
        if (m != -INFINITY && denh[hh] > 0.f) f = exp2f(m - Mh[hh]) / denh[hh];
      }
      fsc[c][hh] = f;
    }
    if (rb > 0) load_pf(rb, nrows);
    // Pin the fragments here: loads from read-only memory may otherwise be
    // sunk to their uses inside the loop below, one round trip per chunk.
#pragma unroll
    for (int t = 0; t < kBtiles; ++t) __asm__ volatile("" : "+v"(pf[t].x), "+v"(pf[t].y), "+v"(pf[t].z), "+v"(pf[t].w));
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();  // Vs, fsc
    // Each chunk (two 32-row tiles) accumulates sum_r P'_r V_r on MFMA; its
    // factor then scales that partial once per lane (a lane's accumulators all
    // belong to head h).
#pragma unroll
    for (int c = 0; c < kFc; ++c) {
      // a uniform guard, not a break: the loop then unrolls fully and pf stays
      // in registers (indexed by constants)
      if (kArows * c >= nrows) continue;
      f32x4 part[kDsl / 16];
#pragma unroll
      for (int tt = 0; tt < kCtiles; ++tt) {
        const int t = kCtiles * c + tt;
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pf[t]);
        // V^T fragments by transposed LDS reads: lane (d = l16, g) gets rows
        // 8g..8g+7 of column 16*dt + l16. Lane j of a 16-lane group reads 8
        // bytes at row ra = 32t + 8g + j/4 (+4), columns 16 dt + 4 (j%4) ..+3:
        // chunk 2 dt + (j%4)/2 of the row, swizzled as stored (ra % 4 = j/4;
        // (ra / 8) % 2 = g % 2, also for ra + 4).
        const int ra = 32 * t + 8 * g + l16 / 4;
        const int sw = DSL == 64 ? 2 * (l16 / 4) : 2 * (g % 2);
#pragma unroll
        for (int dt = 0; dt < kDsl / 16; ++dt) {
          const int off = (((2 * dt + (l16 % 4) / 2) ^ sw) * 16) + (l16 % 2) * 8;
          const v4i16d lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16d*)(Vs + ra * kDsl * 2 + off));
          const v4i16d hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16d*)(Vs + (ra + 4) * kDsl * 2 + off));
          const short8d vv = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          part[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pb,
                                                              tt ? part[dt] : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }
      }
      const float f = fsc[c][h];
#pragma unroll
      for (int dt = 0; dt < kDsl / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[dt][r] = fmaf(part[dt][r], f, acc[dt][r]);
    }
  }

  // (lse is stored last: a store before a barrier would make the barrier wait
  // for every outstanding copy, the counter being in order)
  if (sl == 0 && p.lse && tid < H)
    p.lse[(int64_t)qrow * H + tid] = Mh[tid] == -INFINITY ? -INFINITY : (Mh[tid] + log2f(denh[tid])) * kLn2D;
  uint16_t* orow = (uint16_t*)p.out + ((int64_t)qrow * H + h) * kDecD + sl * kDsl;
#pragma unroll
  for (int dt = 0; dt < kDsl / 16; ++dt) {
    const uint32_t lo2 = (uint32_t)f32_to_bf16_bits(acc[dt][0]) | ((uint32_t)f32_to_bf16_bits(acc[dt][1]) << 16);
    const uint32_t hi2 = (uint32_t)f32_to_bf16_bits(acc[dt][2]) | ((uint32_t)f32_to_bf16_bits(acc[dt][3]) << 16);
    *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = make_uint2(lo2, hi2);
  }
}

}  // namespace dec
}  // namespace csa
