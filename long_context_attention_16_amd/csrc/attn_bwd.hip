// Backward pass of the CSA / HCA attention (gradients for q, the compressed
// keys and values, the raw window keys and values, and the sinks).
//
// Source: "DeepSeek V4 重磅開源！…" (InfoQ), section 確定性內核: training needs
// a deterministic attention backward (the pages drop split-KV and keep a
// fixed accumulation order) and batch-invariant outputs. Formula (the
// gradient of the forward of attn.hip, which is one softmax over the
// selected compressed rows, the window rows and the sink):
//   P_hr = exp(l_hr - lse_h), l_hr = <RoPE(q_h, t), k_r> / sqrt(D);
//   dP_hr = <dO_h, v_r>, Dl_h = <dO_h, o_h>, dS_hr = P_hr (dP_hr - Dl_h);
//   dq_h = RoPE^T(sum_r dS_hr k_r, t) / sqrt(D);
//   dk_r = sum_h dS_hr RoPE(q_h, t) / sqrt(D)  (window rows: RoPE^T at s);
//   dv_r = sum_h P_hr dO_h;  dz_h = -exp(z_h - lse_h) Dl_h.
//
// Design, in three parts.
//  * Query pass: bf16 with D = 128 on MFMA, workgroup = (query row, group
//    of 16 heads), two waves; the query's source rows stream HBM -> LDS in
//    double-buffered tiles of 32 (the forward's tiles); S^T = K Q^T and
//    dP^T = V dO^T for its 16 rows of each tile per wave, P = exp(l - lse)
//    and dS, the pair swaps dS (bf16) through LDS and each wave adds
//    dq^T += K^T dS^T for its half of D (K read with the LDS transpose).
//    Other shapes: workgroup = (query row, group of 4 heads), tiles of 8 rows
//    in LDS as f32, dot products on the vector units. Either writes, for
//    every (query, source slot, head), P and dS / sqrt(D), and the rotated
//    q, for the second part.
//  * Inverse index (CSA): the (query, slot) pairs that select each
//    compressed entry, grouped by entry (counts, a scan, a fill). HCA entries
//    and window rows need none: the queries that use them form a range.
//  * Key/value pass, workgroup = one compressed entry or one raw row: it
//    walks the row's pairs and sums dk = sum dS RoPE(q) / sqrt(D) and
//    dv = sum P dO over them in float32 in a fixed order (query order;
//    a CSA entry's list, filled in no particular order, is sorted in LDS
//    first), or, for lists too long for LDS, in 64-bit fixed point (units of
//    2^-32, exact and order-free). Deterministic with no atomics on the
//    gradients. Window rows are rotated back.
// The sinks' per-query parts are summed in query order.
#include "common.hpp"
#include "launch.hpp"
#include "attn_tile.hpp"

namespace csa {

namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdHeads = 4;   // heads per query-pass workgroup
constexpr int kBwdRows = 8;    // source rows per tile
constexpr int kKvThreads = 256;
constexpr int kKvWaves = kKvThreads / kWave;
constexpr int kScanBlock = 4096;  // counts per scan block (256 threads x 16)
constexpr float kFixScale = 4294967296.f;  // 2^32: fixed-point unit 2^-32

// Workspace pieces (attn_bwd_ws_bytes), each 256-byte aligned.
struct BwdWs {
  float2* pds;        // [rows][S][H]: (P, dS / sqrt(D)) of each (query, source slot, head)
  void* qr;           // [rows][H][D] RoPE(q, t) in the KV dtype
  float* dsink_part;  // [rows][H]
  int* cnt;           // [E = B * N_cap]: selections of each compressed entry
  int* rank;          // [rows * topk]: each pair's rank among its entry's pairs (the counting atomic's value)
  int* off;           // [E] exclusive offsets within the entry's scan block
  int* bsum;          // [ceil(E / kScanBlock)] block totals, then their exclusive offsets
  int* list;          // [rows * topk] flat pair index qrow * topk + slot, grouped by entry
};

struct AttnBwdArgs {
  AttnArgs a;
  int* cnt;  // CSA: selections of each compressed entry, counted by head group 0 (else nullptr)
  int* rank;  // CSA: each counted pair's rank within its entry
  int S;  // source slots per query row (pds stride): topk + W (CSA), n(t_last) + W (HCA)
  const void* dout;
  float* dq;
  BwdWs w;
};

struct BwdKvArgs {
  AttnArgs a;
  int S;
  int listed;  // CSA with at least one pair: the inverse index is built
  int64_t wr0;  // raw rows [wr0, wr0 + nwr) of each sequence are in some query's window
  int nwr;
  const void* dout;
  BwdWs w;
  float *dk_c, *dv_c, *dk_raw, *dv_raw;
};

__device__ __forceinline__ long long to_fix(float x) {
  x = fminf(fmaxf(x, -1073741824.f), 1073741824.f);  // |x| <= 2^30: no overflow of the 64-bit units
  return __float2ll_rn(x * kFixScale);
}

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) {
  return Elem<T>::load(p + i);
}

// N consecutive elements of T at p (N * sizeof(T) bytes, aligned to that size
// up to 16) as floats.
template <typename T, int N>
__device__ __forceinline__ void ld_vec(const T* p, float* o) {
  if constexpr (sizeof(T) == 2) {
    static_assert(N % 2 == 0, "bf16 pairs");
    uint32_t w[N / 2];
    if constexpr (N == 2) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
#pragma unroll
      for (int i = 0; i < N / 8; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(p + 8 * i);
        w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
      }
    }
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    if constexpr (N == 2) {
      const float2 v = *reinterpret_cast<const float2*>(p);
      o[0] = v.x; o[1] = v.y;
    } else {
#pragma unroll
      for (int i = 0; i < N / 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(p + 4 * i);
        o[4 * i] = v.x; o[4 * i + 1] = v.y; o[4 * i + 2] = v.z; o[4 * i + 3] = v.w;
      }
    }
  }
}

// Source row sp of query row qrow: kind 0 masked, 1 compressed entry j, 2
// window row at absolute position *pos; *row = the row's index in k_c / v_c
// (kind 1: b * N_cap + j) or k_raw / v_raw (kind 2: b * T_raw + s - raw_pos0).
template <bool HCA>
__device__ __forceinline__ int bwd_source(const AttnArgs& p, int b, int64_t qrow, int n_c, int64_t lo, int n_w, int sp,
                                          int64_t* row, int64_t* pos) {
  *row = 0;
  *pos = 0;
  if (sp < n_c) {
    const int64_t j = HCA ? sp : (int64_t)p.idx[qrow * p.topk + sp];
    if (j < 0 || j >= p.N_cap) return 0;
    *row = (int64_t)b * p.N_cap + j;
    return 1;
  }
  const int w = sp - n_c;
  if (w >= n_w) return 0;
  *pos = lo + w;
  *row = (int64_t)b * p.T_raw + (lo + w - p.raw_pos0);
  return 2;
}

// Query pass: dq, the rotated q, (P, dS / sqrt(D)) of every source slot and
// the query's sink parts.
template <typename T, int D, bool HCA>
__global__ __launch_bounds__(kBwdThreads) void attn_bwd_q_kernel(AttnBwdArgs g) {
  const AttnArgs& p = g.a;
  constexpr int NT = kBwdThreads, HG = kBwdHeads, R = kBwdRows;
  constexpr int EPT = HG * D / NT;  // (head, d) elements of a thread: e = tid + NT * k
  static_assert(EPT >= 1 && HG * D % NT == 0, "whole elements per thread");
  __shared__ float s_q[HG][D], s_do[HG][D];
  __shared__ float s_k[R][D], s_v[R][D];
  __shared__ float s_l[HG][R], s_dp[HG][R], s_ds[HG][R];
  __shared__ float s_lse[HG], s_dl[HG];
  __shared__ int s_kind[R];
  __shared__ int64_t s_row[R], s_pos[R];

  const int tid = threadIdx.x;
  const int ngroups = (p.H + HG - 1) / HG;
  const int64_t qrow = blockIdx.x / ngroups;
  const int h0 = (int)(blockIdx.x % ngroups) * HG;
  const int b = (int)(qrow / p.Lq);
  const int64_t t = p.q_pos0 + qrow % p.Lq;
  const int n_c = HCA ? (int)((t + 1) / p.m) : p.topk;
  const int64_t lo = t - p.W + 1 > 0 ? t - p.W + 1 : 0;
  const int n_w = p.W > 0 ? (int)(t - lo + 1) : 0;
  const int S = n_c + p.W;
  const float rs = 1.f / sqrtf((float)D);
  if (!HCA && g.cnt && h0 == 0)
    for (int r = tid; r < n_c; r += NT) {
      const int32_t j = p.idx[qrow * p.topk + r];
      if (j >= 0 && j < p.N_cap) g.rank[qrow * p.topk + r] = atomicAdd(g.cnt + (int64_t)b * p.N_cap + j, 1);
    }

  // q (rotated at t), dO, and Dl_h = <dO_h, o_h> for the group's heads
  const T* qb = (const T*)p.q + (qrow * p.H) * D;
  const T* ob = (const T*)p.out + (qrow * p.H) * D;
  const T* db = (const T*)g.dout + (qrow * p.H) * D;
  for (int e = tid; e < HG * D; e += NT) {
    const int hh = e / D, d = e % D, h = h0 + hh;
    const bool hok = h < p.H;
    s_q[hh][d] = hok ? ld(qb, (int64_t)h * D + d) : 0.f;
    s_do[hh][d] = hok ? ld(db, (int64_t)h * D + d) : 0.f;
  }
  if (tid < HG) s_lse[tid] = h0 + tid < p.H ? p.lse[qrow * p.H + h0 + tid] : 0.f;
  __syncthreads();
  for (int e = tid; e < HG * kRopePairs; e += NT) {
    const int hh = e / kRopePairs, pr = e % kRopePairs, d = D - kRopeDims + 2 * pr;
    float c, sn;
    rope_cos_sin(t, pr, &c, &sn);
    const float x0 = s_q[hh][d], x1 = s_q[hh][d + 1];
    s_q[hh][d] = x0 * c - x1 * sn;
    s_q[hh][d + 1] = x0 * sn + x1 * c;
  }
  // Dl: thread group of NT / HG threads per head, strided over d, then a reduction
  {
    constexpr int TPH = NT / HG;
    const int hh = tid / TPH, part = tid % TPH, h = h0 + hh;
    float acc = 0.f;
    if (h < p.H)
      for (int d = part; d < D; d += TPH) acc = fmaf(s_do[hh][d], ld(ob, (int64_t)h * D + d), acc);
#pragma unroll
    for (int o = TPH / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, kWave);
    if (part == 0) s_dl[hh] = acc;
  }
  __syncthreads();
  // the rotated q for the key/value pass
  T* qrb = (T*)g.w.qr + (qrow * p.H) * D;
  for (int e = tid; e < HG * D; e += NT) {
    const int hh = e / D, d = e % D, h = h0 + hh;
    if (h < p.H) Elem<T>::store(qrb + (int64_t)h * D + d, s_q[hh][d]);
  }

  float dq[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) dq[k] = 0.f;

  float2* pdq = g.w.pds + qrow * (int64_t)g.S * p.H;
  for (int r0 = 0; r0 < S; r0 += R) {
    // The tile's rows: sources (the previous tile's last readers of s_kind
    // and s_row passed the barrier before its dq update, which reads only
    // s_ds and s_k), then K (window rows rotated at their position) and V.
    if (tid < R) {
      int64_t row = 0, pos = 0;  // slots past the list: masked, row 0
      s_kind[tid] = r0 + tid < S ? bwd_source<HCA>(p, b, qrow, n_c, lo, n_w, r0 + tid, &row, &pos) : 0;
      s_row[tid] = row;
      s_pos[tid] = pos;
    }
    __syncthreads();
    for (int e = tid; e < R * D; e += NT) {
      const int r = e / D, d = e % D, kd = s_kind[r];
      const T* kp = (const T*)(kd == 2 ? p.k_raw : p.k_c);
      const T* vp = (const T*)(kd == 2 ? p.v_raw : p.v_c);
      s_k[r][d] = kd ? ld(kp, s_row[r] * D + d) : 0.f;
      s_v[r][d] = kd ? ld(vp, s_row[r] * D + d) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < R * kRopePairs; e += NT) {
      const int r = e / kRopePairs, pr = e % kRopePairs, d = D - kRopeDims + 2 * pr;
      if (s_kind[r] != 2) continue;
      float c, sn;
      rope_cos_sin(s_pos[r], pr, &c, &sn);
      const float x0 = s_k[r][d], x1 = s_k[r][d + 1];
      s_k[r][d] = x0 * c - x1 * sn;
      s_k[r][d + 1] = x0 * sn + x1 * c;
    }
    __syncthreads();
    // logits (dot < HG*R) and dP (the rest): 4 threads per dot product
    for (int dot = tid / 4; dot < 2 * HG * R; dot += NT / 4) {
      const int part = tid % 4;
      const int hh = (dot % (HG * R)) / R, r = dot % R;
      const bool is_l = dot < HG * R;
      float acc = 0.f;
      for (int d = part; d < D; d += 4)
        acc = fmaf(is_l ? s_q[hh][d] : s_do[hh][d], is_l ? s_k[r][d] : s_v[r][d], acc);
      acc += __shfl_xor(acc, 1, kWave);
      acc += __shfl_xor(acc, 2, kWave);
      if (part == 0) {
        if (is_l) s_l[hh][r] = acc * rs;
        else s_dp[hh][r] = acc;
      }
    }
    __syncthreads();
    if (tid < HG * R) {
      const int hh = tid / R, r = tid % R;
      const bool ok = s_kind[r] != 0 && h0 + hh < p.H;
      const float pv = ok ? __expf(s_l[hh][r] - s_lse[hh]) : 0.f;
      const float ds = ok ? pv * (s_dp[hh][r] - s_dl[hh]) : 0.f;
      s_ds[hh][r] = ds;
      if (r0 + r < S && h0 + hh < p.H) pdq[(int64_t)(r0 + r) * p.H + h0 + hh] = make_float2(pv, ds * rs);
    }
    __syncthreads();
    // dq += dS k (unscaled; 1/sqrt(D) at the end)
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = tid + NT * k, hh = e / D, d = e % D;
#pragma unroll
      for (int r = 0; r < R; ++r) dq[k] = fmaf(s_ds[hh][r], s_k[r][d], dq[k]);
    }
  }
  __syncthreads();  // every thread is done with s_q's last reader above (none) and s_k

  // dq: back to the unrotated frame (pairs in LDS), scaled by 1/sqrt(D)
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + NT * k;
    s_q[e / D][e % D] = dq[k] * rs;
  }
  __syncthreads();
  for (int e = tid; e < HG * kRopePairs; e += NT) {
    const int hh = e / kRopePairs, pr = e % kRopePairs, d = D - kRopeDims + 2 * pr;
    float c, sn;
    rope_cos_sin(t, pr, &c, &sn);
    const float x0 = s_q[hh][d], x1 = s_q[hh][d + 1];
    s_q[hh][d] = x0 * c + x1 * sn;
    s_q[hh][d + 1] = -x0 * sn + x1 * c;
  }
  __syncthreads();
  for (int e = tid; e < HG * D; e += NT) {
    const int hh = e / D, d = e % D, h = h0 + hh;
    if (h < p.H) g.dq[(qrow * p.H + h) * D + d] = s_q[hh][d];
  }
  if (tid < HG && h0 + tid < p.H) {
    const int h = h0 + tid;
    g.w.dsink_part[qrow * p.H + h] = p.sink ? -__expf(p.sink[h] - s_lse[tid]) * s_dl[tid] : 0.f;
  }
}

// Query pass on MFMA (bf16, D = 128): see the header comment. Wave w of the
// pair computes S and dP for rows 16w..16w+15 of each 32-row tile (lane
// (g, l16): head l16, rows 4g..4g+3 of those), and accumulates dq for dims
// w*D/2 .. w*D/2 + D/2 - 1 over all 32 rows.
template <int D, bool HCA, int CAP>
__global__ __launch_bounds__(2 * kWave) void attn_bwd_q_mfma_kernel(AttnBwdArgs g) {
  using T = uint16_t;
  const AttnArgs& p = g.a;
  constexpr int NW = 2, NT = NW * kWave;
  constexpr int ROWB = D * 2;
  constexpr int NL = 32 * ROWB / 1024;  // LDS lines per tile
  constexpr int LOADS = 2 * NL / NW;    // copies per wave per tile
  constexpr int QN = D / 32;            // k-steps of 32 dims
  // CAP: idx slots staged (topk <= CAP). LDS stays under 40 KB at CAP 1024,
  // four workgroups per CU.
  static_assert(D == 128, "double-buffered tiles of 32 rows of 256 bytes");
  __shared__ __attribute__((aligned(16))) uint8_t Ks0[NL * k_line<T, D>()];
  __shared__ __attribute__((aligned(16))) uint8_t Vs0[NL * kLineB];
  __shared__ __attribute__((aligned(16))) uint8_t Ks1[NL * k_line<T, D>()];
  __shared__ __attribute__((aligned(16))) uint8_t Vs1[NL * kLineB];
  __shared__ __attribute__((aligned(16))) int kind[2][32];  // read 16 bytes at a time
  __shared__ int64_t rpos[2][32];
  __shared__ float qcos[kRopePairs], qsin[kRopePairs];
  __shared__ int sidx[HCA ? 1 : CAP];
  __shared__ __attribute__((aligned(16))) uint2 xch[NW][kWave];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int gq = lane / 16, l16 = lane % 16;
  const int ngroups = (p.H + 15) / 16;
  const int64_t qrow = blockIdx.x / ngroups;
  const int h = (int)(blockIdx.x % ngroups) * 16 + l16;
  const bool hok = h < p.H;
  SplitInfo si;
  si.b = (int)(qrow / p.Lq);
  si.t = p.q_pos0 + qrow % p.Lq;
  si.n_c = HCA ? (int)((si.t + 1) / p.m) : p.topk;
  si.lo = si.t - p.W + 1 > 0 ? si.t - p.W + 1 : 0;
  si.row_lo = attn_raw_row(p, si.lo);
  si.n_w = p.W > 0 ? (int)(si.t - si.lo + 1) : 0;
  const int S = si.n_c + p.W;
  si.s0 = 0;
  si.s1 = S;
  const int ntiles = (S + 31) / 32;

  // The query's idx slots into LDS; head group 0 counts each entry's
  // selections, keeping the ranks the counters return in registers until the
  // end (storing them here would wait for every atomic's round trip).
  constexpr int RK = HCA ? 1 : (CAP + NT - 1) / NT;
  int rk[RK];
  const bool count = !HCA && g.cnt && blockIdx.x % ngroups == 0;
  if constexpr (!HCA) {
#pragma unroll
    for (int it = 0; it < RK; ++it) {
      const int r = tid + it * NT;
      rk[it] = -1;
      if (r < si.n_c) {
        const int32_t j = p.idx[qrow * p.topk + r];
        sidx[r] = j;
        if (count && j >= 0 && j < p.N_cap) rk[it] = atomicAdd(g.cnt + (int64_t)si.b * p.N_cap + j, 1);
      }
    }
  }
  const double rev = kRopeRev[tid % kRopePairs];
  if (tid < kRopePairs) rope_cos_sin_f(si.t, rev, &qcos[tid], &qsin[tid]);
  __syncthreads();
  // q, dO and out fragments (B operands: head l16, dims 32s + 8g ..), issued
  // before the tile copies so that waiting for them leaves the copies in flight
  const int64_t hrow = (qrow * p.H + (hok ? h : 0)) * D;
  uint4 qraw[QN], draw[QN], oraw[QN];
#pragma unroll
  for (int s = 0; s < QN; ++s) {
    qraw[s] = *reinterpret_cast<const uint4*>((const T*)p.q + hrow + 32 * s + 8 * gq);
    draw[s] = *reinterpret_cast<const uint4*>((const T*)g.dout + hrow + 32 * s + 8 * gq);
    oraw[s] = *reinterpret_cast<const uint4*>((const T*)p.out + hrow + 32 * s + 8 * gq);
  }
  const float lse = hok ? p.lse[qrow * p.H + h] : 0.f;
  issue_tile<T, D, NW, HCA, CAP>(p, si, sidx, 0, Ks0, Vs0, kind[0], rpos[0]);
  issue_tile<T, D, NW, HCA, CAP>(p, si, sidx, 32, Ks1, Vs1, kind[1], rpos[1]);
  bf16x8 qf[QN], dof[QN];
  float dl = 0.f;
#pragma unroll
  for (int s = 0; s < QN; ++s) {
    const int d0 = 32 * s + 8 * gq;
    uint4 raw = hok ? qraw[s] : make_uint4(0, 0, 0, 0);
    if (d0 >= D - kRopeDims) {
      float v[8];
      Chunk<T>::unpack(raw, v);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int pr = (d0 + e - (D - kRopeDims)) / 2;
        const float c = qcos[pr], sn = qsin[pr], x0 = v[e], x1 = v[e + 1];
        v[e] = x0 * c - x1 * sn;
        v[e + 1] = x0 * sn + x1 * c;
      }
      raw = Chunk<T>::pack(v);
    }
    qf[s] = __builtin_bit_cast(bf16x8, raw);
    const uint4 dr = hok ? draw[s] : make_uint4(0, 0, 0, 0);
    dof[s] = __builtin_bit_cast(bf16x8, dr);
    float dv[8], ov[8];
    Chunk<T>::unpack(dr, dv);
    Chunk<T>::unpack(oraw[s], ov);
#pragma unroll
    for (int e = 0; e < 8; ++e) dl = fmaf(dv[e], ov[e], dl);
    // the rotated q (bf16, as attended) for the key/value pass
    if (wave == 0 && hok) *reinterpret_cast<uint4*>((T*)g.w.qr + hrow + d0) = raw;
  }
  dl += __shfl_xor(dl, 16, kWave);
  dl += __shfl_xor(dl, 32, kWave);
  if (wave == 0 && gq == 0 && hok)
    g.w.dsink_part[qrow * p.H + h] = p.sink ? -__expf(p.sink[h] - lse) * dl : 0.f;
  const float lse2 = hok ? lse * kLog2e : INFINITY;  // padded heads: P = 0
  const float cscale = kLog2e / sqrtf((float)D);
  const float rsq = 1.f / sqrtf((float)D);
  f32x4 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float2* pdq = g.w.pds + qrow * (int64_t)g.S * p.H + h;
  attn_lds_barrier();  // row kinds/positions of the first tiles are visible

  auto step = [&](int tt, uint8_t* Kb, uint8_t* Vb, int bi) {
    const int ts = 32 * tt;
    const bool win = si.n_w > 0 && ts + 32 > si.n_c;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));  // this tile's copies (the next tile's may fly)
    attn_lds_barrier();
    if (win) {  // window keys rotated in LDS; thread t always takes pair t % 32
      for (int e = tid; e < 32 * kRopePairs; e += NT) {
        const int r = e / kRopePairs, pr = e % kRopePairs;
        if (kind[bi][r] != 2) continue;
        float c, sn;
        rope_cos_sin_f(rpos[bi][r], rev, &c, &sn);
        uint32_t* wp = reinterpret_cast<uint32_t*>(Kb + lds_pos<ROWB, k_line<T, D>()>(r, (D - kRopeDims + 2 * pr) * 2));
        const uint32_t v = *wp;
        const float x0 = bf16_bits_to_f32((uint16_t)(v & 0xFFFF)), x1 = bf16_bits_to_f32((uint16_t)(v >> 16));
        *wp = (uint32_t)f32_to_bf16_bits(x0 * c - x1 * sn) | ((uint32_t)f32_to_bf16_bits(x0 * sn + x1 * c) << 16);
      }
      attn_lds_barrier();
    }
    // This wave's tile reads and the pair's exchange are inline-asm blocks,
    // each waiting for its own reads before it ends: the compiler's wait
    // analysis loses these reads' LDS alias information and would otherwise
    // drain every copy in flight (the next tile's too) before them.
    const uint32_t kr = lds_addr(Kb) + lds_pos<ROWB, k_line<T, D>()>(16 * wave + l16, 16 * gq);
    const uint32_t vr = lds_addr(Vb) + lds_pos<ROWB, kLineB>(16 * wave + l16, 16 * gq);
    const uint32_t ka = lds_addr(&kind[bi][16 * wave + 4 * gq]);
    u32x4 kf0, kf1, kf2, kf3, vf0, vf1, vf2, vf3, kd;
    __asm__ volatile(
        "ds_read_b128 %0, %9\n\t"
        "ds_read_b128 %1, %9 offset:64\n\t"
        "ds_read_b128 %2, %9 offset:128\n\t"
        "ds_read_b128 %3, %9 offset:192\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %10 offset:64\n\t"
        "ds_read_b128 %6, %10 offset:128\n\t"
        "ds_read_b128 %7, %10 offset:192\n\t"
        "ds_read_b128 %8, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kf0), "=&v"(kf1), "=&v"(kf2), "=&v"(kf3), "=&v"(vf0), "=&v"(vf1), "=&v"(vf2), "=&v"(vf3), "=&v"(kd)
        : "v"(kr), "v"(vr), "v"(ka)
        : "memory");
    const u32x4 kf[QN] = {kf0, kf1, kf2, kf3}, vf[QN] = {vf0, vf1, vf2, vf3};
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f}, pacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < QN; ++s) {
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[s]), qf[s], sacc, 0, 0, 0);
      pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[s]), dof[s], pacc, 0, 0, 0);
    }
    float ds[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 16 * wave + 4 * gq + v, sp = ts + row;
      const bool ok = hok && kd[v] != 0;
      const float pv = ok ? exp2f(sacc[v] * cscale - lse2) : 0.f;
      ds[v] = pv * (pacc[v] - dl);
      if (hok && sp < S) pdq[(int64_t)sp * p.H] = make_float2(pv, ds[v] * rsq);
    }
    // dS^T of all 32 rows as the B operand: rows 4g..4g+3 and 16+4g..16+4g+3
    const u32x2 mine = {(uint32_t)f32_to_bf16_bits(ds[0]) | ((uint32_t)f32_to_bf16_bits(ds[1]) << 16),
                        (uint32_t)f32_to_bf16_bits(ds[2]) | ((uint32_t)f32_to_bf16_bits(ds[3]) << 16)};
    u32x2 oth;
    __asm__ volatile(
        "ds_write_b64 %1, %2\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_barrier\n\t"
        "ds_read_b64 %0, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(oth)
        : "v"(lds_addr(&xch[wave][lane])), "v"(mine), "v"(lds_addr(&xch[wave ^ 1][lane]))
        : "memory");
    const u32x2 t0 = wave == 0 ? mine : oth, t1 = wave == 0 ? oth : mine;
    const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{t0[0], t0[1], t1[0], t1[1]});
    // dq^T += K^T dS^T for this wave's half of D (transposed LDS reads of K)
    const int dt0 = wave * (D / 32);
    const int j4 = l16 / 4, jm = l16 % 4;
    const uint32_t ta = lds_addr(Kb) + lds_pos<ROWB, k_line<T, D>()>(4 * gq + j4, jm * 8) + dt0 * 32;
    const uint32_t tb = lds_addr(Kb) + lds_pos<ROWB, k_line<T, D>()>(16 + 4 * gq + j4, jm * 8) + dt0 * 32;
    u32x2 a0, a1, a2, a3, b0, b1, b2, b3;
    __asm__ volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:32\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:96\n\t"
        "ds_read_b64_tr_b16 %4, %9\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:32\n\t"
        "ds_read_b64_tr_b16 %6, %9 offset:64\n\t"
        "ds_read_b64_tr_b16 %7, %9 offset:96\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3)
        : "v"(ta), "v"(tb)
        : "memory");
    const u32x2 lo[4] = {a0, a1, a2, a3}, hi[4] = {b0, b1, b2, b3};
#pragma unroll
    for (int q = 0; q < D / 32; ++q) {
      const bf16x8 kk = __builtin_bit_cast(bf16x8, u32x4{lo[q][0], lo[q][1], hi[q][0], hi[q][1]});
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, pf, acc[q], 0, 0, 0);
    }
    attn_lds_barrier();
    issue_tile<T, D, NW, HCA, CAP>(p, si, sidx, 32 * (tt + 2), Kb, Vb, kind[bi], rpos[bi]);
  };
  for (int tt = 0; tt < ntiles; tt += 2) {
    step(tt, Ks0, Vs0, 0);
    if (tt + 1 < ntiles) step(tt + 1, Ks1, Vs1, 1);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS outlives the workgroup
  if constexpr (!HCA) {
    if (count)
#pragma unroll
      for (int it = 0; it < RK; ++it)
        if (rk[it] >= 0) g.rank[qrow * p.topk + tid + it * NT] = rk[it];
  }
  if (!hok) return;
  // dq = RoPE^T(sum dS k, t) / sqrt(D): lane holds dims 16(dt0 + q) + 4g .. + 3 of head h
  float* dqrow = g.dq + (qrow * p.H + h) * D;
#pragma unroll
  for (int q = 0; q < D / 32; ++q) {
    const int d = 16 * (wave * (D / 32) + q) + 4 * gq;
    float x[4] = {acc[q][0] * rsq, acc[q][1] * rsq, acc[q][2] * rsq, acc[q][3] * rsq};
    if (d >= D - kRopeDims) {
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const int pr = (d + e - (D - kRopeDims)) / 2;
        const float c = qcos[pr], sn = qsin[pr], x0 = x[e], x1 = x[e + 1];
        x[e] = x0 * c + x1 * sn;
        x[e + 1] = -x0 * sn + x1 * c;
      }
    }
    *reinterpret_cast<float4*>(dqrow + d) = make_float4(x[0], x[1], x[2], x[3]);
  }
}

// ------------------------------------------------------ inverse index (CSA)
__global__ void bwd_zero_kernel(int* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

// Exclusive scan of 256 per-thread values in LDS (Hillis-Steele); returns
// this thread's exclusive prefix and *total.
__device__ __forceinline__ int scan256(int v, int* buf, int* total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int x = tid >= o ? buf[tid - o] : 0;
    __syncthreads();
    buf[tid] += x;
    __syncthreads();
  }
  const int inc = buf[tid];
  *total = buf[255];
  __syncthreads();
  return inc - v;
}

// off[e] = exclusive prefix of cnt within its block of kScanBlock entries;
// bsum[block] = the block's total.
__global__ __launch_bounds__(256) void bwd_scan_block_kernel(const int* cnt, int64_t E, int* off, int* bsum) {
  __shared__ int buf[256];
  constexpr int PER = kScanBlock / 256;
  const int64_t e0 = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * PER;
  int v[PER], s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    v[i] = e0 + i < E ? cnt[e0 + i] : 0;
    s += v[i];
  }
  int total;
  int run = scan256(s, buf, &total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (e0 + i < E) off[e0 + i] = run;
    run += v[i];
  }
  if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

// bsum[0..n) -> exclusive prefix sums, one workgroup, 256 at a time.
__global__ __launch_bounds__(256) void bwd_scan_top_kernel(int* bsum, int n) {
  __shared__ int buf[256];
  int carry = 0;
  for (int c0 = 0; c0 < n; c0 += 256) {
    const int i = c0 + threadIdx.x;
    const int v = i < n ? bsum[i] : 0;
    int total;
    const int ex = scan256(v, buf, &total);
    if (i < n) bsum[i] = carry + ex;
    carry += total;
  }
}

// Each valid pair i (= qrow * topk + slot, < 2^31) into its entry's list, at
// its rank from the counting atomics (no atomics here).
__global__ void bwd_fill_kernel(AttnArgs p, int npairs, const int* off, const int* bsum, const int* rank, int* list) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < npairs; i += gridDim.x * blockDim.x) {
    const int32_t j = p.idx[i];
    if (j < 0 || j >= p.N_cap) continue;
    const int64_t e = (int64_t)(i / p.topk / p.Lq) * p.N_cap + j;
    list[off[e] + bsum[e / kScanBlock] + rank[i]] = i;
  }
}

// ------------------------------------------------------- key/value pass
// Sort a[0..m) ascending in LDS (m a power of two; bitonic network, one
// barrier per stage, every thread of the workgroup taking part).
__device__ __forceinline__ void bitonic_sort_lds(int* a, int m) {
  for (int k = 2; k <= m; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < m / 2; i += blockDim.x) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1)), hi = lo | j;
        const bool up = (lo & k) == 0;
        const int x = a[lo], y = a[hi];
        if ((x > y) == up) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
}

// Sort a[0..n) (distinct values, n <= 2 * blockDim.x) ascending in LDS:
// every element's rank is the count of smaller ones (broadcast reads), one
// barrier, then each is written at its rank.
__device__ __forceinline__ void rank_sort_lds(int* a, int n) {
  const int t = threadIdx.x, nt = blockDim.x;
  const int x0 = t < n ? a[t] : 0, x1 = t + nt < n ? a[t + nt] : 0;
  int r0 = 0, r1 = 0;
  for (int j = 0; j < n; ++j) {
    const int y = a[j];
    r0 += y < x0;
    r1 += y < x1;
  }
  __syncthreads();
  if (t < n) a[r0] = x0;
  if (t + nt < n) a[r1] = x1;
  __syncthreads();
}

// Workgroup = one compressed entry (blocks [0, B * N_cap)) or one raw row of
// the window range (the rest; raw rows outside it are zeroed by
// bwd_zero_rows_kernel). A lane owns 8 consecutive dims of the row; the D/8 lanes of a
// lane group take one pair at a time, so a wave works on 64 / (D/8) pairs
// per step and the workgroup on kKvWaves times as many, pair k going to
// lane group k mod NP. The pairs of a window row or an HCA entry are a query
// range in query order; a CSA entry's list (filled in no particular order)
// is sorted in LDS first. Each lane group then sums its pairs in float32 in
// that fixed order, and the NP partial sums are added in a fixed order: the
// same bits on every call. A list too long for LDS is instead summed in
// 64-bit fixed point (units of 2^-32, exact, so order-free) in chunks.
constexpr int kKvCap = 8192;  // pairs of an entry staged and sorted in LDS

template <typename T, int D, bool HCA>
__global__ __launch_bounds__(kKvThreads) void attn_bwd_kv_kernel(BwdKvArgs g) {
  constexpr int LPP = D / 8;           // lanes per pair
  constexpr int GP = kWave / LPP;      // pairs per wave step
  constexpr int NP = kKvWaves * GP;    // pairs per workgroup step
  static_assert(NP * 2 * D * 8 <= kKvCap * 4, "partial sums fit the list buffer");
  const AttnArgs& p = g.a;
  __shared__ __attribute__((aligned(16))) int s_buf[kKvCap];  // the list, then the partial sums

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int gp = lane / LPP, d0 = (lane % LPP) * 8;
  const int64_t ecount = (int64_t)p.B * p.N_cap;
  const int64_t blk = blockIdx.x;
  const bool win = blk >= ecount;
  const int b = (int)(win ? (blk - ecount) / g.nwr : blk / p.N_cap);
  const int64_t r = win ? g.wr0 + (blk - ecount) % g.nwr : blk % p.N_cap;
  const int64_t s_pos = p.raw_pos0 + r;  // window rows: absolute position
  int64_t n = 0, start = 0, i0 = 0;
  if (win) {
    if (p.W > 0) {
      const int64_t a0 = s_pos - p.q_pos0, a1 = s_pos + p.W - 1 - p.q_pos0;
      i0 = a0 > 0 ? a0 : 0;
      const int64_t i1 = a1 < p.Lq - 1 ? a1 : p.Lq - 1;
      n = i1 >= i0 ? i1 - i0 + 1 : 0;
    }
  } else if (HCA) {
    const int64_t a0 = (r + 1) * p.m - 1 - p.q_pos0;
    i0 = a0 > 0 ? a0 : 0;
    n = p.Lq > i0 ? p.Lq - i0 : 0;
  } else if (g.listed) {
    n = g.w.cnt[blk];
    start = g.w.off[blk] + g.w.bsum[blk / kScanBlock];
  }
  const bool listed = !win && !HCA;
  const bool exact = listed && n > kKvCap;

  const T* qr = (const T*)g.w.qr;
  const T* dout = (const T*)g.dout;
  // One step of lane group gp over pairs [0, cn) of the current range:
  // pair k = kb + gp; the sums over heads of dS qr (u) and P dO (w).
  auto pair_sums = [&](int ks, int64_t base, float* u, float* w) {
    int64_t qrow, slot;
    if (listed) {
      const int pi = s_buf[ks];
      qrow = pi / p.topk;
      slot = pi - qrow * p.topk;
    } else {
      const int64_t i = i0 + base + ks;
      qrow = (int64_t)b * p.Lq + i;
      if (win) {
        const int64_t t = p.q_pos0 + i;
        const int64_t lo = t - p.W + 1 > 0 ? t - p.W + 1 : 0;
        slot = (HCA ? (t + 1) / p.m : p.topk) + (s_pos - lo);
      } else {
        slot = r;
      }
    }
    const float2* pd = g.w.pds + (qrow * g.S + slot) * p.H;
    const T* qh = qr + qrow * p.H * D + d0;
    const T* oh = dout + qrow * p.H * D + d0;
#pragma unroll
    for (int v = 0; v < 8; ++v) u[v] = w[v] = 0.f;
    auto head = [&](int h, float2 w2) {
      float xq[8], xo[8];
      ld_vec<T, 8>(qh + h * D, xq);
      ld_vec<T, 8>(oh + h * D, xo);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        u[v] = fmaf(w2.y, xq[v], u[v]);
        w[v] = fmaf(w2.x, xo[v], w[v]);
      }
    };
    if (p.H % 2 == 0) {  // two heads' (P, dS) per 16-byte load
#pragma unroll 2
      for (int h = 0; h < p.H; h += 2) {
        const float4 w4 = *reinterpret_cast<const float4*>(pd + h);
        head(h, make_float2(w4.x, w4.y));
        head(h + 1, make_float2(w4.z, w4.w));
      }
    } else {
      for (int h = 0; h < p.H; ++h) head(h, pd[h]);
    }
  };
  const int part = wave * GP + gp;
  // The NP partial sums, added in index order; a thread finishes dims 2e,
  // 2e+1 of dk (e < D/2) or dv (e >= D/2) and writes them.
  auto finish = [&](float x0, float x1, int kv, int d) {
    if (win && kv == 0 && d >= D - kRopeDims) {  // window keys: back to the unrotated frame
      float c, sn;
      rope_cos_sin(s_pos, (d - (D - kRopeDims)) / 2, &c, &sn);
      const float y0 = x0 * c + x1 * sn, y1 = -x0 * sn + x1 * c;
      x0 = y0;
      x1 = y1;
    }
    float* o = (kv == 0 ? (win ? g.dk_raw : g.dk_c) : (win ? g.dv_raw : g.dv_c)) +
               (win ? (int64_t)b * p.T_raw + r : (int64_t)b * p.N_cap + r) * D;
    *reinterpret_cast<float2*>(o + d) = make_float2(x0, x1);
  };

  if (!exact) {
    if (listed && n > 0) {
      if (n <= 2 * kKvThreads) {
        for (int i = tid; i < n; i += kKvThreads) s_buf[i] = g.w.list[start + i];
        __syncthreads();
        rank_sort_lds(s_buf, (int)n);
      } else {
        const int m = 1 << (32 - __clz((int)n - 1));
        for (int i = tid; i < m; i += kKvThreads) s_buf[i] = i < n ? g.w.list[start + i] : 0x7FFFFFFF;
        __syncthreads();
        bitonic_sort_lds(s_buf, m);
      }
    }
    float fk[8], fv[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) fk[v] = fv[v] = 0.f;
    for (int kb = wave * GP; kb < n; kb += NP) {
      const int kk = kb + gp;
      float u[8], w[8];
      pair_sums(kk < n ? kk : kb, 0, u, w);
      if (kk < n)
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          fk[v] += u[v];
          fv[v] += w[v];
        }
    }
    __syncthreads();  // the list's readers are done
    float* sf = reinterpret_cast<float*>(s_buf);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      sf[(part * 2 + 0) * D + d0 + v] = fk[v];
      sf[(part * 2 + 1) * D + d0 + v] = fv[v];
    }
    __syncthreads();
    for (int e = tid; e < D; e += kKvThreads) {
      const int kv = e / (D / 2), d = 2 * (e % (D / 2));
      float x0 = 0.f, x1 = 0.f;
      for (int q = 0; q < NP; ++q) {
        x0 += sf[(q * 2 + kv) * D + d];
        x1 += sf[(q * 2 + kv) * D + d + 1];
      }
      finish(x0, x1, kv, d);
    }
  } else {
    long long ak[8], av[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) ak[v] = av[v] = 0;
    for (int64_t c0 = 0; c0 < n; c0 += kKvCap) {
      const int cn = (int)(n - c0 < kKvCap ? n - c0 : kKvCap);
      __syncthreads();  // the previous chunk's readers are done
      for (int i = tid; i < cn; i += kKvThreads) s_buf[i] = g.w.list[start + c0 + i];
      __syncthreads();
      for (int kb = wave * GP; kb < cn; kb += NP) {
        const int kk = kb + gp;
        float u[8], w[8];
        pair_sums(kk < cn ? kk : kb, c0, u, w);
        if (kk < cn)
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            ak[v] += to_fix(u[v]);
            av[v] += to_fix(w[v]);
          }
      }
    }
    __syncthreads();
    long long* sl = reinterpret_cast<long long*>(s_buf);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      sl[(part * 2 + 0) * D + d0 + v] = ak[v];
      sl[(part * 2 + 1) * D + d0 + v] = av[v];
    }
    __syncthreads();
    for (int e = tid; e < D; e += kKvThreads) {
      const int kv = e / (D / 2), d = 2 * (e % (D / 2));
      long long s0 = 0, s1 = 0;
      for (int q = 0; q < NP; ++q) {
        s0 += sl[(q * 2 + kv) * D + d];
        s1 += sl[(q * 2 + kv) * D + d + 1];
      }
      finish((float)((double)s0 * (1.0 / 4294967296.0)), (float)((double)s1 * (1.0 / 4294967296.0)), kv, d);
    }
  }
}

// Raw rows of no query's window: zero gradients.
__global__ void bwd_zero_rows_kernel(float* dk, float* dv, int B, int T_raw, int D, int64_t wr0, int nwr) {
  const int64_t n = (int64_t)B * T_raw * D;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = (i / D) % T_raw;
    if (r < wr0 || r >= wr0 + nwr) {
      dk[i] = 0.f;
      dv[i] = 0.f;
    }
  }
}

// dsink[h] = sum over query rows in a fixed order: workgroup h, thread t
// sums rows t, t + 256, ... in order, then a fixed tree over the threads.
__global__ __launch_bounds__(256) void dsink_sum_kernel(const float* part, int64_t rows, int H, float* dsink) {
  __shared__ float red[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  float s = 0.f;
  for (int64_t r = tid; r < rows; r += 256) s += part[r * H + h];
  red[tid] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) dsink[h] = red[0];
}

inline size_t al256(size_t n) { return (n + 255) / 256 * 256; }

struct BwdSizes {
  size_t pds, qr, sink, cnt, off, bsum, list, rank;
  size_t total() const { return pds + qr + sink + cnt + off + bsum + list + rank; }
};

BwdSizes bwd_sizes(int B, int Lq, int H, int D, int64_t N_cap, int S, int topk) {
  const size_t rows = (size_t)B * Lq, E = topk > 0 ? (size_t)B * N_cap : 0;
  BwdSizes z;
  z.pds = al256(rows * S * H * sizeof(float2));
  z.qr = al256(rows * H * D * sizeof(float));  // room for f32 q
  z.sink = al256(rows * H * sizeof(float));
  z.cnt = al256(E * sizeof(int));
  z.off = al256(E * sizeof(int));
  z.bsum = al256((E + kScanBlock - 1) / kScanBlock * sizeof(int));
  z.list = al256(rows * (size_t)topk * sizeof(int));
  z.rank = z.list;
  return z;
}

}  // namespace

size_t attn_bwd_ws_bytes(int B, int Lq, int H, int D, int64_t N_cap, int S, int topk) {
  return bwd_sizes(B, Lq, H, D, N_cap, S, topk).total() + 256;
}

int launch_attn_bwd(const AttnArgs& a, bool hca, int S, int kv_dtype, const void* dout, float* dq, float* dk_c,
                    float* dv_c, float* dk_raw, float* dv_raw, float* dsink, void* ws, hipStream_t st) {
  const BwdSizes z = bwd_sizes(a.B, a.Lq, a.H, a.D, a.N_cap, S, hca ? 0 : a.topk);
  uint8_t* w8 = (uint8_t*)ws;
  BwdWs w;
  w.pds = (float2*)w8;             w8 += z.pds;
  w.qr = w8;                       w8 += z.qr;
  w.dsink_part = (float*)w8;       w8 += z.sink;
  w.cnt = (int*)w8;                w8 += z.cnt;
  w.off = (int*)w8;                w8 += z.off;
  w.bsum = (int*)w8;               w8 += z.bsum;
  w.list = (int*)w8;               w8 += z.list;
  w.rank = (int*)w8;
  const int64_t rows = (int64_t)a.B * a.Lq;
  const int64_t E = (int64_t)a.B * a.N_cap;
  const int64_t npairs = rows * a.topk;
  const bool listed = !hca && npairs > 0;
  if (listed) {  // counters of the inverse index, counted by the query pass
    const int64_t nz = E;
    const int zb = (int)((nz + 255) / 256 < 4096 ? (nz + 255) / 256 : 4096);
    hipLaunchKernelGGL(bwd_zero_kernel, dim3(zb), dim3(256), 0, st, w.cnt, nz);
  }
  if (rows > 0) {
    AttnBwdArgs g;
    g.a = a;
    g.cnt = listed ? w.cnt : nullptr;
    g.rank = listed ? w.rank : nullptr;
    g.S = S;
    g.dout = dout;
    g.dq = dq;
    g.w = w;
    const dim3 grid((unsigned)(rows * ((a.H + kBwdHeads - 1) / kBwdHeads)));
#define CSA_BWD(TT, DD)                                                                                    \
  if (hca) hipLaunchKernelGGL((attn_bwd_q_kernel<TT, DD, true>), grid, dim3(kBwdThreads), 0, st, g);      \
  else hipLaunchKernelGGL((attn_bwd_q_kernel<TT, DD, false>), grid, dim3(kBwdThreads), 0, st, g)
    if (kv_dtype == 0) {
      if (a.D == 128) { CSA_BWD(float, 128); } else { CSA_BWD(float, 512); }
    } else if (a.D == 128) {
      const dim3 mgrid((unsigned)(rows * ((a.H + 15) / 16)));
      if (hca) hipLaunchKernelGGL((attn_bwd_q_mfma_kernel<128, true, 1>), mgrid, dim3(2 * kWave), 0, st, g);
      else if (a.topk <= 1024) hipLaunchKernelGGL((attn_bwd_q_mfma_kernel<128, false, 1024>), mgrid, dim3(2 * kWave), 0, st, g);
      else hipLaunchKernelGGL((attn_bwd_q_mfma_kernel<128, false, 2048>), mgrid, dim3(2 * kWave), 0, st, g);
    } else {
      CSA_BWD(uint16_t, 512);
    }
#undef CSA_BWD
  }
  if (listed) {  // offsets (scan of the counts), then the lists
    const int nblk = (int)((E + kScanBlock - 1) / kScanBlock);
    hipLaunchKernelGGL(bwd_scan_block_kernel, dim3(nblk), dim3(256), 0, st, w.cnt, E, w.off, w.bsum);
    hipLaunchKernelGGL(bwd_scan_top_kernel, dim3(1), dim3(256), 0, st, w.bsum, nblk);
    const int pb = (int)((npairs + 255) / 256 < 4096 ? (npairs + 255) / 256 : 4096);
    hipLaunchKernelGGL(bwd_fill_kernel, dim3(pb), dim3(256), 0, st, a, (int)npairs, w.off, w.bsum, w.rank, w.list);
  }
  // raw rows in some query's window: positions max(0, q_pos0 - W + 1) .. q_pos0 + Lq - 1
  const int64_t lo_first = a.q_pos0 - a.W + 1 > 0 ? a.q_pos0 - a.W + 1 : 0;
  const int64_t wr0 = a.W > 0 && a.Lq > 0 ? lo_first - a.raw_pos0 : 0;
  const int nwr = a.W > 0 && a.Lq > 0 ? (int)(a.q_pos0 + a.Lq - lo_first) : 0;
  if ((int64_t)a.B * a.T_raw > 0 && nwr < a.T_raw) {
    const int64_t nz = (int64_t)a.B * a.T_raw * a.D;
    const int zb = (int)((nz + 255) / 256 < 4096 ? (nz + 255) / 256 : 4096);
    hipLaunchKernelGGL(bwd_zero_rows_kernel, dim3(zb), dim3(256), 0, st, dk_raw, dv_raw, a.B, a.T_raw, a.D, wr0, nwr);
  }
  const int64_t kv_blocks = E + (int64_t)a.B * nwr;
  if (kv_blocks > 0) {
    BwdKvArgs g;
    g.a = a;
    g.S = S;
    g.listed = listed;
    g.wr0 = wr0;
    g.nwr = nwr;
    g.dout = dout;
    g.w = w;
    g.dk_c = dk_c; g.dv_c = dv_c; g.dk_raw = dk_raw; g.dv_raw = dv_raw;
    const dim3 grid((unsigned)kv_blocks);
#define CSA_BWD_KV(TT, DD)                                                                                  \
  if (hca) hipLaunchKernelGGL((attn_bwd_kv_kernel<TT, DD, true>), grid, dim3(kKvThreads), 0, st, g);      \
  else hipLaunchKernelGGL((attn_bwd_kv_kernel<TT, DD, false>), grid, dim3(kKvThreads), 0, st, g)
    if (kv_dtype == 0) {
      if (a.D == 128) { CSA_BWD_KV(float, 128); } else { CSA_BWD_KV(float, 512); }
    } else {
      if (a.D == 128) { CSA_BWD_KV(uint16_t, 128); } else { CSA_BWD_KV(uint16_t, 512); }
    }
#undef CSA_BWD_KV
  }
  // with no query rows the kernel writes zeros
  if (dsink) hipLaunchKernelGGL(dsink_sum_kernel, dim3(a.H), dim3(256), 0, st, w.dsink_part, rows, a.H, dsink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
