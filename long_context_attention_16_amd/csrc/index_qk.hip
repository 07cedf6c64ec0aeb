// K2 — Lightning Indexer scores on MFMA.
//
// I[t, j] = sum_h w[t, h] * max(0, <q_I[t, h, :], k_I[j, :]>) for j < n(t).
// Source: "DeepSeek V4 重磅開源！…" (InfoQ), section 混合注意力機制 (a light
// indexer selects the important compressed blocks per query) and section
// FP4 量化 (the indexer's QK path runs in FP4). The pages give no formula; the
// ReLU'd per-head dot product mixed by per-query head weights is the reading
// taken here.
//
// Design: the contraction over d_I is a dense GEMM with the (query, head)
// rows as M and the compressed entries as N, so it runs on MFMA 32x32 tiles
// (f32: 32x32x2; bf16: 32x32x16; fp8 e4m3 and MXFP4 e2m1: the scaled
// 32x32x64 f8f6f4 form, whose per-lane e8m0 scale covers exactly one 32-wide
// block of d_I). In the 32x32 result layout a lane holds one entry (column)
// and 16 rows, four consecutive rows per register group, so ReLU, the head
// weight and the sum over a query's heads are done in registers; only heads
// split across the two half-waves need one cross-lane add. Each workgroup
// holds one group of queries (64 or 128 rows) in registers for the whole
// launch and streams 32-entry tiles of k_I straight from HBM with the next
// tile's loads in flight while the current one is multiplied.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr int kIdxWaves = 4;
constexpr int kIdxTilesPerWave = 16;
constexpr int kIdxColsPerWG = kIdxWaves * kIdxTilesPerWave * 32;

// Operand fragment of one MFMA k-step for one lane, by format.
template <int FMT> struct IdxOp;

template <> struct IdxOp<0> {  // f32, 32x32x2: lane holds element k = 2s + half
  static constexpr int KW = 2;
  typedef float Frag;
  static __device__ __forceinline__ Frag load(const uint8_t* row, const uint8_t*, int DI, int s, int half, int* sc) {
    *sc = 127;
    return reinterpret_cast<const float*>(row)[s * 2 + half];
  }
  static __device__ __forceinline__ Frag zero() { return 0.f; }
  static __device__ __forceinline__ void mma(const Frag& a, int, const Frag& b, int, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static constexpr int row_bytes(int DI) { return DI * 4; }
};

template <> struct IdxOp<1> {  // bf16, 32x32x16: lane holds 8 elements at 16s + 8*half
  static constexpr int KW = 16;
  typedef bf16x8 Frag;
  static __device__ __forceinline__ Frag load(const uint8_t* row, const uint8_t*, int DI, int s, int half, int* sc) {
    *sc = 127;
    uint4 v = *reinterpret_cast<const uint4*>(row + (s * 16 + half * 8) * 2);
    return __builtin_bit_cast(Frag, v);
  }
  static __device__ __forceinline__ Frag zero() { return __builtin_bit_cast(Frag, make_uint4(0, 0, 0, 0)); }
  static __device__ __forceinline__ void mma(const Frag& a, int, const Frag& b, int, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static constexpr int row_bytes(int DI) { return DI * 2; }
};

template <> struct IdxOp<2> {  // fp8 e4m3, scaled 32x32x64 (unit scales): 32 bytes at 64s + 32*half
  static constexpr int KW = 64;
  typedef i32x8 Frag;
  static __device__ __forceinline__ Frag load(const uint8_t* row, const uint8_t*, int DI, int s, int half, int* sc) {
    *sc = 127;
    const int k0 = s * 64 + half * 32;
    if (k0 >= DI) return zero();
    uint4 a = *reinterpret_cast<const uint4*>(row + k0);
    uint4 b = *reinterpret_cast<const uint4*>(row + k0 + 16);
    Frag f;
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    return f;
  }
  static __device__ __forceinline__ Frag zero() { Frag f; for (int i = 0; i < 8; ++i) f[i] = 0; return f; }
  static __device__ __forceinline__ void mma(const Frag& a, int, const Frag& b, int, f32x16& c) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
  static constexpr int row_bytes(int DI) { return DI; }
};

template <> struct IdxOp<3> {  // MXFP4: 32 e2m1 codes (16 bytes) at 64s + 32*half, one e8m0 scale
  static constexpr int KW = 64;
  typedef i32x8 Frag;
  static __device__ __forceinline__ Frag load(const uint8_t* row, const uint8_t* srow, int DI, int s, int half, int* sc) {
    const int k0 = s * 64 + half * 32;
    if (k0 >= DI) { *sc = 127; return zero(); }
    *sc = srow[k0 / 32];
    uint4 a = *reinterpret_cast<const uint4*>(row + k0 / 2);
    Frag f;
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = 0; f[5] = 0; f[6] = 0; f[7] = 0;
    return f;
  }
  static __device__ __forceinline__ Frag zero() { Frag f; for (int i = 0; i < 8; ++i) f[i] = 0; return f; }
  static __device__ __forceinline__ void mma(const Frag& a, int sa, const Frag& b, int sb, f32x16& c) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
  }
  static constexpr int row_bytes(int DI) { return DI / 2; }
};

// Scores for one group of queries (MTILES*32 rows = G queries x H_i heads)
// against kIdxColsPerWG entries.
template <int FMT, int MTILES, int DI>
__global__ __launch_bounds__(kIdxWaves * kWave) void index_qk_kernel(
    int Lq, int64_t q_pos0, int m, int64_t N_cap, int H_i, int G, int ngroups, int nchunks,
    const uint8_t* __restrict__ q_i, const uint8_t* __restrict__ q_s, const float* __restrict__ w_i,
    const uint8_t* __restrict__ k_i, const uint8_t* __restrict__ k_s, float* __restrict__ scores) {
  typedef IdxOp<FMT> Op;
  constexpr int KS = (DI + Op::KW - 1) / Op::KW;
  constexpr int RB = Op::row_bytes(DI);
  constexpr int SB = DI / 32;  // scale bytes per row (fp4)

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32;
  const int l32 = lane % 32;
  const int chunk = blockIdx.x % nchunks;
  const int gg = blockIdx.x / nchunks;
  const int b = gg / ngroups;
  const int i0 = (gg % ngroups) * G;
  const int nq = min(G, Lq - i0);
  const int64_t n_last = (q_pos0 + i0 + nq) / m;  // visible entries of the group's last query
  const int64_t col0 = (int64_t)chunk * kIdxColsPerWG;
  if (col0 >= n_last) return;

  // A operand: this lane's row of each M tile, all k-steps.
  typename Op::Frag a[MTILES][KS];
  int asc[MTILES][KS];
#pragma unroll
  for (int mt = 0; mt < MTILES; ++mt) {
    const int row = mt * 32 + l32;
    const int qq = row / H_i, h = row % H_i;
    const bool ok = qq < nq;
    const int64_t qrow = ((int64_t)b * Lq + i0 + (ok ? qq : 0)) * H_i + h;
    const uint8_t* rp = q_i + qrow * RB;
    const uint8_t* sp = FMT == 3 ? q_s + qrow * SB : nullptr;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      a[mt][s] = ok ? Op::load(rp, sp, DI, s, half, &asc[mt][s]) : Op::zero();
      if (!ok) asc[mt][s] = 127;
    }
  }
  // Head weights of this lane's 16 result rows per tile.
  float wv[MTILES][16];
#pragma unroll
  for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = mt * 32 + 8 * (r / 4) + 4 * half + (r % 4);
      const int qq = row / H_i;
      wv[mt][r] = qq < nq ? w_i[((int64_t)b * Lq + i0 + qq) * H_i + row % H_i] : 0.f;
    }

  const int gpq = H_i / 8;  // register groups (of 4 rows x 2 halves) per query, H_i >= 8
  const int64_t kbase = (int64_t)b * N_cap;

  auto load_b = [&](int64_t j0, typename Op::Frag* bf, int* bsc) {
    int64_t j = j0 + l32;
    if (j >= N_cap) j = N_cap - 1;
    const uint8_t* rp = k_i + (kbase + j) * RB;
    const uint8_t* sp = FMT == 3 ? k_s + (kbase + j) * SB : nullptr;
#pragma unroll
    for (int s = 0; s < KS; ++s) bf[s] = Op::load(rp, sp, DI, s, half, &bsc[s]);
  };

  int tile = wave;
  int64_t j0 = col0 + (int64_t)tile * 32;
  if (tile >= kIdxTilesPerWave * kIdxWaves || j0 >= n_last) return;
  typename Op::Frag bcur[KS];
  int bsc[KS];
  load_b(j0, bcur, bsc);

  while (true) {
    const int ntile = tile + kIdxWaves;
    const int64_t nj0 = col0 + (int64_t)ntile * 32;
    const bool more = ntile < kIdxTilesPerWave * kIdxWaves && nj0 < n_last;
    typename Op::Frag bnext[KS];
    int bnsc[KS];
    if (more) load_b(nj0, bnext, bnsc);

    f32x16 acc[MTILES];
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) Op::mma(a[mt][s], asc[mt][s], bcur[s], bsc[s], acc[mt]);
    }

    const int64_t j = j0 + l32;
    float* srow = scores + ((int64_t)b * Lq + i0) * N_cap + j;
    if (H_i == 4) {
      // each group of 4 registers is one query's 4 heads
#pragma unroll
      for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          float v = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) v = fmaf(wv[mt][a4 * 4 + r], fmaxf(acc[mt][a4 * 4 + r], 0.f), v);
          const int qq = mt * 8 + a4 * 2 + half;
          if (qq < nq && j < (q_pos0 + i0 + qq + 1) / m) srow[(int64_t)qq * N_cap] = v;
        }
    } else {
      float run = 0.f;
#pragma unroll
      for (int g = 0; g < MTILES * 4; ++g) {
        const int mt = g / 4, a4 = g % 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) run = fmaf(wv[mt][a4 * 4 + r], fmaxf(acc[mt][a4 * 4 + r], 0.f), run);
        if ((g + 1) % gpq == 0) {
          run += __shfl_xor(run, 32, kWave);
          const int qq = g / gpq;
          if (half == 0 && qq < nq && j < (q_pos0 + i0 + qq + 1) / m) srow[(int64_t)qq * N_cap] = run;
          run = 0.f;
        }
      }
    }

    if (!more) break;
    tile = ntile;
    j0 = nj0;
#pragma unroll
    for (int s = 0; s < KS; ++s) { bcur[s] = bnext[s]; bsc[s] = bnsc[s]; }
  }
}

template <int FMT, int MTILES>
static void launch_idx_di(int DI, dim3 grid, dim3 block, hipStream_t st, int Lq, int64_t q_pos0, int m,
                          int64_t N_cap, int H_i, int G, int ngroups, int nchunks, const uint8_t* q,
                          const uint8_t* qs, const float* w, const uint8_t* k, const uint8_t* ks,
                          float* sc) {
#define CSA_IDX_LAUNCH(DD)                                                                       \
  hipLaunchKernelGGL((index_qk_kernel<FMT, MTILES, DD>), grid, block, 0, st, Lq, q_pos0, m, N_cap, \
                     H_i, G, ngroups, nchunks, q, qs, w, k, ks, sc)
  if (DI == 32) CSA_IDX_LAUNCH(32);
  else if (DI == 64) CSA_IDX_LAUNCH(64);
  else CSA_IDX_LAUNCH(128);
#undef CSA_IDX_LAUNCH
}

int launch_index_qk(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, int H_i, int d_i,
                    int fmt, const void* q_i, const uint8_t* q_s, const float* w_i,
                    const void* k_i, const uint8_t* k_s, float* scores, hipStream_t stream) {
  const int mtiles = H_i == 128 ? 4 : 2;
  const int G = (mtiles * 32) / H_i;
  const int ngroups = (Lq + G - 1) / G;
  const int64_t n_max = (q_pos0 + Lq) / m;
  const int nchunks = (int)((n_max + kIdxColsPerWG - 1) / kIdxColsPerWG);
  if (nchunks == 0 || B == 0 || Lq == 0) return 0;
  const dim3 grid((unsigned)((int64_t)B * ngroups * nchunks));
  const dim3 block(kIdxWaves * kWave);
  const uint8_t* q = (const uint8_t*)q_i;
  const uint8_t* k = (const uint8_t*)k_i;
#define CSA_IDX_FMT(F)                                                                              \
  if (mtiles == 2) launch_idx_di<F, 2>(d_i, grid, block, stream, Lq, q_pos0, m, N_cap, H_i, G, ngroups, \
                                       nchunks, q, q_s, w_i, k, k_s, scores);                        \
  else launch_idx_di<F, 4>(d_i, grid, block, stream, Lq, q_pos0, m, N_cap, H_i, G, ngroups, nchunks, q, \
                           q_s, w_i, k, k_s, scores)
  switch (fmt) {
    case 0: CSA_IDX_FMT(0); break;
    case 1: CSA_IDX_FMT(1); break;
    case 2: CSA_IDX_FMT(2); break;
    default: CSA_IDX_FMT(3); break;
  }
#undef CSA_IDX_FMT
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
