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
// holds one group of queries (64 or 128 rows) in LDS for the whole launch and
// streams 32-entry tiles of k_I from HBM through a ring of register buffers,
// with the next tiles' loads in flight while the current one is multiplied. Per-query
// visibility limits are computed once per workgroup into LDS, so the tile
// loop does no 64-bit arithmetic.
#pragma once
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace csa {

constexpr int kIdxWaves = 4;
constexpr int kIdxTilesPerWave = 16;  // 32-entry tiles per wave: scores to HBM, and fused with k <= 512
constexpr int kIdxColsPerWG = kIdxWaves * kIdxTilesPerWave * 32;  // entries per workgroup (2048)

// Operand fragment of one MFMA k-step for one lane, by format. The order in
// which the d_I elements of a row are fed to the k-steps is free as long as
// the q and k operands use the same one; each format picks one that lets a
// lane fetch 16 contiguous bytes per load.
template <int FMT> struct IdxOp;

template <> struct IdxOp<0> {  // f32, 32x32x2: step s, half h holds element 8(s/4) + 4h + s%4
  static constexpr int KW = 2;
  typedef float Frag;
  template <int DI>
  static __device__ __forceinline__ Frag load(const uint8_t* row, const uint8_t*, int s, int half, int* sc) {
    *sc = 127;
    return reinterpret_cast<const float*>(row)[8 * (s / 4) + 4 * half + s % 4];
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
  template <int DI>
  static __device__ __forceinline__ Frag load(const uint8_t* row, const uint8_t*, int s, int half, int* sc) {
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
  template <int DI>
  static __device__ __forceinline__ Frag load(const uint8_t* row, const uint8_t*, int s, int half, int* sc) {
    *sc = 127;
    const int k0 = s * 64 + half * 32;
    const bool in = DI >= 64 || k0 < DI;  // d_I = 32: the upper half-wave has no data
    // Loads stay unconditional (a branch around them would make the memory
    // counter waits of the tile loop conservative); the empty half is zeroed.
    uint4 a = *reinterpret_cast<const uint4*>(row + (in ? k0 : 0));
    uint4 b = *reinterpret_cast<const uint4*>(row + (in ? k0 : 0) + 16);
    Frag f;
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    return in ? f : zero();
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
  template <int DI>
  static __device__ __forceinline__ Frag load(const uint8_t* row, const uint8_t* srow, int s, int half, int* sc) {
    const int k0 = s * 64 + half * 32;
    const bool in = DI >= 64 || k0 < DI;  // d_I = 32: the upper half-wave has no data
    const int kk = in ? k0 : 0;           // unconditional loads, as for fp8
    const int sv = srow[kk / 32];
    uint4 a = *reinterpret_cast<const uint4*>(row + kk / 2);
    *sc = in ? sv : 127;
    Frag f;
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = 0; f[5] = 0; f[6] = 0; f[7] = 0;
    return in ? f : zero();
  }
  static __device__ __forceinline__ Frag zero() { Frag f; for (int i = 0; i < 8; ++i) f[i] = 0; return f; }
  static __device__ __forceinline__ void mma(const Frag& a, int sa, const Frag& b, int sb, f32x16& c) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
  }
  static constexpr int row_bytes(int DI) { return DI / 2; }
};

// Register ring depth for k_I tiles. Two (one tile in flight while the
// previous one is multiplied) measured fastest on MI355X for every format:
// deeper rings keep more bytes in flight per wave but lengthen the ring's
// fill and drain at the ends of each wave's tile chain, and the HBM system is
// already saturated at this occupancy (two waves per SIMD).
template <int FMT, int MTILES, int DI> constexpr int idx_nbuf() { return 2; }

// Scores for one group of queries (MTILES*32 rows = G queries x HI heads)
// against the kIdxWaves * TPW * 32 entries of chunk c. Wave w takes the 32-entry
// tiles w, w + 4, w + 8, ... of the chunk; its trip count nt is wave-uniform.
// Tiles stream through a ring of NBUF register buffers: the loads of tile
// i + NBUF - 1 are issued before tile i is multiplied, so up to NBUF - 1
// tiles are in flight per wave. No load or store in the tile loop is
// conditional: the loop runs a multiple of NBUF steps, prefetches past the
// wave's last tile re-load that tile (an L2 hit), and score stores of
// invisible entries go out as raw buffer stores with an offset past the
// buffer's end, which the hardware drops. The memory counters then stay
// exact and the wait before each tile's MFMAs covers only that tile's loads.
//
// FUSE (groups of one query): the chunk's scores go to LDS instead of HBM
// and the workgroup then selects their top k (select.hpp), writing one
// candidate list of k (key, index) pairs per (row, chunk) in ascending index
// order, padded with key 0 / index -1. The lists of a row are merged by the
// top-k merge kernel; every entry of the row's top k is in its chunk's top k.
// A fused chunk holds at least 4k entries (TPW = 16 tiles per wave, 2048
// entries, for k <= 512; 32 tiles, 4096 entries, for k <= 1024), so the lists
// carry at most a quarter of the scores.
// LDS of one indexer workgroup (a struct, so that a kernel running several
// kinds of work can overlay it with the others' in one buffer).
template <int FMT, int HI, int DI, bool FUSE, int TPW> struct IdxShared {
  static constexpr int COLS = kIdxWaves * TPW * 32;  // entries per chunk
  static constexpr int MTILES = HI == 128 ? 4 : 2;
  static constexpr int G = MTILES * 32 / HI;  // queries per group
  typedef IdxOp<FMT> Op;
  typedef typename Op::Frag Frag;
  static constexpr int KS = (DI + Op::KW - 1) / Op::KW;
  static constexpr int kSelThreads = kIdxWaves * kWave;
  static constexpr int kSelKPT = COLS / kSelThreads;
  typedef TopkShared<kSelThreads, kSelKPT> SelShared;
  static constexpr int kScBytes = (COLS + kWave) * 4;
  int s_lim[G];                         // per query: visible entries n(t)
  float4 s_w[MTILES * 8];               // head weight of each of the MTILES*32 rows
  Frag s_a[MTILES * KS * kWave];        // q operand fragments
  uint8_t s_asc[FMT == 3 ? MTILES * KS * kWave : 1];  // their e8m0 scales (fp4)
  // Fused mode only: the chunk's scores (plus a dump row for masked lanes)
  // and the selection's scratch, carved from one buffer (16 bytes otherwise).
  __attribute__((aligned(16))) uint8_t s_fuse[FUSE ? kScBytes + sizeof(SelShared) : 16];
};

// One indexer work unit: blk is the unit's index (a kernel's block index).
template <int FMT, int HI, int DI, bool FUSE, int TPW>
__device__ __forceinline__ void index_qk_body(
    IdxShared<FMT, HI, DI, FUSE, TPW>& S, const int blk,
    int Lq, int64_t q_pos0, const int64_t* __restrict__ q_pos, int m, int64_t N_cap, int ngroups, int nchunks,
    const uint8_t* __restrict__ q_i, const uint8_t* __restrict__ q_s, const float* __restrict__ w_i,
    const uint8_t* __restrict__ k_i, const uint8_t* __restrict__ k_s, float* __restrict__ scores, int sbf,
    int topk, uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_idx) {
  typedef IdxShared<FMT, HI, DI, FUSE, TPW> Sh;
  constexpr int COLS = Sh::COLS;
  constexpr int MTILES = Sh::MTILES;
  constexpr int G = Sh::G;
  constexpr int NBUF = idx_nbuf<FMT, MTILES, DI>();
  // Padded steps of the ring then only ever fall on tiles past the group's
  // visible entries (stores masked), never past the end of the chunk.
  static_assert(TPW % NBUF == 0, "ring depth divides the tiles per wave");
  constexpr int kSelThreads = Sh::kSelThreads;
  constexpr int kSelKPT = Sh::kSelKPT;
  typedef IdxOp<FMT> Op;
  typedef typename Op::Frag Frag;
  constexpr int KS = Sh::KS;
  constexpr int RB = Op::row_bytes(DI);
  constexpr int SB = DI / 32;  // scale bytes per row (fp4)
  constexpr int NLIM = HI == 4 ? MTILES * 4 : G;  // visibility limits held per lane
  int* s_lim = S.s_lim;
  float4* s_w = S.s_w;
  Frag* s_a = S.s_a;
  uint8_t* s_asc = S.s_asc;
  typedef typename Sh::SelShared SelShared;
  constexpr int kScBytes = Sh::kScBytes;
  float* s_sc = reinterpret_cast<float*>(S.s_fuse);
  SelShared& s_sel = *reinterpret_cast<SelShared*>(S.s_fuse + (FUSE ? kScBytes : 0));

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32;
  const int l32 = lane % 32;
  const int c = blk % nchunks;  // chunk of COLS entries
  const int gg = blk / nchunks;
  const int b = gg / ngroups;
  q_pos0 = seq_pos(q_pos, q_pos0, b);  // from here on: this sequence's row-0 position
  const int i0 = (gg % ngroups) * G;
  const int nq = min(G, Lq - i0);
  const int64_t n_last = (q_pos0 + i0 + nq) / m;  // visible entries of the group's last query
  const int ntiles = (int)((n_last + 31) / 32);   // 32-entry tiles holding any of them
  const int tile0 = c * kIdxWaves * TPW;
  auto tile_of = [&](int i) { return tile0 + kIdxWaves * i + wave; };
  if (tile0 >= ntiles) {
    if constexpr (FUSE) {  // an empty chunk: a padding list
      const int64_t o = ((int64_t)b * Lq + i0) * nchunks + c;
      for (int p = threadIdx.x; p < topk; p += kSelThreads) {
        cand_key[o * topk + p] = 0u;
        cand_idx[o * topk + p] = -1;
      }
    }
    return;
  }
  const int nt = tile0 + wave < ntiles
                     ? min(TPW, (ntiles - tile0 - wave + kIdxWaves - 1) / kIdxWaves) : 0;
  const int tmax = max(nt - 1, 0);

  const int64_t kbase = (int64_t)b * N_cap;
  auto load_b = [&](int i, Frag* bf, int* bsc) {
    int64_t j = (int64_t)tile_of(min(i, tmax)) * 32 + l32;
    if (j >= N_cap) j = N_cap - 1;
    const uint8_t* rp = k_i + (kbase + j) * RB;
    const uint8_t* sp = FMT == 3 ? k_s + (kbase + j) * SB : nullptr;
#pragma unroll
    for (int s = 0; s < KS; ++s) bf[s] = Op::template load<DI>(rp, sp, s, half, &bsc[s]);
  };

  // Ring prologue: tiles 0 .. NBUF-2.
  Frag bb[NBUF][KS];
  int bs[NBUF][KS];
#pragma unroll
  for (int u = 0; u + 1 < NBUF; ++u) load_b(u, bb[u], bs[u]);

  // A operand (the group's q rows) into LDS in MFMA fragment order: entry
  // (mt, s, lane) is what lane `lane` feeds to k-step s of M tile mt, so the
  // tile loop reads it back with one conflict-free 16/32-byte LDS read per
  // lane. Rows past the group's last query are zero.
  for (int f = threadIdx.x; f < MTILES * KS * kWave; f += kIdxWaves * kWave) {
    const int ln = f % kWave, s_ = (f / kWave) % KS, mt = f / (kWave * KS);
    const int row = mt * 32 + ln % 32;
    const int qq = row / HI, h = row % HI;
    const int64_t qrow = ((int64_t)b * Lq + i0 + (qq < nq ? qq : 0)) * HI + h;
    int sc;
    Frag v = Op::template load<DI>(q_i + qrow * RB, FMT == 3 ? q_s + qrow * SB : nullptr, s_, ln / 32, &sc);
    if (qq >= nq) { v = Op::zero(); sc = 127; }
    s_a[f] = v;
    if constexpr (FMT == 3) s_asc[f] = (uint8_t)sc;
  }
  if (threadIdx.x < MTILES * 32) {
    const int row = threadIdx.x, qq = row / HI;
    reinterpret_cast<float*>(s_w)[row] = qq < nq ? w_i[((int64_t)b * Lq + i0 + qq) * HI + row % HI] : 0.f;
  }
  if (threadIdx.x < G) {
    const int qq = threadIdx.x;
    s_lim[qq] = qq < nq ? (int)((q_pos0 + i0 + qq + 1) / m) : -1;
  }
  __syncthreads();
  if (!FUSE && nt == 0) return;

  int lim[NLIM];
#pragma unroll
  for (int x = 0; x < NLIM; ++x) lim[x] = HI == 4 ? s_lim[(x / 4) * 8 + (x % 4) * 2 + half] : s_lim[x];

  // Score stores: raw buffer stores relative to row i0 of the group; a lane
  // with nothing to store uses an offset past num_records. The resource is
  // built from wave-uniform values, read as scalars (built from a
  // min<int64_t>, it would be taken as divergent and every store wrapped in a
  // loop over lanes). Fused: an LDS store, masked lanes writing a dump row.
  // bf16 scores (sbf): rows of score_stride(N_cap, 1) entries, each lane pair
  // stored as one word by its even lane (score_word), so every lane still
  // issues exactly one store per put (the 4-head layout instead pairs two
  // query rows per store, see compute_store).
  const int esz = sbf ? 2 : 4;
  const int64_t sstride = score_stride(N_cap, sbf);
  const uint64_t sbase = FUSE ? 0 : (uint64_t)((uint8_t*)scores + ((int64_t)b * Lq + i0) * sstride * esz);
  const uint32_t slo = __builtin_amdgcn_readfirstlane((uint32_t)sbase);
  const uint32_t shi = __builtin_amdgcn_readfirstlane((uint32_t)(sbase >> 32));
  const int snum = __builtin_amdgcn_readfirstlane((int)((int64_t)nq * sstride * esz));
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(((uint64_t)shi << 32) | slo), 0, snum, 0x00020000);
  constexpr int kDrop = 0x7FFFFFF0;
  const uint32_t srow = (uint32_t)(sstride * esz);
  const bool s_lane = !sbf || (lane & 1) == 0;  // lanes that store
  const int col0 = tile0 * 32;
  auto put = [&](int qq, int jrel, bool ok, float v) {
    if constexpr (FUSE) {
      s_sc[ok ? jrel - col0 : COLS + lane] = v;  // one query: qq == 0 whenever ok
    } else {
      const uint32_t word = score_word(v, sbf);
      const int off = ok && s_lane ? (int)((uint32_t)qq * srow + (uint32_t)jrel * (uint32_t)esz) : kDrop;
      __builtin_amdgcn_raw_buffer_store_b32(word, srsrc, off, 0, 0);
    }
  };

  auto compute_store = [&](const Frag* bf, const int* bsc, int i) {
    // The q fragments and head weights are re-read from LDS for every tile:
    // the barrier keeps them from being hoisted out of the loop into
    // MTILES * KS * sizeof(Frag) / 4 + 16 * MTILES loop-invariant registers.
    __asm__ volatile("" ::: "memory");
    f32x16 acc[MTILES];
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int f = (mt * KS + s) * kWave + lane;
        Op::mma(s_a[f], FMT == 3 ? (int)s_asc[f] : 127, bf[s], bsc[s], acc[mt]);
      }
    }
    const int jrel = tile_of(i) * 32 + l32;  // entry index
    if constexpr (HI == 4) {
      // each group of 4 registers is one query's 4 heads
      float vv[MTILES * 4];
#pragma unroll
      for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const float4 w4 = s_w[mt * 8 + a4 * 2 + half];
          float v = w4.x * relu_bits(acc[mt][a4 * 4]);
          v = fmaf(w4.y, relu_bits(acc[mt][a4 * 4 + 1]), v);
          v = fmaf(w4.z, relu_bits(acc[mt][a4 * 4 + 2]), v);
          v = fmaf(w4.w, relu_bits(acc[mt][a4 * 4 + 3]), v);
          vv[mt * 4 + a4] = v;
        }
      if (!FUSE && sbf) {
        // bf16 scores, two query rows per store: of rows A = (mt, a4) and
        // B = (mt, a4 + 1), the even lane of a pair writes A's entries
        // (2i, 2i+1) and the odd lane B's, each getting the value it lacks
        // from its neighbour in one swap, so every lane stores and a tile
        // takes half the stores (the kernel is bound by their issue).
        const bool even = (lane & 1) == 0;
        const int j0 = jrel & ~1;
#pragma unroll
        for (int p = 0; p < MTILES * 4; p += 2) {
          const int mt = p / 4, a4 = p % 4 + (even ? 0 : 1);
          const float send = even ? vv[p + 1] : vv[p];
          const float recv = __builtin_bit_cast(
              float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
          const float lo = even ? vv[p] : recv, hi = even ? recv : vv[p + 1];
          const uint32_t word = (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
          const int qq = mt * 8 + a4 * 2 + half;
          const int off = j0 < lim[mt * 4 + a4] ? (int)((uint32_t)qq * srow + (uint32_t)j0 * 2u) : kDrop;
          if constexpr (!FUSE) __builtin_amdgcn_raw_buffer_store_b32(word, srsrc, off, 0, 0);
        }
      } else {
#pragma unroll
        for (int p = 0; p < MTILES * 4; ++p)
          put((p / 4) * 8 + (p % 4) * 2 + half, jrel, jrel < lim[p], vv[p]);
      }
    } else {
      constexpr int gpq = HI / 8;  // register groups (of 4 rows x 2 halves) per query
      float run = 0.f;
#pragma unroll
      for (int g = 0; g < MTILES * 4; ++g) {
        const int mt = g / 4, a4 = g % 4;
        const float4 w4 = s_w[mt * 8 + a4 * 2 + half];
        run = fmaf(w4.x, relu_bits(acc[mt][a4 * 4]), run);
        run = fmaf(w4.y, relu_bits(acc[mt][a4 * 4 + 1]), run);
        run = fmaf(w4.z, relu_bits(acc[mt][a4 * 4 + 2]), run);
        run = fmaf(w4.w, relu_bits(acc[mt][a4 * 4 + 3]), run);
        if ((g + 1) % gpq == 0) {
          run += __shfl_xor(run, 32, kWave);
          const int qq = g / gpq;
          put(qq, jrel, half == 0 && jrel < lim[qq], run);
          run = 0.f;
        }
      }
    }
  };

  // Everything issued so far has landed before the loop, so the loop-entry
  // state of the memory counters is the steady state's.
  __builtin_amdgcn_s_waitcnt(0);
  for (int i = 0; i < nt; i += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      load_b(i + u + NBUF - 1, bb[(u + NBUF - 1) % NBUF], bs[(u + NBUF - 1) % NBUF]);
      compute_store(bb[u], bs[u], i + u);
    }
  }

  if constexpr (FUSE) {
    __syncthreads();  // the chunk's scores are in s_sc
    const int n = (int)max<int64_t>(0, min<int64_t>(COLS, (int64_t)s_lim[0] - col0));
    const int64_t o = (((int64_t)b * Lq + i0) * nchunks + c) * topk;
    uint32_t* ok = cand_key + o;
    int32_t* oi = cand_idx + o;
    // bf16 scores: keys of the rounded scores, selected as 16-bit keys
    auto keyof = [&](float x) { return sbf ? score_key_bf16(x) : score_key(x); };
    const int ksh = sbf ? 16 : 0;
    if (n <= topk) {  // every visible entry of the chunk is a candidate
      for (int p = threadIdx.x; p < topk; p += kSelThreads) {
        const bool v = p < n;
        ok[p] = v ? keyof(s_sc[p]) : 0u;
        oi[p] = v ? col0 + p : -1;
      }
      return;
    }
    uint32_t key[kSelKPT];
    {
      float v[kSelKPT];
      load_run<kSelKPT>(s_sc, (int)threadIdx.x * kSelKPT, n, v);
#pragma unroll
      for (int u = 0; u < kSelKPT; ++u) key[u] = keyof(v[u]) >> ksh;
    }
    block_select<kSelThreads, kSelKPT>(key, n, topk, s_sel, [&](int slot, int u) {
      s_sel.stage[slot] = key[u] << ksh;
      s_sel.hist[slot] = col0 + (int)threadIdx.x * kSelKPT + u;
    });
    block_select_out(s_sel, topk, oi, ok);
  }
}

template <int FMT, int HI, int DI, bool FUSE, int TPW>
__global__ __launch_bounds__(kIdxWaves * kWave) void index_qk_kernel(
    int Lq, int64_t q_pos0, const int64_t* __restrict__ q_pos, int m, int64_t N_cap, int ngroups, int nchunks,
    const uint8_t* __restrict__ q_i, const uint8_t* __restrict__ q_s, const float* __restrict__ w_i,
    const uint8_t* __restrict__ k_i, const uint8_t* __restrict__ k_s, float* __restrict__ scores, int sbf,
    int topk, uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_idx) {
  __shared__ IdxShared<FMT, HI, DI, FUSE, TPW> S;
  index_qk_body<FMT, HI, DI, FUSE, TPW>(S, blockIdx.x, Lq, q_pos0, q_pos, m, N_cap, ngroups, nchunks, q_i, q_s, w_i, k_i,
                                   k_s, scores, sbf, topk, cand_key, cand_idx);
}

// ---------------------------------------------------------------- launch
struct IdxArgs {
  dim3 grid;
  hipStream_t st;
  int Lq;
  int64_t q_pos0;
  const int64_t* q_pos;
  int m;
  int64_t N_cap;
  int ngroups, nchunks;
  const uint8_t *q, *qs;
  const float* w;
  const uint8_t *k, *ks;
  float* sc;
  int sbf;
  int topk;
  uint32_t* ck;
  int32_t* ci;
};

template <int FMT, int HI, int DI, bool FUSE, int TPW>
void idx_go(const IdxArgs& a) {
  hipLaunchKernelGGL((index_qk_kernel<FMT, HI, DI, FUSE, TPW>), a.grid, dim3(kIdxWaves * kWave), 0, a.st, a.Lq,
                     a.q_pos0, a.q_pos, a.m, a.N_cap, a.ngroups, a.nchunks, a.q, a.qs, a.w, a.k, a.ks, a.sc, a.sbf, a.topk,
                     a.ck, a.ci);
}

template <int FMT, bool FUSE, int TPW = kIdxTilesPerWave>
void idx_dispatch(int H_i, int d_i, const IdxArgs& a) {
#define CSA_IDX_D(HH)                                        \
  if (d_i == 32) idx_go<FMT, HH, 32, FUSE, TPW>(a);          \
  else if (d_i == 64) idx_go<FMT, HH, 64, FUSE, TPW>(a);     \
  else idx_go<FMT, HH, 128, FUSE, TPW>(a)
  switch (H_i) {
    case 4: CSA_IDX_D(4); break;
    case 8: CSA_IDX_D(8); break;
    case 16: CSA_IDX_D(16); break;
    case 32: CSA_IDX_D(32); break;
    case 64: CSA_IDX_D(64); break;
    default: CSA_IDX_D(128); break;
  }
#undef CSA_IDX_D
}

inline IdxArgs idx_args(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int64_t N_cap, int H_i,
                        const void* q_i, const uint8_t* q_s, const float* w_i, const void* k_i,
                        const uint8_t* k_s, hipStream_t stream, int nchunks) {
  IdxArgs a{};
  const int G = index_qk_queries_per_group(H_i);
  a.ngroups = (Lq + G - 1) / G;
  a.nchunks = nchunks;
  a.grid = dim3((unsigned)((int64_t)B * a.ngroups * a.nchunks));
  a.st = stream;
  a.Lq = Lq; a.q_pos0 = q_pos0; a.q_pos = q_pos; a.m = m; a.N_cap = N_cap;
  a.q = (const uint8_t*)q_i; a.qs = q_s; a.w = w_i; a.k = (const uint8_t*)k_i; a.ks = k_s;
  return a;
}

}  // namespace csa
