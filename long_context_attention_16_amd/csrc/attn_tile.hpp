// Tiles of source rows staged HBM -> LDS for the attention kernels (the
// forward in attn.hip and the backward's query pass in attn_bwd.hip): the LDS
// line layout, the row sources, the direct-to-LDS tile copies and the RoPE of
// window rows in LDS.
#pragma once
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

// LDS tile of 32 source rows: 1 KB lines (every wave load writes one line),
// each followed by a pad so the fragment reads spread over the LDS banks. A
// 16-byte read serves 16 lanes (256 bytes, all 64 banks) per cycle: the K
// reads of 16 consecutive one-line rows are conflict-free with a 1040-byte
// line (260 words, 4 banks apart), while the transposed 8-byte V reads
// (8 rows x 4 lanes per 32 lanes) want 1056 (264 words, 8 apart).
constexpr int kLineB = 1024 + 32;
template <typename T, int D> constexpr int k_line() { return sizeof(T) == 2 && D == 512 ? 1024 + 16 : kLineB; }
constexpr int kMaxSplitRows = 576;  // CSA splits: at most 576 rows (k <= 2048, W <= 1024: S <= 3072)

// LDS offset of byte `byte` of tile row r (rows longer than a line continue
// in the next line, after the pad).
template <int ROWB, int LINE = kLineB>
__device__ __forceinline__ int lds_pos(int r, int byte) {
  const int b = r * ROWB + byte;
  return (b >> 10) * LINE + (b & 1023);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Workgroup barrier for LDS data: waits for this wave's LDS operations only,
// then s_barrier. __syncthreads' fence would also wait for every outstanding
// global-to-LDS copy (the counter is in order), draining the tile prefetch;
// copies are waited for explicitly (vmcnt) where their tile is used.
__device__ __forceinline__ void attn_lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding; expcnt and lgkmcnt not waited).
__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
  return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 0x3) << 14);
}

struct SplitInfo {
  int64_t t, lo, row_lo;  // row_lo: raw row of window position lo
  int b, n_c, n_w, s0, s1;
};

// Source of split row sp: kind 0 = masked, 1 = compressed entry, 2 = window
// row at absolute position *pos; *src = element offset of the row. Branch
// free (selects, and an idx slot read clamped into the split's range), so
// the copy loops around it stay straight-line code.
template <int D, bool HCA, int CAP = kMaxSplitRows>
__device__ __forceinline__ int row_source(const AttnArgs& p, const SplitInfo& si, const int* sidx, int sp,
                                          int64_t* src, int64_t* pos) {
  const bool in_split = sp < si.s1;
  const bool comp = sp < si.n_c;
  int64_t j = sp;
  if constexpr (!HCA) {
    int slot = sp - si.s0;
    slot = slot < 0 ? 0 : (slot > CAP - 1 ? CAP - 1 : slot);
    j = sidx[slot];
  }
  const bool jok = j >= 0 && j < p.N_cap;
  const int64_t wpos = si.lo + (sp - si.n_c);
  const bool wok = sp - si.n_c < si.n_w;
  const int kind = !in_split ? 0 : (comp ? (jok ? 1 : 0) : (wok ? 2 : 0));
  *src = kind == 1 ? ((int64_t)si.b * p.N_cap + j) * D
                   : (kind == 2 ? ((int64_t)si.b * p.T_raw + attn_window_row(p, si.row_lo, sp - si.n_c)) * D : 0);
  *pos = kind == 2 ? wpos : 0;
  return kind;
}

// Issue the direct-to-LDS loads of the tile starting at split row ts, and
// record each row's kind and position. Every wave issues 2*NL/NW loads.
template <typename T, int D, int NW, bool HCA, int CAP = kMaxSplitRows>
__device__ __forceinline__ void issue_tile(const AttnArgs& p, const SplitInfo& si, const int* sidx, int ts,
                                           uint8_t* Ks, uint8_t* Vs, int* kind_out, int64_t* pos_out) {
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int NL = 32 * ROWB / 1024;
  // A fixed trip count and a scalar wave index keep the copies in
  // straight-line code: behind per-lane branches the compiler's own wait
  // analysis loses track of which buffer has copies in flight and drains
  // them all before the next LDS read.
  constexpr int PER = (NL + NW - 1) / NW;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const uint8_t* kc = (const uint8_t*)p.k_c;
  const uint8_t* vc = (const uint8_t*)p.v_c;
  const uint8_t* kr = (const uint8_t*)p.k_raw;
  const uint8_t* vr = (const uint8_t*)p.v_raw;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int L = wave + NW * u;
    if (NL % NW != 0 && L >= NL) break;  // wave-uniform: only when waves outnumber lines
    const int byte = L * 1024 + lane * 16;
    const int r = byte / ROWB;
    const int in_row = byte % ROWB;
    int64_t src, pos;
    const int kind = row_source<D, HCA, CAP>(p, si, sidx, ts + r, &src, &pos);
    // every lane of row r stores the same kind and position (no branch)
    kind_out[r] = kind;
    pos_out[r] = pos;
    const int64_t off = kind ? src * (int64_t)sizeof(T) + in_row : in_row;  // masked: row 0 (finite)
    const uint8_t* ks = (kind == 2 ? kr : kc) + off;
    const uint8_t* vs = (kind == 2 ? vr : vc) + off;
    __builtin_amdgcn_global_load_lds((const void*)ks, (__attribute__((address_space(3))) void*)(Ks + L * k_line<T, D>()), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)vs, (__attribute__((address_space(3))) void*)(Vs + L * kLineB), 16, 0, 0);
  }
}

// cos/sin of the tile's window rows (only rows of kind 2 are filled). A
// thread always evaluates pair threadIdx.x % 32 (the thread count is a
// multiple of 32), whose frequency `rev` it loaded once: a table load here,
// in the tile loop, would be waited for with every copy issued before it.
__device__ __forceinline__ void rope_table(const int* kind, const int64_t* pos, float (*rc)[kRopePairs + 1],
                                           float (*rs)[kRopePairs + 1], int nt_threads, double rev) {
  for (int e = threadIdx.x; e < 32 * kRopePairs; e += nt_threads) {
    const int r = e / kRopePairs, pr = e % kRopePairs;
    if (kind[r] == 2) rope_cos_sin_f(pos[r], rev, &rc[r][pr], &rs[r][pr]);
  }
}

// Rotate, in LDS, the last 64 dims of the tile's window rows.
template <typename T, int D>
__device__ __forceinline__ void rope_rows_lds(uint8_t* Ks, const int* kind, float (*rc)[kRopePairs + 1],
                                              float (*rs)[kRopePairs + 1], int nt_threads) {
  constexpr int ROWB = D * (int)sizeof(T);
  for (int e = threadIdx.x; e < 32 * kRopePairs; e += nt_threads) {
    const int r = e / kRopePairs, pr = e % kRopePairs;
    if (kind[r] != 2) continue;
    const int d = D - kRopeDims + 2 * pr;
    const float c = rc[r][pr], sn = rs[r][pr];
    if constexpr (sizeof(T) == 2) {
      uint32_t* w = reinterpret_cast<uint32_t*>(Ks + lds_pos<ROWB, k_line<T, D>()>(r, d * 2));
      const uint32_t v = *w;
      const float x0 = bf16_bits_to_f32((uint16_t)(v & 0xFFFF)), x1 = bf16_bits_to_f32((uint16_t)(v >> 16));
      *w = (uint32_t)f32_to_bf16_bits(x0 * c - x1 * sn) | ((uint32_t)f32_to_bf16_bits(x0 * sn + x1 * c) << 16);
    } else {
      float2* w = reinterpret_cast<float2*>(Ks + lds_pos<ROWB, k_line<T, D>()>(r, d * 4));
      const float2 v = *w;
      *w = make_float2(v.x * c - v.y * sn, v.x * sn + v.y * c);
    }
  }
}

// Rotate, in LDS, the last 64 dims of the tile's window rows, evaluating
// each cos/sin where it is used: thread t always takes pair t % 32, whose
// frequency `rev` it holds (the thread count is a multiple of 32). Same
// values as rope_table + rope_rows_lds, without the tables' LDS.
template <typename T, int D>
__device__ __forceinline__ void rope_rows_lds_direct(uint8_t* Ks, const int* kind, const int64_t* pos, double rev,
                                                     int nt_threads) {
  constexpr int ROWB = D * (int)sizeof(T);
  for (int e = threadIdx.x; e < 32 * kRopePairs; e += nt_threads) {
    const int r = e / kRopePairs, pr = e % kRopePairs;
    if (kind[r] != 2) continue;
    float c, sn;
    rope_cos_sin_f(pos[r], rev, &c, &sn);
    const int d = D - kRopeDims + 2 * pr;
    if constexpr (sizeof(T) == 2) {
      uint32_t* w = reinterpret_cast<uint32_t*>(Ks + lds_pos<ROWB, k_line<T, D>()>(r, d * 2));
      const uint32_t v = *w;
      const float x0 = bf16_bits_to_f32((uint16_t)(v & 0xFFFF)), x1 = bf16_bits_to_f32((uint16_t)(v >> 16));
      *w = (uint32_t)f32_to_bf16_bits(x0 * c - x1 * sn) | ((uint32_t)f32_to_bf16_bits(x0 * sn + x1 * c) << 16);
    } else {
      float2* w = reinterpret_cast<float2*>(Ks + lds_pos<ROWB, k_line<T, D>()>(r, d * 4));
      const float2 v = *w;
      *w = make_float2(v.x * c - v.y * sn, v.x * sn + v.y * c);
    }
  }
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Byte address of an LDS object (its offset in the workgroup's LDS), for
// LDS reads written in inline asm.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <typename T, int D>
constexpr bool attn_double_buffered(int nw) {
  return 2 * (32 * D * (int)sizeof(T) / 1024) / nw <= 32 &&
         2 * (32 * D * (int)sizeof(T) / 1024) * (k_line<T, D>() + kLineB) <= 140 * 1024;
}

}  // namespace csa
