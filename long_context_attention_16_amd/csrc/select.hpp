// Workgroup-wide radix select of the k largest 32-bit keys (the top-k rule
// of the indexer: key order first, then position). Shared by the top-k
// kernels and the indexer's fused per-chunk selection.
//
// Keys live in registers, KPT per thread, key[u] of thread t at position
// KPT*t + u (each thread owns a run of consecutive positions). A radix select
// on digits of at most 11 bits counts into an LDS histogram (each thread owns
// kTopkBins / THREADS bins for the search); every prefix sum is a DPP wave
// scan plus one LDS exchange of wave totals. Compaction: a thread's selected
// keys are a bit mask over its run, so one exclusive scan of the per-thread
// counts gives every selected position its output slot in ascending order
// (and, when keys equal to the threshold must be ranked, one more scan of
// the per-thread counts of equal keys), with no sort and no per-row ballots.
#pragma once
#include "common.hpp"

namespace csa {

constexpr int kTopkBins = 2048;

template <int THREADS, int KPT> struct TopkShared {
  // the radix histogram; after the search, free for staging the selected
  // entries' indices (with `stage` for their keys), so they reach HBM in
  // coalesced stores (emit scatters one slot per selected key)
  int hist[kTopkBins];
  uint32_t stage[kTopkBins];
  uint32_t wmin[THREADS / kWave], wmax[THREADS / kWave];
  int wtot[2][THREADS / kWave];
  uint32_t sel_digit;
  int sel_above;
  int sel_count;  // keys in the selected digit's bin
};

// Inclusive scan over the 64 lanes of a wave with DPP moves: shifts by 1, 2,
// 4 and 8 lanes within each row of 16, then the last lane of row 0 added to
// row 1 and of row 2 to row 3 (row_bcast:15), then the last lane of row 1 to
// rows 2 and 3 (row_bcast:31). Lanes whose source is outside the pattern
// add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive scan over the workgroup of v >= 0; *total gets the sum. Every
// thread calls it in the same order; `par` (a register) alternates the LDS
// buffer of wave totals, so one barrier per scan suffices.
template <int THREADS, int KPT>
__device__ __forceinline__ int block_scan(int v, int* total, TopkShared<THREADS, KPT>& S, int& par) {
  constexpr int NW = THREADS / kWave;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int inc = wave_incl_scan(v);
  const int pre = inc - v;
  const int wt = __builtin_amdgcn_readlane(inc, kWave - 1);
  const int buf = par;
  par ^= 1;
  if (lane == 0) S.wtot[buf][w] = wt;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int x = S.wtot[buf][i];
    off += i < w ? x : 0;
    tot += x;
  }
  *total = tot;
  return off + pre;
}

// One radix pass over the register keys, counted as key - base: count digit
// (x >> shift) & dmask of valid x whose higher bits equal `prefix` (under
// `pmask`); find the digit
// holding the kr-th largest. Returns it; *above = counted keys in higher digits,
// *count = keys in its bin (read after the pass's last barrier; the next pass
// writes these fields only after barriers every thread has passed).
// Thread t owns the BPT consecutive bins just below nb - BPT*t (nb = dmask + 1).
template <int THREADS, int KPT>
__device__ __forceinline__ uint32_t radix_pass(const uint32_t (&key)[KPT], uint32_t base, int n, uint32_t prefix, uint32_t pmask,
                                               int shift, uint32_t dmask, int kr, TopkShared<THREADS, KPT>& S,
                                               int& par, int* above, int* count) {
  constexpr int BPT = kTopkBins / THREADS;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < BPT; ++q) S.hist[tid + q * THREADS] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if (tid * KPT + u < n && ((key[u] - base) & pmask) == prefix)
      atomicAdd(&S.hist[((key[u] - base) >> shift) & dmask], 1);
  __syncthreads();
  const int nb = (int)dmask + 1;
  const int top = nb - 1 - BPT * tid;  // this thread's highest bin; bins top, top-1, ... top-BPT+1
  int h[BPT], sum = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    h[q] = top - q >= 0 ? S.hist[top - q] : 0;
    sum += h[q];
  }
  int tot;
  const int ab = block_scan<THREADS, KPT>(sum, &tot, S, par);
  if (top >= 0 && ab < kr && ab + sum >= kr) {
    int acc = ab;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (acc < kr && acc + h[q] >= kr) {
        S.sel_digit = (uint32_t)(top - q);
        S.sel_above = acc;
        S.sel_count = h[q];
      }
      acc += h[q];
    }
  }
  __syncthreads();
  *above = S.sel_above;
  *count = S.sel_count;
  return S.sel_digit;
}

// Top k (k < n <= THREADS*KPT) of the register keys, key[u] of thread t being
// position KPT*t + u; emit(slot, u) on the threads whose key[u] is selected,
// slots ascending with position. emit may write S.hist and S.stage
// (k <= kTopkBins); block_select_out copies them out after a barrier.
template <int THREADS, int KPT, class Emit>
__device__ __forceinline__ void block_select(const uint32_t (&key)[KPT], int n, int k, TopkShared<THREADS, KPT>& S,
                                             const Emit& emit) {
  constexpr int NW = THREADS / kWave;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  int par = 0, above, bc;
  // Keys are counted as key - min over the valid keys, and digits cover only
  // the bits of max - min: the top bits of float keys (sign, exponent) take
  // few values, and a first digit taken there would pile most keys into a
  // few histogram bins (serialized LDS atomics) and resolve little.
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if (tid * KPT + u < n) { mn = min(mn, key[u]); mx = max(mx, key[u]); }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, kWave));
  }
  if (lane == 0) { S.wmin[w] = mn; S.wmax[w] = mx; }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) { mn = min(mn, S.wmin[i]); mx = max(mx, S.wmax[i]); }
  // Threshold T and whether every key equal to T is taken. Up to three
  // digits of at most 11 bits cover the bits of max - min; a pass
  // whose selected bin is taken whole ends the search early (the selection is
  // then every key at or above the bin's lower bound, no ties to rank).
  const uint32_t base = mn;
  int rem = mn == mx ? 0 : 32 - __builtin_clz(mx - mn);  // digit bits left
  uint32_t pmask = rem == 32 ? 0u : ~0u << rem;
  uint32_t prefix = 0;  // of key - base
  uint32_t T = base;
  bool all_eq = false, done = false;
  int need_eq = 0;
  int kr = k;
  bc = n;  // with no bits left (all keys equal) the bin is every key
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    if (done || rem == 0) break;
    const int wd = rem < 11 ? rem : 11;
    const int shift = rem - wd;
    const uint32_t dmask = (1u << wd) - 1u;
    const uint32_t d = radix_pass<THREADS, KPT>(key, base, n, prefix, pmask, shift, dmask, kr, S, par, &above, &bc);
    kr -= above;
    prefix |= d << shift;
    pmask |= dmask << shift;
    rem = shift;
    if (kr == bc) {  // the bin is taken whole
      T = base + prefix;
      all_eq = true;
      done = true;
    }
  }
  if (!done) {  // no bits left: the bin holds the single key value T
    T = base + prefix;
    need_eq = kr;
    all_eq = kr == bc;
  }

  int tot;
  static_assert(KPT <= 32, "selection bits of a thread fit one word");
  uint32_t take = 0;  // bit u: key[u] is selected
  if (all_eq) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) take |= (uint32_t)(tid * KPT + u < n && key[u] >= T) << u;
  } else {
    // keys above T are taken; of the keys equal to T the need_eq first in
    // position order, ranked by a scan of each thread's count of them
    uint32_t eq = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool ok = tid * KPT + u < n;
      take |= (uint32_t)(ok && key[u] > T) << u;
      eq |= (uint32_t)(ok && key[u] == T) << u;
    }
    int r = block_scan<THREADS, KPT>(__popc(eq), &tot, S, par);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool e = (eq >> u) & 1u;
      take |= (uint32_t)(e && r < need_eq) << u;
      r += e;
    }
  }
  int slot = block_scan<THREADS, KPT>(__popc(take), &tot, S, par);
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    if ((take >> u) & 1u) emit(slot, u);
    slot += (take >> u) & 1u;
  }
}

// v[u] = src[min(p0 + u, n - 1)], u < KPT (n >= 1): this thread's run of
// positions. A run entirely below n is read as whole vectors of up to 16
// bytes (the source need only be 4-byte aligned; the vector type says so).
typedef uint32_t sel_u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t sel_u32x2 __attribute__((ext_vector_type(2), aligned(4)));
template <int KPT, typename E>
__device__ __forceinline__ void load_run(const E* src, int p0, int n, E (&v)[KPT]) {
  constexpr int BYTES = KPT * (int)sizeof(E) < 16 ? KPT * (int)sizeof(E) : 16;
  constexpr int PER = BYTES / (int)sizeof(E);
  static_assert(KPT % PER == 0 && (BYTES == 16 || BYTES == 8), "runs of whole 8- or 16-byte vectors");
  if (p0 + KPT <= n) {
#pragma unroll
    for (int c = 0; c < KPT / PER; ++c) {
      if constexpr (BYTES == 16) {
        const sel_u32x4 x = *reinterpret_cast<const sel_u32x4*>(src + p0 + c * PER);
        __builtin_memcpy(&v[c * PER], &x, 16);
      } else {
        const sel_u32x2 x = *reinterpret_cast<const sel_u32x2*>(src + p0 + c * PER);
        __builtin_memcpy(&v[c * PER], &x, 8);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < KPT; ++u) v[u] = src[min(p0 + u, n - 1)];
  }
}

// Write the k slots staged by an emit into S.hist (indices) and S.stage
// (keys, if okey) to HBM with consecutive threads on consecutive slots.
template <int THREADS, int KPT>
__device__ __forceinline__ void block_select_out(TopkShared<THREADS, KPT>& S, int k, int32_t* oidx, uint32_t* okey) {
  __syncthreads();
  for (int p = threadIdx.x; p < k; p += THREADS) {
    oidx[p] = S.hist[p];
    if (okey) okey[p] = S.stage[p];
  }
}

// The top k of n (key, index) candidates, consecutive lists of k in
// ascending index order each (a list's position order is index order and
// lists come in chunk order, so ties still go to the lower index), written as
// indices to oidx (and keys to okey, if not null) in ascending index order.
// n <= k passes the candidates through.
template <int THREADS, int KPT>
__device__ __forceinline__ void merge_lists(TopkShared<THREADS, KPT>& S, int n, int k, const uint32_t* __restrict__ ik,
                                            const int32_t* __restrict__ ii, int32_t* __restrict__ oidx,
                                            uint32_t* __restrict__ okey) {
  const int tid = threadIdx.x;
  if (n <= k) {  // a single list passes through
    for (int p = tid; p < k; p += THREADS) {
      oidx[p] = ii[p];
      if (okey) okey[p] = ik[p];
    }
    return;
  }
  uint32_t key[KPT];
  int32_t idx[KPT];
  load_run<KPT>(ik, tid * KPT, n, key);
  load_run<KPT>(ii, tid * KPT, n, idx);
  block_select<THREADS, KPT>(key, n, k, S, [&](int slot, int u) {
    S.hist[slot] = idx[u];
    S.stage[slot] = key[u];
  });
  block_select_out(S, k, oidx, okey);
}

}  // namespace csa
