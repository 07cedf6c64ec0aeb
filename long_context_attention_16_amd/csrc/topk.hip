// K3 — per-query top-k over the indexer scores.
//
// Source: "DeepSeek V4 重磅開源！…" (InfoQ), section 混合注意力機制: each query
// attends only k compressed entries (k = 512..1024) picked by the indexer.
// Rule fixed here (the pages are silent): order by (-score, j), so equal
// scores go to the lower index; -0 equals +0; the first min(k, n) entries are
// written in ascending j and the remaining slots hold -1.
//
// Design: one workgroup per query row. Scores map to order-preserving uint32
// keys; for rows that fit, the keys stay resident in LDS (128 KB). A 4-pass
// 8-bit radix select finds the k-th largest key T and how many entries equal
// to T must be taken. The histogram lives in LDS; the bin search is a
// block-wide scan over the 256 bins. Compaction then gives each thread a
// contiguous run of up to 64 entries whose "greater" and "equal" flags are
// 64-bit masks, so only two block scans are needed to place every selected
// index, in ascending order, with no sorting.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr int kTopkThreads = 512;
constexpr int kTopkLdsKeys = 32768;

// Exclusive scan over the workgroup; *total receives the sum. Every thread
// of the workgroup must call it.
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* sh) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) sh[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTopkThreads / kWave; ++i) {
    const int s = sh[i];
    off += i < w ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

template <bool LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(int Lq, int64_t q_pos0, int m,
                                                            int64_t N_cap,
                                                            const float* __restrict__ scores,
                                                            int topk, int32_t* __restrict__ idx_out) {
  const int64_t row = blockIdx.x;
  const int i = (int)(row % Lq);
  const int n = (int)((q_pos0 + i + 1) / m);
  const float* s = scores + row * N_cap;
  int32_t* out = idx_out + row * topk;
  const int tid = threadIdx.x;

  if (n <= topk) {
    for (int j = tid; j < topk; j += kTopkThreads) out[j] = j < n ? j : -1;
    return;
  }

  __shared__ uint32_t keys[LDS ? kTopkLdsKeys : 1];
  __shared__ int hist[256];
  __shared__ int sh[kTopkThreads / kWave];
  __shared__ uint32_t sel_digit;
  __shared__ int sel_above;

  if (LDS) {
    for (int j = tid; j < n; j += kTopkThreads) keys[j] = score_key(s[j]);
  }
  auto key_at = [&](int j) -> uint32_t { return LDS ? keys[j] : score_key(s[j]); };

  // Radix select of the k-th largest key.
  uint32_t prefix = 0, pmask = 0;
  int kr = topk;  // rank still wanted among keys matching the prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += kTopkThreads) {
      const uint32_t k = key_at(j);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 0xFF], 1);
    }
    __syncthreads();
    const int bin = 255 - tid;  // descending digits over threads 0..255
    const int c = tid < 256 ? hist[bin] : 0;
    int tot;
    const int above = block_excl_scan(c, &tot, sh);
    if (tid < 256 && above < kr && above + c >= kr) {
      sel_digit = (uint32_t)bin;
      sel_above = above;
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    pmask |= 0xFFu << shift;
    kr -= sel_above;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = kr;  // entries equal to T to take, lowest indices first

  // Compaction in rounds of up to 64 entries per thread.
  int out_base = 0, eq_taken = 0;
  for (int base = 0; base < n; base += kTopkThreads * 64) {
    const int cnt = min(kTopkThreads * 64, n - base);
    const int ept = (cnt + kTopkThreads - 1) / kTopkThreads;
    const int my0 = base + tid * ept;
    const int my_end = min(base + cnt, my0 + ept);
    uint64_t gt = 0, eq = 0;
    for (int e = 0; e < ept; ++e) {
      const int ee = (e + tid) % ept;  // rotated start spreads LDS banks
      const int j = my0 + ee;
      if (j < my_end) {
        const uint32_t k = key_at(j);
        gt |= (uint64_t)(k > T) << ee;
        eq |= (uint64_t)(k == T) << ee;
      }
    }
    const int ne = __popcll(eq);
    int eq_tot;
    const int eq_before = block_excl_scan(ne, &eq_tot, sh);
    int take = need_eq - eq_taken - eq_before;
    take = max(0, min(take, ne));
    uint64_t keep = 0, rest = eq;
    for (int q = 0; q < take; ++q) {
      const uint64_t low = rest & (~rest + 1);
      keep |= low;
      rest ^= low;
    }
    uint64_t sel = gt | keep;
    int sel_tot;
    int pos = out_base + block_excl_scan(__popcll(sel), &sel_tot, sh);
    while (sel) {
      const int bit = __builtin_ctzll(sel);
      sel &= sel - 1;
      out[pos++] = my0 + bit;
    }
    out_base += sel_tot;
    eq_taken += min(eq_tot, need_eq - eq_taken);
  }
}

int launch_topk(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, const float* scores, int topk,
                int32_t* idx_out, hipStream_t stream) {
  const int64_t rows = (int64_t)B * Lq;
  if (rows == 0) return 0;
  const int64_t n_max = (q_pos0 + Lq) / m;
  const dim3 grid((unsigned)rows), block(kTopkThreads);
  if (n_max <= kTopkLdsKeys)
    hipLaunchKernelGGL((topk_kernel<true>), grid, block, 0, stream, Lq, q_pos0, m, N_cap, scores, topk, idx_out);
  else
    hipLaunchKernelGGL((topk_kernel<false>), grid, block, 0, stream, Lq, q_pos0, m, N_cap, scores, topk, idx_out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
