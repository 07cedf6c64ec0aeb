// K3 — per-query top-k over the indexer scores.
//
// Source: "DeepSeek V4 重磅開源！…" (InfoQ), section 混合注意力機制: each query
// attends only k compressed entries (k = 512..1024) picked by the indexer.
// Rule fixed here (the pages are silent): order by (-score, j), so equal
// scores go to the lower index; -0 equals +0; the first min(k, n) entries are
// written in ascending j and the remaining slots hold -1.
//
// Design. Scores map to order-preserving uint32 keys. One 1024-thread
// workgroup selects the top k of up to 32768 keys held in registers, 32 per
// thread: key[u] of thread t is position 1024u + t, so every load is
// coalesced. A radix select on 11-, 11- and 10-bit digits counts into an LDS
// histogram (each thread owns two bins for the search); every prefix sum is a
// ballot-built wave scan plus one LDS exchange of wave totals. Compaction
// counts, per (row u, wave), the equal and the selected keys with ballots and
// scans those 512 counts once each, so every selected position gets its
// output slot in ascending order with no sort.
// Rows longer than 32768 entries are cut into chunks; each chunk's top k
// (every global top-k entry is in its chunk's top k) forms a candidate list in
// ascending index order, and merge levels take the top k of groups of
// consecutive lists (list position order is index order, so ties still go to
// the lower index) until one list remains.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;  // 16
constexpr int kKPT = 32;                       // keys per thread
constexpr int kTkKeys = kTkThreads * kKPT;     // 32768
constexpr int kBins = 2048;

struct TkShared {
  int hist[kBins];
  int wtot[2][kTkWaves];
  int cnt[kKPT * kTkWaves];  // per (row, wave) counts, scanned in place
  uint32_t sel_digit;
  int sel_above;
};

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive scan over the workgroup of v in [0, 2^BITS); *total gets the sum.
// Every thread calls it in the same order; `par` (a register) alternates the
// LDS buffer of wave totals, so one barrier per scan suffices.
template <int BITS>
__device__ __forceinline__ int block_scan(int v, int* total, TkShared& S, int& par) {
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  int pre = 0, wt = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const uint64_t m = __ballot((v >> b) & 1);
    pre += lanes_below(m) << b;
    wt += __popcll(m) << b;
  }
  const int buf = par;
  par ^= 1;
  if (lane == 0) S.wtot[buf][w] = wt;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTkWaves; ++i) {
    const int x = S.wtot[buf][i];
    off += i < w ? x : 0;
    tot += x;
  }
  *total = tot;
  return off + pre;
}

// One radix pass over the register keys: count digit (key >> shift) & dmask of
// valid keys whose higher bits equal `prefix` (under `pmask`); find the digit
// holding the kr-th largest. Returns it; *above = counted keys in higher digits.
__device__ __forceinline__ uint32_t radix_pass(const uint32_t (&key)[kKPT], int n, uint32_t prefix, uint32_t pmask,
                                               int shift, uint32_t dmask, int kr, TkShared& S, int& par,
                                               int* above) {
  const int tid = threadIdx.x;
  S.hist[tid] = 0;
  S.hist[tid + kTkThreads] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kKPT; ++u)
    if (u * kTkThreads + tid < n && (key[u] & pmask) == prefix) atomicAdd(&S.hist[(key[u] >> shift) & dmask], 1);
  __syncthreads();
  // thread t owns bins hi = nb-1-2t and hi-1 (nb = dmask + 1; threads past nb/2 own none)
  const int nb = (int)dmask + 1;
  const int hi = nb - 1 - 2 * tid;
  const int h0 = hi >= 1 ? S.hist[hi] : 0;
  const int h1 = hi >= 1 ? S.hist[hi - 1] : 0;
  int tot;
  const int ab = block_scan<16>(h0 + h1, &tot, S, par);
  if (hi >= 1 && ab < kr && ab + h0 + h1 >= kr) {
    const bool first = ab + h0 >= kr;
    S.sel_digit = (uint32_t)(first ? hi : hi - 1);
    S.sel_above = first ? ab : ab + h0;
  }
  __syncthreads();
  *above = S.sel_above;
  return S.sel_digit;
}

// Top k (k < n <= 32768) of the register keys; emit(slot, u) on the threads
// whose key[u] is selected, slots ascending with position 1024u + tid.
template <class Emit>
__device__ __forceinline__ void block_select(const uint32_t (&key)[kKPT], int n, int k, TkShared& S,
                                             const Emit& emit) {
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  int par = 0, above;
  const uint32_t d0 = radix_pass(key, n, 0u, 0u, 21, 0x7FFu, k, S, par, &above);
  int kr = k - above;
  const uint32_t d1 = radix_pass(key, n, d0 << 21, 0x7FFu << 21, 10, 0x7FFu, kr, S, par, &above);
  kr -= above;
  const uint32_t pre = (d0 << 21) | (d1 << 10);
  const uint32_t d2 = radix_pass(key, n, pre, 0xFFFFFC00u, 0, 0x3FFu, kr, S, par, &above);
  const int need_eq = kr - above;
  const uint32_t T = pre | d2;
  const bool all_eq = need_eq == S.hist[d2];  // every key equal to T is taken: no ranks needed

  int tot;
  uint32_t take = 0;  // bit u: key[u] is selected
  if (all_eq) {
#pragma unroll
    for (int u = 0; u < kKPT; ++u) take |= (uint32_t)(u * kTkThreads + tid < n && key[u] >= T) << u;
  } else {
    // ranks of the keys equal to T, in position order (row-major over (u, wave, lane))
#pragma unroll
    for (int u = 0; u < kKPT; ++u) {
      const uint64_t me = __ballot(u * kTkThreads + tid < n && key[u] == T);
      if (lane == 0) S.cnt[u * kTkWaves + w] = __popcll(me);
    }
    __syncthreads();
    {
      const int c = tid < kKPT * kTkWaves ? S.cnt[tid] : 0;
      const int off = block_scan<7>(c, &tot, S, par);
      __syncthreads();
      if (tid < kKPT * kTkWaves) S.cnt[tid] = off;
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < kKPT; ++u) {
      const bool ok = u * kTkThreads + tid < n;
      const bool e = ok && key[u] == T;
      const uint64_t me = __ballot(e);
      const bool sel = (ok && key[u] > T) || (e && S.cnt[u * kTkWaves + w] + lanes_below(me) < need_eq);
      take |= (uint32_t)sel << u;
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kKPT; ++u) {
    const uint64_t ms = __ballot((take >> u) & 1);
    if (lane == 0) S.cnt[u * kTkWaves + w] = __popcll(ms);
  }
  __syncthreads();
  {
    const int c = tid < kKPT * kTkWaves ? S.cnt[tid] : 0;
    const int off = block_scan<7>(c, &tot, S, par);
    __syncthreads();
    if (tid < kKPT * kTkWaves) S.cnt[tid] = off;
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < kKPT; ++u) {
    const bool sel = (take >> u) & 1;
    const uint64_t ms = __ballot(sel);
    if (sel) emit(S.cnt[u * kTkWaves + w] + lanes_below(ms), u);
  }
}

// Chunk level: workgroup = (row, chunk of 32768 entries). final_idx !=
// nullptr: the row fits one chunk and the final indices are written;
// otherwise the chunk's list of k (key, index), padded with key 0 / index -1.
__global__ __launch_bounds__(kTkThreads) void topk_chunk_kernel(
    int Lq, int64_t q_pos0, int m, int64_t N_cap, const float* __restrict__ scores, int topk, int nchunks,
    int32_t* __restrict__ final_idx, uint32_t* __restrict__ out_key, int32_t* __restrict__ out_idx) {
  __shared__ TkShared S;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / nchunks;
  const int chunk = (int)(blockIdx.x % nchunks);
  const int i = (int)(row % Lq);
  const int n_row = (int)((q_pos0 + i + 1) / m);
  const int j0 = chunk * kTkKeys;
  const int n = max(0, min(kTkKeys, n_row - j0));
  int32_t* oi = final_idx ? final_idx + row * topk : out_idx + (row * nchunks + chunk) * topk;
  uint32_t* ok = final_idx ? nullptr : out_key + (row * nchunks + chunk) * topk;
  const float* s = scores + row * N_cap + j0;

  if (n <= topk) {  // every entry of the chunk is selected
    for (int p = tid; p < topk; p += kTkThreads) {
      const bool v = p < n;
      const float x = s[v ? p : 0];
      oi[p] = v ? j0 + p : -1;
      if (ok) ok[p] = v ? score_key(x) : 0u;
    }
    return;
  }
  uint32_t key[kKPT];
#pragma unroll
  for (int u = 0; u < kKPT; ++u) key[u] = score_key(s[min(u * kTkThreads + tid, n - 1)]);
  block_select(key, n, topk, S, [&](int slot, int u) {
    oi[slot] = j0 + u * kTkThreads + tid;
    if (ok) ok[slot] = key[u];
  });
}

// Merge level: workgroup = (row, group of G consecutive lists of k). The
// last level writes the final indices.
__global__ __launch_bounds__(kTkThreads) void topk_merge_kernel(
    int topk, int nlists, int G, const uint32_t* __restrict__ in_key, const int32_t* __restrict__ in_idx,
    int32_t* __restrict__ final_idx, uint32_t* __restrict__ out_key, int32_t* __restrict__ out_idx) {
  __shared__ TkShared S;
  const int tid = threadIdx.x;
  const int nout = (nlists + G - 1) / G;
  const int64_t row = blockIdx.x / nout;
  const int grp = (int)(blockIdx.x % nout);
  const int l0 = grp * G;
  const int n = min(G, nlists - l0) * topk;
  const uint32_t* ik = in_key + (row * nlists + l0) * topk;
  const int32_t* ii = in_idx + (row * nlists + l0) * topk;
  int32_t* oi = final_idx ? final_idx + row * topk : out_idx + (row * nout + grp) * topk;
  uint32_t* ok = final_idx ? nullptr : out_key + (row * nout + grp) * topk;
  if (n <= topk) {  // a single list passes through
    for (int p = tid; p < topk; p += kTkThreads) {
      oi[p] = ii[p];
      if (ok) ok[p] = ik[p];
    }
    return;
  }
  uint32_t key[kKPT];
  int32_t idx[kKPT];
#pragma unroll
  for (int u = 0; u < kKPT; ++u) {
    const int p = min(u * kTkThreads + tid, n - 1);
    key[u] = ik[p];
    idx[u] = ii[p];
  }
  block_select(key, n, topk, S, [&](int slot, int u) {
    oi[slot] = idx[u];
    if (ok) ok[slot] = key[u];
  });
}

static int topk_nchunks(int64_t n_max) { return (int)((n_max + kTkKeys - 1) / kTkKeys); }

// Lists merged per workgroup at each level: as many as fit in 32768 keys.
static int topk_group(int topk) { return max(2, kTkKeys / topk); }

size_t topk_ws_bytes(int B, int Lq, int64_t n_max, int topk) {
  const int nc = topk_nchunks(n_max);
  if (nc <= 1) return 0;
  const int G = topk_group(topk);
  const size_t rows = (size_t)B * Lq;
  const size_t lvl0 = rows * nc * topk * 8;
  const size_t lvl1 = rows * ((nc + G - 1) / G) * topk * 8;
  return lvl0 + lvl1;
}

int launch_topk(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, const float* scores, int topk,
                int32_t* idx_out, void* ws, hipStream_t stream) {
  const int64_t rows = (int64_t)B * Lq;
  if (rows == 0) return 0;
  const int64_t n_max = (q_pos0 + Lq) / m;
  const int nc = max(1, topk_nchunks(n_max));
  const dim3 block(kTkThreads);
  if (nc == 1) {
    hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)rows), block, 0, stream, Lq, q_pos0, m, N_cap, scores,
                       topk, 1, idx_out, (uint32_t*)nullptr, (int32_t*)nullptr);
    return hipGetLastError() == hipSuccess ? 0 : 1;
  }
  const int G = topk_group(topk);
  // two ping-pong regions: level 0 (nc lists per row) and level 1 (ceil(nc/G))
  const int nc1 = (nc + G - 1) / G;
  uint32_t* k0 = (uint32_t*)ws;
  int32_t* i0 = (int32_t*)(k0 + rows * nc * topk);
  uint32_t* k1 = (uint32_t*)(i0 + rows * nc * topk);
  int32_t* i1 = (int32_t*)(k1 + rows * nc1 * topk);
  hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)(rows * nc)), block, 0, stream, Lq, q_pos0, m, N_cap,
                     scores, topk, nc, (int32_t*)nullptr, k0, i0);
  int nlists = nc;
  bool in0 = true;
  while (nlists > 1) {
    const int nout = (nlists + G - 1) / G;
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)(rows * nout)), block, 0, stream, topk, nlists, G,
                       in0 ? k0 : k1, in0 ? i0 : i1, nout == 1 ? idx_out : (int32_t*)nullptr, in0 ? k1 : k0,
                       in0 ? i1 : i0);
    nlists = nout;
    in0 = !in0;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
