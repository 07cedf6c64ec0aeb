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
// thread (key[u] of thread t is position 1024u + t, so every load is
// coalesced), with the radix select of select.hpp.
// Rows longer than 32768 entries are cut into chunks; each chunk's top k
// (every global top-k entry is in its chunk's top k) forms a candidate list in
// ascending index order, and merge levels take the top k of groups of
// consecutive lists (list position order is index order, so ties still go to
// the lower index) until one list remains.
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace csa {

constexpr int kTkThreads = 1024;
constexpr int kKPT = 32;                       // keys per thread
constexpr int kTkKeys = kTkThreads * kKPT;     // 32768

// Chunk level: workgroup = (row, chunk of 32768 entries). final_idx !=
// nullptr: the row fits one chunk and the final indices are written;
// otherwise the chunk's list of k (key, index), padded with key 0 / index -1.
// SBF: bf16 scores in rows of score_stride(N_cap, 1) entries, selected on
// 16-bit keys (score_key_bf16 >> 16). THREADS: the workgroup's width (1024
// for few rows; narrower ones, with 32 keys per thread, put more rows in
// flight per CU when there are many: the selection is a latency chain).
template <int THREADS, int KPT, bool SBF>
__global__ __launch_bounds__(THREADS) void topk_chunk_kernel(
    int Lq, int64_t q_pos0, const int64_t* __restrict__ q_pos, int m, int64_t N_cap,
    const float* __restrict__ scores, int topk, int nchunks,
    int32_t* __restrict__ final_idx, uint32_t* __restrict__ out_key, int32_t* __restrict__ out_idx) {
  __shared__ TopkShared<THREADS, KPT> S;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / nchunks;
  const int chunk = (int)(blockIdx.x % nchunks);
  const int i = (int)(row % Lq);
  const int n_row = (int)((seq_pos(q_pos, q_pos0, (int)(row / Lq)) + i + 1) / m);
  const int j0 = chunk * kTkKeys;
  const int n = max(0, min(kTkKeys, n_row - j0));
  int32_t* oi = final_idx ? final_idx + row * topk : out_idx + (row * nchunks + chunk) * topk;
  uint32_t* ok = final_idx ? nullptr : out_key + (row * nchunks + chunk) * topk;
  const float* s = scores + row * N_cap + j0;
  const uint16_t* s16 = reinterpret_cast<const uint16_t*>(scores) + row * score_stride(N_cap, 1) + j0;
  auto keyat = [&](int p) { return SBF ? score_key_bf16(bf16_bits_to_f32(s16[p])) : score_key(s[p]); };
  constexpr int ksh = SBF ? 16 : 0;

  if (n <= topk) {  // every entry of the chunk is selected
    for (int p = tid; p < topk; p += THREADS) {
      const bool v = p < n;
      const uint32_t x = keyat(v ? p : 0);
      oi[p] = v ? j0 + p : -1;
      if (ok) ok[p] = v ? x : 0u;
    }
    return;
  }
  uint32_t key[KPT];
  if constexpr (SBF) {
    uint16_t v[KPT];
    load_run<KPT>(s16, tid * KPT, n, v);
#pragma unroll
    for (int u = 0; u < KPT; ++u) key[u] = score_key_bf16(bf16_bits_to_f32(v[u])) >> 16;
  } else {
    float v[KPT];
    load_run<KPT>(s, tid * KPT, n, v);
#pragma unroll
    for (int u = 0; u < KPT; ++u) key[u] = score_key(v[u]);
  }
  block_select<THREADS, KPT>(key, n, topk, S, [&](int slot, int u) {
    S.hist[slot] = j0 + tid * KPT + u;
    S.stage[slot] = key[u] << ksh;
  });
  block_select_out(S, topk, oi, ok);
}

// Merge level: workgroup = (row, group of G consecutive lists of k). The
// last level writes the final indices.
template <int KPT>
__global__ __launch_bounds__(kTkThreads) void topk_merge_kernel(
    int topk, int nlists, int G, const uint32_t* __restrict__ in_key, const int32_t* __restrict__ in_idx,
    int32_t* __restrict__ final_idx, uint32_t* __restrict__ out_key, int32_t* __restrict__ out_idx) {
  __shared__ TopkShared<kTkThreads, KPT> S;
  const int nout = (nlists + G - 1) / G;
  const int64_t row = blockIdx.x / nout;
  const int grp = (int)(blockIdx.x % nout);
  const int l0 = grp * G;
  const int n = min(G, nlists - l0) * topk;
  int32_t* oi = final_idx ? final_idx + row * topk : out_idx + (row * nout + grp) * topk;
  uint32_t* ok = final_idx ? nullptr : out_key + (row * nout + grp) * topk;
  merge_lists<kTkThreads, KPT>(S, n, topk, in_key + (row * nlists + l0) * topk, in_idx + (row * nlists + l0) * topk,
                               oi, ok);
}

// Keys per thread of a 1024-thread selection over up to n keys: the work of
// every phase scales with it, so it follows the list length.
static int kpt_for(int64_t n) { return n <= 4096 ? 4 : n <= 8192 ? 8 : n <= 16384 ? 16 : 32; }

#define CSA_TOPK_KPT(kpt, KERNEL, ...)                                                               \
  switch (kpt) {                                                                                    \
    case 4: hipLaunchKernelGGL(KERNEL<4>, __VA_ARGS__); break;                                      \
    case 8: hipLaunchKernelGGL(KERNEL<8>, __VA_ARGS__); break;                                      \
    case 16: hipLaunchKernelGGL(KERNEL<16>, __VA_ARGS__); break;                                    \
    default: hipLaunchKernelGGL(KERNEL<32>, __VA_ARGS__); break;                                    \
  }

static int topk_nchunks(int64_t n_max) { return (int)((n_max + kTkKeys - 1) / kTkKeys); }

// Lists merged per workgroup at each level: as many as fit in 8192 keys (at
// least two). A workgroup's select time grows with its keys, so many small
// merges in parallel beat a few large ones: k = 1024 over 64 lists takes two
// levels of 8192-key merges rather than 32768-key ones. The grouping cannot
// change the result: every group keeps its own top k, and (-score, j) is a
// total order, so the final level selects the row's exact top k.
static int topk_group(int topk) { return max(2, 8192 / topk); }

size_t topk_merge_ws_bytes(int64_t rows, int nlists, int topk) {
  if (nlists <= 1) return (size_t)rows * nlists * topk * 8;
  const int G = topk_group(topk);
  return (size_t)rows * topk * 8 * ((size_t)nlists + (nlists + G - 1) / G);
}

// idx[i] = -1 for i < n: the output of rows that see no entry yet (a fill
// kernel rather than a memset, so a captured graph replays it as it is).
__global__ __launch_bounds__(256) void fill_pad_kernel(int32_t* __restrict__ idx, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) idx[i] = -1;
}

int launch_topk_merge(int64_t rows, int nlists, int topk, void* lists, int32_t* idx_out, hipStream_t stream) {
  if (rows == 0) return 0;
  if (nlists == 0) {  // no row has a visible entry: every slot is padding
    const int64_t n = rows * topk;
    const int nb = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    hipLaunchKernelGGL(fill_pad_kernel, dim3(nb), dim3(256), 0, stream, idx_out, n);
    return hipGetLastError() == hipSuccess ? 0 : 1;
  }
  const int G = topk_group(topk);
  // two ping-pong regions: level 0 (nlists lists per row) and level 1 (ceil(nlists/G))
  const int n1 = (nlists + G - 1) / G;
  uint32_t* k0 = (uint32_t*)lists;
  int32_t* i0 = (int32_t*)(k0 + rows * nlists * topk);
  uint32_t* k1 = (uint32_t*)(i0 + rows * nlists * topk);
  int32_t* i1 = (int32_t*)(k1 + rows * n1 * topk);
  int n = nlists;
  bool in0 = true;
  do {
    const int nout = (n + G - 1) / G;
    CSA_TOPK_KPT(kpt_for((int64_t)min(n, G) * topk), topk_merge_kernel, dim3((unsigned)(rows * nout)),
                 dim3(kTkThreads), 0, stream, topk, n, G, in0 ? k0 : k1, in0 ? i0 : i1,
                 nout == 1 ? idx_out : (int32_t*)nullptr, in0 ? k1 : k0, in0 ? i1 : i0);
    n = nout;
    in0 = !in0;
  } while (n > 1);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

size_t topk_ws_bytes(int B, int Lq, int64_t n_max, int topk) {
  const int nc = topk_nchunks(n_max);
  if (nc <= 1) return 0;
  return topk_merge_ws_bytes((int64_t)B * Lq, nc, topk);
}

int launch_topk(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int64_t N_cap, const float* scores,
                int sbf, int topk, int32_t* idx_out, void* ws, hipStream_t stream) {
  const int64_t rows = (int64_t)B * Lq;
  if (rows == 0) return 0;
  const int64_t n_max = (q_pos0 + Lq) / m;
  const int nc = max(1, topk_nchunks(n_max));
  const dim3 block(kTkThreads);
  // Rows of one chunk: with many rows (at least four workgroups per CU) a
  // row takes the narrowest workgroup that holds it at 32 keys per thread.
  const bool narrow = rows >= 1024 && n_max <= 16384;
#define CSA_TOPK_CHUNK(SB, ...)                                                                          \
  if (narrow && n_max <= 8192) hipLaunchKernelGGL((topk_chunk_kernel<256, 32, SB>), dim3((unsigned)rows), \
                                                  dim3(256), __VA_ARGS__);                              \
  else if (narrow) hipLaunchKernelGGL((topk_chunk_kernel<512, 32, SB>), dim3((unsigned)rows), dim3(512),  \
                                      __VA_ARGS__);                                                     \
  else switch (kpt_for(n_max)) {                                                                        \
    case 4: hipLaunchKernelGGL((topk_chunk_kernel<kTkThreads, 4, SB>), dim3((unsigned)rows), block,       \
                               __VA_ARGS__); break;                                                     \
    case 8: hipLaunchKernelGGL((topk_chunk_kernel<kTkThreads, 8, SB>), dim3((unsigned)rows), block,       \
                               __VA_ARGS__); break;                                                     \
    case 16: hipLaunchKernelGGL((topk_chunk_kernel<kTkThreads, 16, SB>), dim3((unsigned)rows), block,     \
                                __VA_ARGS__); break;                                                    \
    default: hipLaunchKernelGGL((topk_chunk_kernel<kTkThreads, 32, SB>), dim3((unsigned)rows), block,     \
                                __VA_ARGS__); break;                                                    \
  }
  if (nc == 1) {
    if (sbf) {
      CSA_TOPK_CHUNK(true, 0, stream, Lq, q_pos0, q_pos, m, N_cap, scores, topk, 1, idx_out, (uint32_t*)nullptr,
                     (int32_t*)nullptr)
    } else {
      CSA_TOPK_CHUNK(false, 0, stream, Lq, q_pos0, q_pos, m, N_cap, scores, topk, 1, idx_out, (uint32_t*)nullptr,
                     (int32_t*)nullptr)
    }
    return hipGetLastError() == hipSuccess ? 0 : 1;
  }
#undef CSA_TOPK_CHUNK
  uint32_t* k0 = (uint32_t*)ws;
  int32_t* i0 = (int32_t*)(k0 + rows * nc * topk);
  if (sbf)
    hipLaunchKernelGGL((topk_chunk_kernel<kTkThreads, kKPT, true>), dim3((unsigned)(rows * nc)), block, 0, stream,
                       Lq, q_pos0, q_pos, m, N_cap, scores, topk, nc, (int32_t*)nullptr, k0, i0);
  else
    hipLaunchKernelGGL((topk_chunk_kernel<kTkThreads, kKPT, false>), dim3((unsigned)(rows * nc)), block, 0, stream,
                       Lq, q_pos0, q_pos, m, N_cap, scores, topk, nc, (int32_t*)nullptr, k0, i0);
  if (hipGetLastError() != hipSuccess) return 1;
  return launch_topk_merge(rows, nc, topk, ws, idx_out, stream);
}

}  // namespace csa
