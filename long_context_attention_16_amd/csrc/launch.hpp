// Host-side launchers of the kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace csa {

// Arguments of the attention kernels (CSA gathered rows and HCA dense rows).
struct AttnArgs {
  int B, Lq;
  int64_t q_pos0;    // position of query row 0, or the bound of q_pos
  const int64_t* q_pos;  // per-sequence positions of query row 0 [B], or nullptr
  int m;             // HCA block (visible entries n(t) = (t+1)/m)
  int H, D;
  const void* q;
  int64_t N_cap;
  const void* k_c;
  const void* v_c;
  int topk;          // CSA only
  const int32_t* idx;
  int T_raw;
  int64_t raw_pos0;
  int ring;          // raw rows are a ring of T_raw slots (position s in slot s % T_raw)
  const void* k_raw;
  const void* v_raw;
  int W;
  const float* sink;
  void* out;
  float* lse;
  void* ws_o;        // split partials [B*Lq][nsplit_max][H][D], KV dtype (bf16 or f32)
  float* ws_ml;      // split (max, sum) [B*Lq][nsplit_max][H][2]
  int nsplit_max;
};

// Row of absolute position s within a sequence's raw rows (one division per
// query, for the first window position)...
__device__ __forceinline__ int64_t attn_raw_row(const AttnArgs& p, int64_t s) {
  return p.ring ? s % p.T_raw : s - p.raw_pos0;
}
// ... and of window row w, from that first row: a window never exceeds the
// ring, so it wraps at most once.
__device__ __forceinline__ int64_t attn_window_row(const AttnArgs& p, int64_t row_lo, int w) {
  const int64_t r = row_lo + w;
  return p.ring && r >= p.T_raw ? r - p.T_raw : r;
}

// Rows per split of a query with S sources: S/16 rounded up to a multiple of
// 32 (long lists: many splits per query keep every CU busy at decode sizes),
// at least 96 (three 32-row tiles, so each workgroup pipelines loads with
// compute); for lists of at most 4096 sources at least half the list, up to
// 576 rows (18 tiles): a split's fixed costs (the idx lookup before its first
// copies, the partial write, its share of the combine) then stay small next
// to its stream. A function of S alone, so the split structure never depends
// on the batch.
__host__ __device__ inline int attn_split_rows(int S) {
  int ch = ((S + 15) / 16 + 31) / 32 * 32;
  if (S <= 4096) {
    int half = ((S + 1) / 2 + 31) / 32 * 32;
    half = half < 576 ? half : 576;
    ch = ch > half ? ch : half;
  }
  return ch < 96 ? 96 : ch;
}
__host__ __device__ inline int attn_nsplit(int S) {
  const int ch = attn_split_rows(S);
  const int ns = (S + ch - 1) / ch;
  return ns < 1 ? 1 : ns;
}

// d_i > 0: also fold the raw indexer keys ki_raw [B, T, d_i] (KV dtype) into
// ki_c [B, N_cap, d_i] in idx_fmt (+ e8m0 scales for MXFP4).
int launch_compress(int B, int T, int D, int m, int64_t pos0, int kv_dtype, const void* k_raw,
                    const void* v_raw, const float* w_gate, void* k_c, void* v_c, int64_t N_cap, int d_i,
                    int idx_fmt, const void* ki_raw, void* ki_c, uint8_t* ki_c_scale, hipStream_t stream);
// One decode step of the state cache (ring append + completed-block compression).
int launch_state_append(int B, int D, int m, int R, int kv_dtype, const int64_t* pos, const void* k_new,
                        const void* v_new, const float* w_gate, void* k_ring, void* v_ring, void* k_c, void* v_c,
                        int64_t N_cap, int d_i, int idx_fmt, const void* ki_new, void* ki_ring, void* ki_c,
                        uint8_t* ki_c_scale, hipStream_t stream);
// Query rows scored together by one indexer workgroup (64 / H_i, 1 for H_i = 128).
int index_qk_queries_per_group(int H_i);
// Chunks of entries per row scored by the indexer workgroups when scores go
// to HBM (2048 entries each).
int index_qk_nchunks(int64_t q_pos0, int Lq, int m);
// Fused indexer + chunk top-k: entries per chunk for top-k k (at least 4k:
// 2048 for k <= 512, 4096 for k <= 1024; 0 = k too large to fuse) and the
// chunks (candidate lists) per row.
int index_fused_cols(int topk);
int index_fused_nchunks(int64_t q_pos0, int Lq, int m, int topk);
// Many-query fp8 indexer (64 heads of dim 128, at least 16 query rows per
// sequence): same scores as launch_index_qk.
bool index_qk_prefill_eligible(int fmt, int H_i, int d_i, int Lq);
int launch_index_qk_prefill(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int64_t N_cap,
                            const void* q_i, const float* w_i, const void* k_i, float* scores, int sbf,
                            hipStream_t stream);
// sbf != 0: scores in bfloat16 (rows of score_stride(N_cap, 1) entries) and
// the top-k ordered by the rounded scores.
// Indexer with the per-chunk top-k fused in (groups of one query only): for
// each (row, chunk) a list of topk (key, index) pairs at
// cand_{key,idx}[(row * nchunks + chunk) * topk].
int launch_index_qk_fused(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int64_t N_cap, int H_i,
                          int d_i, int fmt,
                          const void* q_i, const uint8_t* q_s, const float* w_i, const void* k_i,
                          const uint8_t* k_s, int topk, int sbf, uint32_t* cand_key, int32_t* cand_idx,
                          hipStream_t stream);
// Merge levels over nlists candidate lists of topk per row (rows = B * Lq),
// then the final indices; ws holds the lists at level 0 and room for level 1.
int launch_topk_merge(int64_t rows, int nlists, int topk, void* lists, int32_t* idx_out, hipStream_t stream);
size_t topk_merge_ws_bytes(int64_t rows, int nlists, int topk);
// CSA attention in two launches for one bf16 KV head of dim 512 and H a
// multiple of 16 (attn_decode.hip); ws holds the bf16 P' rows and the chunk
// statistics, attn_decode_ws bytes.
bool attn_decode_eligible(int kv_dtype, bool hca, int H, int D, int topk, int W);
size_t attn_decode_ws(int B, int Lq, int H, int topk, int W);
int launch_attn_decode(const AttnArgs& a, void* ws, hipStream_t st);
int launch_index_qk(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int64_t N_cap, int H_i,
                    int d_i, int fmt,
                    const void* q_i, const uint8_t* q_s, const float* w_i, const void* k_i,
                    const uint8_t* k_s, float* scores, int sbf, hipStream_t stream);
size_t topk_ws_bytes(int B, int Lq, int64_t n_max, int topk);
int launch_topk(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int64_t N_cap, const float* scores,
                int sbf, int topk, int32_t* idx_out, void* ws, hipStream_t stream);
int launch_attn(const AttnArgs& a, int kv_dtype, bool hca, hipStream_t stream);
// Attention backward (attn_bwd.hip). S = source slots per query row (topk +
// W for CSA, n(t_last) + W for HCA); ws holds the per-slot weights, the
// rotated q, the sink parts and the inverse index (attn_bwd_ws_bytes).
size_t attn_bwd_ws_bytes(int B, int Lq, int H, int D, int64_t N_cap, int S, int topk);
int launch_attn_bwd(const AttnArgs& a, bool hca, int S, int kv_dtype, const void* dout, float* dq, float* dk_c,
                    float* dv_c, float* dk_raw, float* dv_raw, float* dsink, void* ws, hipStream_t st);

}  // namespace csa
