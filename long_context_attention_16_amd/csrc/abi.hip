// C ABI of the library: argument checks on the host, then the launches.
// Every check runs before anything is enqueued, allocates nothing and costs
// well under a microsecond.
#include "../../include/csa.h"
#include "launch.hpp"

#include <mutex>

using namespace csa;

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool kv_ok(int dt) { return dt == CSA_F32 || dt == CSA_BF16; }
inline bool head_dim_ok(int D) { return D == 128 || D == 512; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Visible compressed entries of the last query row.
inline int64_t n_last(int64_t q_pos0, int Lq, int m) { return (q_pos0 + Lq) / m; }

int check_window(int Lq, int64_t q_pos0, int W, int T_raw, int64_t raw_pos0, bool ring) {
  if (W < 0 || W > 1024 || T_raw < 0) return CSA_ERR_SHAPE;
  if (W == 0) return CSA_OK;
  // a ring holds every query's window: W + Lq - 1 distinct positions
  if (ring) return (int64_t)W + Lq - 1 <= T_raw ? CSA_OK : CSA_ERR_SHAPE;
  const int64_t lo = q_pos0 - W + 1 > 0 ? q_pos0 - W + 1 : 0;
  if (raw_pos0 < 0 || raw_pos0 > lo) return CSA_ERR_SHAPE;
  if (q_pos0 + Lq - 1 >= raw_pos0 + T_raw) return CSA_ERR_SHAPE;
  return CSA_OK;
}

int attn_nsplit_max_csa(int topk, int W) { return attn_nsplit(topk + W); }
// HCA rows of one call have different source counts (n(t) grows with t, and
// per-sequence positions vary). The longest row's split count bounds every
// row's only while the count is monotonic in the source count, which holds
// up to 4096 sources; beyond, rounding the split size up to whole tiles makes
// it dip (4608 sources: 16 splits of 288 rows; 4609: 15 of 320), so the grid
// and the partials are sized for the maximum, 16 (a split holds at least
// S/16 rows).
int attn_nsplit_max_hca(int64_t q_pos0, int Lq, int m, int W) {
  const int S = (int)n_last(q_pos0, Lq, m) + W;
  return S > 4096 ? 16 : attn_nsplit(S);
}
// Split partials: O in the KV dtype, then (max, sum) in f32.
size_t attn_ws(int B, int Lq, int H, int D, int nsplit, int kv_bytes) {
  if (nsplit <= 1) return 16;
  const size_t slots = (size_t)B * Lq * nsplit * H;
  return (slots * D * kv_bytes + 15) / 16 * 16 + slots * 2 * 4;
}

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_strerror(int code) {
  switch (code) {
    case CSA_OK: return "ok";
    case CSA_ERR_NULL: return "a required pointer is NULL";
    case CSA_ERR_SHAPE: return "a size or position is outside the supported range";
    case CSA_ERR_DTYPE: return "dtype not supported by this entry point";
    case CSA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int csa_compress(int B, int T, int D, int m, int64_t pos0, int kv_dtype, const void* k_raw,
                 const void* v_raw, const float* w_gate, void* k_c, void* v_c, int64_t N_cap, int d_i,
                 int idx_dtype, const void* ki_raw, void* ki_c, uint8_t* ki_c_scale, void* stream) {
  if (!k_raw || !v_raw || !w_gate || !k_c || !v_c) return CSA_ERR_NULL;
  if (d_i > 0 && (!ki_raw || !ki_c)) return CSA_ERR_NULL;
  if (d_i > 0 && idx_dtype == CSA_FP4_E2M1 && !ki_c_scale) return CSA_ERR_NULL;
  if (!kv_ok(kv_dtype)) return CSA_ERR_DTYPE;
  if (d_i > 0 && (idx_dtype < CSA_F32 || idx_dtype > CSA_FP4_E2M1)) return CSA_ERR_DTYPE;
  if (B < 0 || T < 0 || !head_dim_ok(D) || m < 1 || m > 4096 || pos0 < 0 || pos0 % m != 0 || N_cap < 0)
    return CSA_ERR_SHAPE;
  if (!(d_i == 0 || d_i == 32 || d_i == 64 || d_i == 128)) return CSA_ERR_SHAPE;
  if (pos0 / m + T / m > N_cap) return CSA_ERR_SHAPE;
  if (!aligned16(k_raw) || !aligned16(v_raw) || !aligned16(w_gate) || !aligned16(k_c) || !aligned16(v_c) ||
      (d_i > 0 && (!aligned16(ki_raw) || !aligned16(ki_c))))
    return CSA_ERR_ALIGN;
  return launch_compress(B, T, D, m, pos0, kv_dtype, k_raw, v_raw, w_gate, k_c, v_c, N_cap, d_i, idx_dtype,
                         ki_raw, ki_c, ki_c_scale, as_stream(stream)) ? CSA_ERR_LAUNCH : CSA_OK;
}

size_t csa_topk_ws_bytes(int B, int Lq, int64_t q_pos0, int m, int topk) {
  if (B <= 0 || Lq <= 0 || m < 1 || q_pos0 < 0 || topk < 1) return 16;
  const size_t b = topk_ws_bytes(B, Lq, n_last(q_pos0, Lq, m), topk);
  return b < 16 ? 16 : b;
}

static size_t scores_bytes(int B, int Lq, int64_t N_cap) {
  return ((size_t)B * Lq * N_cap * sizeof(float) + 255) / 256 * 256;
}

int csa_state_append(int B, int D, int m, int R, int kv_dtype, const int64_t* pos, const void* k_new,
                     const void* v_new, const float* w_gate, void* k_ring, void* v_ring, void* k_c, void* v_c,
                     int64_t N_cap, int d_i, int idx_dtype, const void* ki_new, void* ki_ring, void* ki_c,
                     uint8_t* ki_c_scale, void* stream) {
  if (!pos || !k_new || !v_new || !w_gate || !k_ring || !v_ring || !k_c || !v_c) return CSA_ERR_NULL;
  if (d_i > 0 && (!ki_new || !ki_ring || !ki_c)) return CSA_ERR_NULL;
  if (d_i > 0 && idx_dtype == CSA_FP4_E2M1 && !ki_c_scale) return CSA_ERR_NULL;
  if (!kv_ok(kv_dtype)) return CSA_ERR_DTYPE;
  if (d_i > 0 && (idx_dtype < CSA_F32 || idx_dtype > CSA_FP4_E2M1)) return CSA_ERR_DTYPE;
  if (B < 0 || !head_dim_ok(D) || m < 1 || m > 4096 || R < m || R > (1 << 24) || N_cap < 1) return CSA_ERR_SHAPE;
  if (!(d_i == 0 || d_i == 32 || d_i == 64 || d_i == 128)) return CSA_ERR_SHAPE;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(w_gate) || !aligned16(k_ring) || !aligned16(v_ring) ||
      !aligned16(k_c) || !aligned16(v_c) || ((uintptr_t)pos & 7u) ||
      (d_i > 0 && (!aligned16(ki_new) || !aligned16(ki_ring) || !aligned16(ki_c))))
    return CSA_ERR_ALIGN;
  return launch_state_append(B, D, m, R, kv_dtype, pos, k_new, v_new, w_gate, k_ring, v_ring, k_c, v_c, N_cap,
                             d_i, idx_dtype, ki_new, ki_ring, ki_c, ki_c_scale, as_stream(stream))
             ? CSA_ERR_LAUNCH : CSA_OK;
}

// Fused indexer + per-chunk top-k: candidate lists of the chunks of
// index_fused_cols(k) entries, merged by the top-k merge levels.
static size_t fused_bytes(int B, int Lq, int64_t q_pos0, int m, int topk) {
  return topk_merge_ws_bytes((int64_t)B * Lq, index_fused_nchunks(q_pos0, Lq, m, topk), topk);
}

// The indexer's top-k runs fused when every indexer workgroup scores one query
// (H_i >= 64, or a single query row) and k <= 1024 (a chunk of at least 4k
// entries).
static bool use_fused(int Lq, int H_i, int topk) {
  return (index_qk_queries_per_group(H_i) == 1 || Lq == 1) && index_fused_cols(topk) > 0;
}

static int launch_candidates(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int64_t N_cap, int H_i,
                             int d_i, int idx_dtype, const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                             const void* k_i, const uint8_t* k_i_scale, int topk, int sbf, void* cand,
                             hipStream_t st) {
  const int64_t rows = (int64_t)B * Lq;
  uint32_t* ck = (uint32_t*)cand;
  int32_t* ci = (int32_t*)(ck + rows * index_fused_nchunks(q_pos0, Lq, m, topk) * topk);
  return launch_index_qk_fused(B, Lq, q_pos0, q_pos, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i,
                               k_i_scale, topk, sbf, ck, ci, st);
}

size_t csa_index_topk_ws_bytes(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, int topk) {
  if (B <= 0 || Lq <= 0 || N_cap <= 0) return 16;
  const size_t unfused = scores_bytes(B, Lq, N_cap) + csa_topk_ws_bytes(B, Lq, q_pos0, m, topk);
  const size_t fused = fused_bytes(B, Lq, q_pos0, m, topk);
  return unfused > fused ? unfused : fused;
}

static int check_topk_shape(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, int topk) {
  if (B < 0 || Lq < 0 || q_pos0 < 0 || m < 1 || N_cap < 1 || topk < 1 || topk > 2048) return CSA_ERR_SHAPE;
  if (n_last(q_pos0, Lq, m) > N_cap) return CSA_ERR_SHAPE;
  if (N_cap > (int64_t)1 << 30) return CSA_ERR_SHAPE;
  return CSA_OK;
}

static int check_indexer(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, int H_i, int d_i,
                         int idx_dtype, const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                         const void* k_i, const uint8_t* k_i_scale, int topk) {
  if (!q_i || !w_i || !k_i) return CSA_ERR_NULL;
  if (idx_dtype < CSA_F32 || idx_dtype > CSA_FP4_E2M1) return CSA_ERR_DTYPE;
  if (idx_dtype == CSA_FP4_E2M1 && (!q_i_scale || !k_i_scale)) return CSA_ERR_NULL;
  if (int rc = check_topk_shape(B, Lq, q_pos0, m, N_cap, topk)) return rc;
  if (!(H_i == 4 || H_i == 8 || H_i == 16 || H_i == 32 || H_i == 64 || H_i == 128)) return CSA_ERR_SHAPE;
  if (!(d_i == 32 || d_i == 64 || d_i == 128)) return CSA_ERR_SHAPE;
  if ((int64_t)index_qk_queries_per_group(H_i) * N_cap * 4 >= 0x7FFFFFF0LL) return CSA_ERR_SHAPE;
  if (!aligned16(q_i) || !aligned16(w_i) || !aligned16(k_i)) return CSA_ERR_ALIGN;
  return CSA_OK;
}

int csa_index_scores(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, int H_i, int d_i,
                     int idx_dtype, const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                     const void* k_i, const uint8_t* k_i_scale, float* scores, void* stream) {
  if (!scores) return CSA_ERR_NULL;
  if (int rc = check_indexer(B, Lq, q_pos0, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i,
                             k_i_scale, 1))
    return rc;
  if (!aligned16(scores)) return CSA_ERR_ALIGN;
  return launch_index_qk(B, Lq, q_pos0, nullptr, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i,
                         k_i_scale, scores, 0, as_stream(stream)) ? CSA_ERR_LAUNCH : CSA_OK;
}

int csa_index_scores_ex(int B, int Lq, const int64_t* q_pos, int64_t q_pos0, int m, int64_t N_cap, int H_i,
                        int d_i, int idx_dtype, const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                        const void* k_i, const uint8_t* k_i_scale, int score_dtype, void* scores, void* stream) {
  if (!scores) return CSA_ERR_NULL;
  if (score_dtype != CSA_F32 && score_dtype != CSA_BF16) return CSA_ERR_DTYPE;
  if (int rc = check_indexer(B, Lq, q_pos0, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i,
                             k_i_scale, 1))
    return rc;
  if (!aligned16(scores)) return CSA_ERR_ALIGN;
  return launch_index_qk(B, Lq, q_pos0, q_pos, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i,
                         k_i_scale, (float*)scores, score_dtype == CSA_BF16, as_stream(stream))
             ? CSA_ERR_LAUNCH : CSA_OK;
}

// csa_index_topk, csa_index_topk_varlen and csa_index_topk_ex: q_pos ==
// nullptr means every sequence's row 0 is at q_pos0; otherwise q_pos0 bounds
// the q_pos values. sbf: scores rounded to bf16 before the top-k.
static int index_topk(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int64_t N_cap, int H_i,
                      int d_i, int idx_dtype, const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                      const void* k_i, const uint8_t* k_i_scale, int topk, int sbf, int32_t* idx_out, void* ws,
                      size_t ws_bytes, void* stream) {
  if (!idx_out) return CSA_ERR_NULL;
  if (int rc = check_indexer(B, Lq, q_pos0, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i,
                             k_i_scale, topk))
    return rc;
  if (!aligned16(idx_out) || !aligned16(ws)) return CSA_ERR_ALIGN;
  if (!ws || ws_bytes < csa_index_topk_ws_bytes(B, Lq, q_pos0, m, N_cap, topk)) return CSA_ERR_WORKSPACE;
  if ((int64_t)B * Lq == 0) return CSA_OK;
  hipStream_t st = as_stream(stream);
  if (use_fused(Lq, H_i, topk)) {
    if (launch_candidates(B, Lq, q_pos0, q_pos, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i,
                          k_i_scale, topk, sbf, ws, st))
      return CSA_ERR_LAUNCH;
    return launch_topk_merge((int64_t)B * Lq, index_fused_nchunks(q_pos0, Lq, m, topk), topk, ws, idx_out, st)
               ? CSA_ERR_LAUNCH : CSA_OK;
  }
  float* scores = (float*)ws;
  void* cand = (char*)ws + scores_bytes(B, Lq, N_cap);
  if (launch_index_qk(B, Lq, q_pos0, q_pos, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i,
                      k_i_scale, scores, sbf, st))
    return CSA_ERR_LAUNCH;
  return launch_topk(B, Lq, q_pos0, q_pos, m, N_cap, scores, sbf, topk, idx_out, cand, st) ? CSA_ERR_LAUNCH
                                                                                          : CSA_OK;
}

int csa_index_topk(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, int H_i, int d_i,
                   int idx_dtype, const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                   const void* k_i, const uint8_t* k_i_scale, int topk, int32_t* idx_out, void* ws,
                   size_t ws_bytes, void* stream) {
  return index_topk(B, Lq, q_pos0, nullptr, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i, k_i_scale,
                    topk, 0, idx_out, ws, ws_bytes, stream);
}

int csa_index_topk_varlen(int B, int Lq, const int64_t* q_pos, int64_t q_pos_max, int m, int64_t N_cap,
                          int H_i, int d_i, int idx_dtype, const void* q_i, const uint8_t* q_i_scale,
                          const float* w_i, const void* k_i, const uint8_t* k_i_scale, int topk,
                          int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  if (!q_pos) return CSA_ERR_NULL;
  return index_topk(B, Lq, q_pos_max, q_pos, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i, k_i_scale,
                    topk, 0, idx_out, ws, ws_bytes, stream);
}

int csa_index_topk_ex(int B, int Lq, const int64_t* q_pos, int64_t q_pos0, int m, int64_t N_cap, int H_i, int d_i,
                      int idx_dtype, const void* q_i, const uint8_t* q_i_scale, const float* w_i, const void* k_i,
                      const uint8_t* k_i_scale, int topk, int score_dtype, int32_t* idx_out, void* ws,
                      size_t ws_bytes, void* stream) {
  if (score_dtype != CSA_F32 && score_dtype != CSA_BF16) return CSA_ERR_DTYPE;
  return index_topk(B, Lq, q_pos0, q_pos, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i, k_i_scale,
                    topk, score_dtype == CSA_BF16, idx_out, ws, ws_bytes, stream);
}

int csa_topk(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, const float* scores, int topk,
             int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  if (!scores || !idx_out) return CSA_ERR_NULL;
  if (int rc = check_topk_shape(B, Lq, q_pos0, m, N_cap, topk)) return rc;
  if (!aligned16(scores) || !aligned16(idx_out) || !aligned16(ws)) return CSA_ERR_ALIGN;
  if (!ws || ws_bytes < csa_topk_ws_bytes(B, Lq, q_pos0, m, topk)) return CSA_ERR_WORKSPACE;
  return launch_topk(B, Lq, q_pos0, nullptr, m, N_cap, scores, 0, topk, idx_out, ws, as_stream(stream))
             ? CSA_ERR_LAUNCH : CSA_OK;
}

size_t csa_index_candidates_bytes(int B, int Lq, int64_t q_pos0, int m, int topk) {
  if (B <= 0 || Lq <= 0 || m < 1 || q_pos0 < 0 || topk < 1) return 16;
  const size_t b = fused_bytes(B, Lq, q_pos0, m, topk);
  return b < 16 ? 16 : b;
}

int csa_index_candidates(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, int H_i, int d_i, int idx_dtype,
                         const void* q_i, const uint8_t* q_i_scale, const float* w_i, const void* k_i,
                         const uint8_t* k_i_scale, int topk, void* cand, size_t cand_bytes, void* stream) {
  if (!cand) return CSA_ERR_NULL;
  if (int rc = check_indexer(B, Lq, q_pos0, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i,
                             k_i_scale, topk))
    return rc;
  if (!use_fused(Lq, H_i, topk)) return CSA_ERR_SHAPE;
  if (!aligned16(cand)) return CSA_ERR_ALIGN;
  if (cand_bytes < csa_index_candidates_bytes(B, Lq, q_pos0, m, topk)) return CSA_ERR_WORKSPACE;
  if ((int64_t)B * Lq == 0) return CSA_OK;
  return launch_candidates(B, Lq, q_pos0, nullptr, m, N_cap, H_i, d_i, idx_dtype, q_i, q_i_scale, w_i, k_i,
                           k_i_scale, topk, 0, cand, as_stream(stream)) ? CSA_ERR_LAUNCH : CSA_OK;
}

int csa_topk_merge(int B, int Lq, int64_t q_pos0, int m, int topk, void* cand, size_t cand_bytes,
                   int32_t* idx_out, void* stream) {
  if (!cand || !idx_out) return CSA_ERR_NULL;
  if (B < 0 || Lq < 0 || q_pos0 < 0 || m < 1 || topk < 1 || topk > 2048) return CSA_ERR_SHAPE;
  if (index_fused_cols(topk) == 0) return CSA_ERR_SHAPE;
  if (!aligned16(cand) || !aligned16(idx_out)) return CSA_ERR_ALIGN;
  if (cand_bytes < csa_index_candidates_bytes(B, Lq, q_pos0, m, topk)) return CSA_ERR_WORKSPACE;
  if ((int64_t)B * Lq == 0) return CSA_OK;
  return launch_topk_merge((int64_t)B * Lq, index_fused_nchunks(q_pos0, Lq, m, topk), topk, cand, idx_out,
                           as_stream(stream)) ? CSA_ERR_LAUNCH : CSA_OK;
}

static int check_attn_common(int B, int Lq, int64_t q_pos0, int H, int D, int kv_dtype, const void* q,
                             const void* k_c, const void* v_c, int T_raw, int64_t raw_pos0,
                             const void* k_raw, const void* v_raw, int W, const float* sink,
                             void* out, float* lse, void* ws, int64_t N_cap, bool ring) {
  if (!q || !k_c || !v_c || !out) return CSA_ERR_NULL;
  if (W > 0 && (!k_raw || !v_raw)) return CSA_ERR_NULL;
  if (!kv_ok(kv_dtype)) return CSA_ERR_DTYPE;
  if (B < 0 || Lq < 0 || q_pos0 < 0 || H < 1 || H > 128 || !head_dim_ok(D) || N_cap < 1) return CSA_ERR_SHAPE;
  if (int rc = check_window(Lq, q_pos0, W, T_raw, raw_pos0, ring)) return rc;
  if (!aligned16(q) || !aligned16(k_c) || !aligned16(v_c) || !aligned16(out) || !aligned16(ws) ||
      (W > 0 && (!aligned16(k_raw) || !aligned16(v_raw))))
    return CSA_ERR_ALIGN;
  (void)sink;
  (void)lse;
  return CSA_OK;
}

size_t csa_sparse_attn_ws_bytes(int B, int Lq, int H, int D, int topk, int W) {
  if (B <= 0 || Lq <= 0 || topk < 0 || W < 0) return 16;
  const size_t split = attn_ws(B, Lq, H, D, attn_nsplit_max_csa(topk, W), 4);
  // many-head bf16 shapes run the two-launch kernel (the KV dtype is not an
  // argument here, so such shapes get room for both)
  if (!attn_decode_eligible(CSA_BF16, false, H, D, topk, W)) return split;
  const size_t dec = attn_decode_ws(B, Lq, H, topk, W);
  return split > dec ? split : dec;
}

// csa_sparse_attn and csa_sparse_attn_varlen (q_pos != nullptr: per-sequence
// positions bounded by q_pos0, raw rows in a ring of T_raw slots).
static int sparse_attn(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int H, int D, int kv_dtype,
                       const void* q, int64_t N_cap, const void* k_c, const void* v_c, int topk,
                       const int32_t* idx, int T_raw, int64_t raw_pos0, const void* k_raw, const void* v_raw,
                       int W, const float* sink, void* out, float* lse, void* ws, size_t ws_bytes,
                       void* stream) {
  const bool ring = q_pos != nullptr;
  if (topk > 0 && !idx) return CSA_ERR_NULL;
  if (int rc = check_attn_common(B, Lq, q_pos0, H, D, kv_dtype, q, k_c, v_c, T_raw, raw_pos0, k_raw,
                                 v_raw, W, sink, out, lse, ws, N_cap, ring))
    return rc;
  if (topk < 0 || topk > 2048) return CSA_ERR_SHAPE;
  if (!ws || ws_bytes < csa_sparse_attn_ws_bytes(B, Lq, H, D, topk, W)) return CSA_ERR_WORKSPACE;
  AttnArgs a{};
  a.B = B; a.Lq = Lq; a.q_pos0 = q_pos0; a.q_pos = q_pos; a.m = 1; a.H = H; a.D = D; a.q = q; a.N_cap = N_cap;
  a.k_c = k_c; a.v_c = v_c; a.topk = topk; a.idx = idx; a.T_raw = T_raw; a.raw_pos0 = ring ? 0 : raw_pos0;
  a.ring = ring; a.k_raw = k_raw; a.v_raw = v_raw; a.W = W; a.sink = sink; a.out = out; a.lse = lse;
  if (attn_decode_eligible(kv_dtype, false, H, D, topk, W))
    return launch_attn_decode(a, ws, as_stream(stream)) ? CSA_ERR_LAUNCH : CSA_OK;
  a.nsplit_max = attn_nsplit_max_csa(topk, W);
  const size_t slots = (size_t)B * Lq * a.nsplit_max * H;
  a.ws_o = ws;
  a.ws_ml = (float*)((char*)ws + (slots * D * (kv_dtype == CSA_F32 ? 4 : 2) + 15) / 16 * 16);
  return launch_attn(a, kv_dtype, false, as_stream(stream)) ? CSA_ERR_LAUNCH : CSA_OK;
}

int csa_sparse_attn(int B, int Lq, int64_t q_pos0, int H, int D, int kv_dtype, const void* q,
                    int64_t N_cap, const void* k_c, const void* v_c, int topk, const int32_t* idx,
                    int T_raw, int64_t raw_pos0, const void* k_raw, const void* v_raw, int W,
                    const float* sink, void* out, float* lse, void* ws, size_t ws_bytes,
                    void* stream) {
  return sparse_attn(B, Lq, q_pos0, nullptr, H, D, kv_dtype, q, N_cap, k_c, v_c, topk, idx, T_raw, raw_pos0,
                     k_raw, v_raw, W, sink, out, lse, ws, ws_bytes, stream);
}

int csa_sparse_attn_varlen(int B, int Lq, const int64_t* q_pos, int64_t q_pos_max, int H, int D, int kv_dtype,
                           const void* q, int64_t N_cap, const void* k_c, const void* v_c, int topk,
                           const int32_t* idx, int R, const void* k_ring, const void* v_ring, int W,
                           const float* sink, void* out, float* lse, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!q_pos) return CSA_ERR_NULL;
  return sparse_attn(B, Lq, q_pos_max, q_pos, H, D, kv_dtype, q, N_cap, k_c, v_c, topk, idx, R, 0, k_ring,
                     v_ring, W, sink, out, lse, ws, ws_bytes, stream);
}

}  // extern "C"

// Workspace of csa_sparse_attn_noalloc: one array per GPU, in the code
// object's device memory, alive until the process ends. Host code reaches
// it only through the address hipGetSymbolAddress returns for the current
// device (the array's name in host code is a host-side stand-in, not a device
// address). Nothing in it needs to start at zero (the attention kernels
// write every partial and statistic before reading it).
static __device__ __align__(256) uint8_t scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device

// The current device's scratch address, looked up once per device (with that
// device current) and kept; nullptr if the lookup fails.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}
}  // namespace

extern "C" {

int csa_sparse_attn_noalloc(int B, int Lq, int64_t q_pos0, int H, int D, int kv_dtype, const void* q,
                            int64_t N_cap, const void* k_c, const void* v_c, int topk, const int32_t* idx,
                            int T_raw, int64_t raw_pos0, const void* k_raw, const void* v_raw, int W,
                            const float* sink, void* out, float* lse, void* stream) {
  if (B > 0 && Lq > 0 && topk >= 0 && W >= 0 &&
      csa_sparse_attn_ws_bytes(B, Lq, H, D, topk, W) > (size_t)CSA_NOALLOC_SCRATCH_BYTES)
    return CSA_ERR_WORKSPACE;  // the call needs more than the fixed scratch
  void* ws = scratch_address();
  if (!ws) return CSA_ERR_LAUNCH;
  return sparse_attn(B, Lq, q_pos0, nullptr, H, D, kv_dtype, q, N_cap, k_c, v_c, topk, idx, T_raw, raw_pos0,
                     k_raw, v_raw, W, sink, out, lse, ws, CSA_NOALLOC_SCRATCH_BYTES, stream);
}

size_t hca_dense_attn_ws_bytes(int B, int Lq, int64_t q_pos0, int m, int H, int D, int W) {
  if (B <= 0 || Lq <= 0 || m < 1 || W < 0 || q_pos0 < 0) return 16;
  return attn_ws(B, Lq, H, D, attn_nsplit_max_hca(q_pos0, Lq, m, W), 4);
}

// hca_dense_attn and hca_dense_attn_varlen (as sparse_attn above).
static int dense_attn(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int H, int D, int kv_dtype,
                      const void* q, int64_t N_cap, const void* k_c, const void* v_c, int T_raw,
                      int64_t raw_pos0, const void* k_raw, const void* v_raw, int W, const float* sink,
                      void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  const bool ring = q_pos != nullptr;
  if (int rc = check_attn_common(B, Lq, q_pos0, H, D, kv_dtype, q, k_c, v_c, T_raw, raw_pos0, k_raw,
                                 v_raw, W, sink, out, lse, ws, N_cap, ring))
    return rc;
  if (m < 1 || m > 4096) return CSA_ERR_SHAPE;
  if (n_last(q_pos0, Lq, m) > N_cap || n_last(q_pos0, Lq, m) + W > (int64_t)1 << 30) return CSA_ERR_SHAPE;
  if (!ws || ws_bytes < hca_dense_attn_ws_bytes(B, Lq, q_pos0, m, H, D, W)) return CSA_ERR_WORKSPACE;
  AttnArgs a{};
  a.B = B; a.Lq = Lq; a.q_pos0 = q_pos0; a.q_pos = q_pos; a.m = m; a.H = H; a.D = D; a.q = q; a.N_cap = N_cap;
  a.k_c = k_c; a.v_c = v_c; a.topk = 0; a.idx = nullptr; a.T_raw = T_raw; a.raw_pos0 = ring ? 0 : raw_pos0;
  a.ring = ring; a.k_raw = k_raw; a.v_raw = v_raw; a.W = W; a.sink = sink; a.out = out; a.lse = lse;
  a.nsplit_max = attn_nsplit_max_hca(q_pos0, Lq, m, W);
  const size_t slots = (size_t)B * Lq * a.nsplit_max * H;
  a.ws_o = ws;
  a.ws_ml = (float*)((char*)ws + (slots * D * (kv_dtype == CSA_F32 ? 4 : 2) + 15) / 16 * 16);
  return launch_attn(a, kv_dtype, true, as_stream(stream)) ? CSA_ERR_LAUNCH : CSA_OK;
}

int hca_dense_attn(int B, int Lq, int64_t q_pos0, int m, int H, int D, int kv_dtype, const void* q,
                   int64_t N_cap, const void* k_c, const void* v_c, int T_raw, int64_t raw_pos0,
                   const void* k_raw, const void* v_raw, int W, const float* sink, void* out,
                   float* lse, void* ws, size_t ws_bytes, void* stream) {
  return dense_attn(B, Lq, q_pos0, nullptr, m, H, D, kv_dtype, q, N_cap, k_c, v_c, T_raw, raw_pos0, k_raw, v_raw,
                    W, sink, out, lse, ws, ws_bytes, stream);
}

int hca_dense_attn_varlen(int B, int Lq, const int64_t* q_pos, int64_t q_pos_max, int m, int H, int D,
                          int kv_dtype, const void* q, int64_t N_cap, const void* k_c, const void* v_c, int R,
                          const void* k_ring, const void* v_ring, int W, const float* sink, void* out,
                          float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!q_pos) return CSA_ERR_NULL;
  return dense_attn(B, Lq, q_pos_max, q_pos, m, H, D, kv_dtype, q, N_cap, k_c, v_c, R, 0, k_ring, v_ring, W, sink,
                    out, lse, ws, ws_bytes, stream);
}

// Source slots per query row of the backward: the selected entries (CSA) or
// the entries visible to the last query (HCA, m > 0), then the window.
static int64_t bwd_slots(int Lq, int64_t q_pos0, int m, int topk, int W) {
  return (m > 0 ? n_last(q_pos0, Lq, m) : (int64_t)topk) + W;
}

size_t csa_sparse_attn_bwd_ws_bytes(int B, int Lq, int64_t q_pos0, int m, int H, int D, int64_t N_cap, int topk,
                                    int W) {
  if (B <= 0 || Lq <= 0 || q_pos0 < 0 || m < 0 || H <= 0 || D <= 0 || N_cap < 0 || topk < 0 || W < 0) return 16;
  const int64_t S = bwd_slots(Lq, q_pos0, m, topk, W);
  if (S > (1 << 30)) return 16;
  return attn_bwd_ws_bytes(B, Lq, H, D, N_cap, (int)S, m > 0 ? 0 : topk);
}

// csa_sparse_attn_bwd and hca_dense_attn_bwd (m > 0: HCA, every visible entry).
static int attn_bwd(int B, int Lq, int64_t q_pos0, int m, int H, int D, int kv_dtype, const void* q, int64_t N_cap,
                    const void* k_c, const void* v_c, int topk, const int32_t* idx, int T_raw, int64_t raw_pos0,
                    const void* k_raw, const void* v_raw, int W, const float* sink, const void* out,
                    const float* lse, const void* dout, float* dq, float* dk_c, float* dv_c, float* dk_raw,
                    float* dv_raw, float* dsink, void* ws, size_t ws_bytes, void* stream) {
  const bool hca = m > 0;
  if (int rc = check_attn_common(B, Lq, q_pos0, H, D, kv_dtype, q, k_c, v_c, T_raw, raw_pos0, k_raw, v_raw, W, sink,
                                 (void*)out, (float*)lse, ws, N_cap, false))
    return rc;
  if (!lse || !dout || !dq || !dk_c || !dv_c || (T_raw > 0 && (!dk_raw || !dv_raw))) return CSA_ERR_NULL;
  if (sink && !dsink) return CSA_ERR_NULL;
  if (!hca && (topk < 0 || topk > 2048 || (topk > 0 && !idx))) return CSA_ERR_SHAPE;
  if (hca && (m > 4096 || n_last(q_pos0, Lq, m) > N_cap)) return CSA_ERR_SHAPE;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk_c) || !aligned16(dv_c) ||
      (T_raw > 0 && (!aligned16(dk_raw) || !aligned16(dv_raw))))
    return CSA_ERR_ALIGN;
  // pairs are indexed as qrow * topk + slot in 32 bits
  if (!hca && (int64_t)B * Lq * topk >= ((int64_t)1 << 31)) return CSA_ERR_SHAPE;
  const int64_t S = bwd_slots(Lq, q_pos0, m, topk, W);
  if (S > ((int64_t)1 << 30)) return CSA_ERR_SHAPE;  // slots are counted in 32 bits
  if (!ws || ws_bytes < csa_sparse_attn_bwd_ws_bytes(B, Lq, q_pos0, m, H, D, N_cap, topk, W))
    return CSA_ERR_WORKSPACE;
  AttnArgs a{};
  a.B = B; a.Lq = Lq; a.q_pos0 = q_pos0; a.m = hca ? m : 1; a.H = H; a.D = D; a.q = q; a.N_cap = N_cap;
  a.k_c = k_c; a.v_c = v_c; a.topk = hca ? 0 : topk; a.idx = hca ? nullptr : idx; a.T_raw = T_raw;
  a.raw_pos0 = raw_pos0; a.k_raw = k_raw; a.v_raw = v_raw; a.W = W; a.sink = sink; a.out = (void*)out;
  a.lse = (float*)lse;
  return launch_attn_bwd(a, hca, (int)S, kv_dtype, dout, dq, dk_c, dv_c, dk_raw, dv_raw, dsink, ws, as_stream(stream))
             ? CSA_ERR_LAUNCH : CSA_OK;
}

int csa_sparse_attn_bwd(int B, int Lq, int64_t q_pos0, int H, int D, int kv_dtype, const void* q, int64_t N_cap,
                        const void* k_c, const void* v_c, int topk, const int32_t* idx, int T_raw, int64_t raw_pos0,
                        const void* k_raw, const void* v_raw, int W, const float* sink, const void* out,
                        const float* lse, const void* dout, float* dq, float* dk_c, float* dv_c, float* dk_raw,
                        float* dv_raw, float* dsink, void* ws, size_t ws_bytes, void* stream) {
  return attn_bwd(B, Lq, q_pos0, 0, H, D, kv_dtype, q, N_cap, k_c, v_c, topk, idx, T_raw, raw_pos0, k_raw, v_raw, W,
                  sink, out, lse, dout, dq, dk_c, dv_c, dk_raw, dv_raw, dsink, ws, ws_bytes, stream);
}

int hca_dense_attn_bwd(int B, int Lq, int64_t q_pos0, int m, int H, int D, int kv_dtype, const void* q,
                       int64_t N_cap, const void* k_c, const void* v_c, int T_raw, int64_t raw_pos0,
                       const void* k_raw, const void* v_raw, int W, const float* sink, const void* out,
                       const float* lse, const void* dout, float* dq, float* dk_c, float* dv_c, float* dk_raw,
                       float* dv_raw, float* dsink, void* ws, size_t ws_bytes, void* stream) {
  if (m < 1) return CSA_ERR_SHAPE;
  return attn_bwd(B, Lq, q_pos0, m, H, D, kv_dtype, q, N_cap, k_c, v_c, 0, nullptr, T_raw, raw_pos0, k_raw, v_raw, W,
                  sink, out, lse, dout, dq, dk_c, dv_c, dk_raw, dv_raw, dsink, ws, ws_bytes, stream);
}

}  // extern "C"
