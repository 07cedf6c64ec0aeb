/*
 * csa.h — C ABI of the MI355X (gfx950) compressed-attention library.
 *
 * Hybrid compressed attention as described for DeepSeek-V4:
 *   CSA: every m consecutive tokens' KV is folded into one compressed entry; a
 *        light indexer scores the entries per query, a per-query top-k keeps k
 *        of them, and attention runs over those plus a sliding window of raw
 *        recent tokens, with partial RoPE and a per-head attention sink.
 *   HCA: the same folding with m' = 128, attended densely (no top-k).
 * Sources (page title, section):
 *   [P1] "DeepSeek V4 重磅開源！首次打通華為Ascend，也沒丟掉英偉達，百萬上下文奪回國產模型話語權"
 *        (InfoQ), section 拆解關鍵技術創新 -> 混合注意力機制 and FP4 量化.
 *   [P3] 智猩猩 digest of "DeepSeek-V4: Towards Highly Efficient Million-Token
 *        Context Intelligence" (aiorang.com), section 01 架构与基础设施优化.
 * The pages do not define the compressor or the indexer; the forms computed
 * here are stated at each entry point.
 *
 * Conventions for every entry point
 *  - All tensor pointers are caller-owned DEVICE memory, contiguous row-major
 *    in the shapes given, 16-byte aligned. The library never allocates, frees,
 *    synchronises or copies device-to-host; calls enqueue on `stream` (a
 *    hipStream_t, NULL = the default stream) and return.
 *  - Element formats (csa_dtype): CSA_F32 = float32; CSA_BF16 = bfloat16 bits
 *    (uint16); CSA_FP8_E4M3 = OCP e4m3fn codes (uint8); CSA_FP4_E2M1 = MXFP4:
 *    two e2m1 codes per byte (element 2i in the low nibble) plus one e8m0
 *    scale byte (2^(E-127)) per 32 consecutive elements of the last dim.
 *  - Positions: one shared KV head; the query row i of every sequence sits at
 *    absolute position q_pos0 + i (per sequence in the *_varlen calls). Compressed entry j of a cache covers raw
 *    positions j*m .. j*m+m-1 and is visible to a query at t iff j*m+m-1 <= t,
 *    i.e. for j < n(t) = (t+1)/m.
 *  - RoPE: on the last 64 dims of each head, interleaved pairs (2i, 2i+1),
 *    frequency 10000^(-i/32), angle = position * frequency. Compressed keys are
 *    stored rotated (at their block's last position); raw keys and queries are
 *    stored unrotated and rotated inside the kernels.
 *  - Errors: arguments are checked on the host before anything is enqueued; a
 *    failed check returns a nonzero csa_status and launches nothing. A launch
 *    failure returns CSA_ERR_LAUNCH. Faults inside a kernel surface at the
 *    caller's next synchronisation.
 *  - Workspaces: device scratch sized by the matching *_ws_bytes query; no
 *    initial contents are required. Calls that share a workspace must be
 *    ordered on one stream.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 4

typedef enum {
  CSA_F32 = 0,
  CSA_BF16 = 1,
  CSA_FP8_E4M3 = 2,
  CSA_FP4_E2M1 = 3
} csa_dtype;

typedef enum {
  CSA_OK = 0,
  CSA_ERR_NULL = 1,       /* a required pointer is NULL */
  CSA_ERR_SHAPE = 2,      /* a size or position is out of the supported range */
  CSA_ERR_DTYPE = 3,      /* dtype not supported by this entry point */
  CSA_ERR_ALIGN = 4,      /* a pointer is not 16-byte aligned */
  CSA_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than the *_ws_bytes query */
  CSA_ERR_LAUNCH = 6      /* the HIP runtime rejected a kernel launch */
} csa_status;

/* Version of this ABI (CSA_ABI_VERSION). */
int csa_abi_version(void);

/* Static, NUL-terminated description of a csa_status code. */
const char* csa_strerror(int code);

/*
 * csa_compress — fold every m raw tokens' K and V (and optionally the
 * indexer's raw keys) into one compressed entry.
 * [P1] 混合注意力機制: CSA compresses each m = 4 tokens' KV cache into one
 * entry (sequence length 1/m) and its light indexer picks among those
 * compressed blocks; HCA uses m' = 128. [P1] FP4 量化: the indexer's QK path
 * runs in FP4. Form taken (the pages give none): a softmax-gated weighted
 * sum. For the block j of absolute positions s = j*m .. j*m+m-1:
 *   g_s = <w_gate, K_raw[s]>,  alpha = softmax_s(g),
 *   K_c[j] = RoPE(sum_s alpha_s K_raw[s], j*m+m-1),  V_c[j] = sum_s alpha_s V_raw[s],
 *   KI_c[j] = sum_s alpha_s KI_raw[s]   (unrotated: the indexer has no RoPE),
 * KI_c stored in idx_dtype as csa_state_append stores it: f32; bf16 (nearest
 * even); e4m3fn (nearest even, magnitudes above 448 saturate to 448); MXFP4
 * (per 32 elements the e8m0 code floor(log2 amax) - 2 + 127 clamped to
 * 0..254, 0 for an all-zero block; elements nearest e2m1, ties to the even
 * code, saturating at 6; sign bits copied).
 * RoPE angles are computed inside the kernels (position times frequency
 * reduced to a fraction of a revolution in double precision, then sin/cos in
 * float on [-pi, pi]), so no cos/sin table is passed.
 *
 *   B, T, D      sequences, raw tokens per sequence, head dim (128 or 512)
 *   m            block size, 1..4096
 *   pos0         absolute position of raw row 0; must be a multiple of m
 *   kv_dtype     CSA_F32 or CSA_BF16 (raw and compressed rows alike)
 *   k_raw, v_raw [B, T, D] unrotated keys, values
 *   w_gate       [D] float32
 *   k_c, v_c     [B, N_cap, D]; rows pos0/m .. pos0/m + T/m - 1 are written,
 *                others untouched. A trailing partial block (T % m tokens)
 *                produces nothing. Requires pos0/m + T/m <= N_cap.
 *   d_i          0 (no indexer key) or 32, 64, 128
 *   idx_dtype    storage of ki_c (any csa_dtype; ignored when d_i = 0)
 *   ki_raw       [B, T, d_i] raw indexer keys in kv_dtype (d_i > 0)
 *   ki_c         [B, N_cap, d_i] (fp4: [B, N_cap, d_i/2] bytes), the same rows
 *                as k_c written; ki_c_scale [B, N_cap, d_i/32] e8m0 (fp4 only)
 */
int csa_compress(int B, int T, int D, int m, int64_t pos0, int kv_dtype,
                 const void* k_raw, const void* v_raw, const float* w_gate,
                 void* k_c, void* v_c, int64_t N_cap,
                 int d_i, int idx_dtype, const void* ki_raw, void* ki_c, uint8_t* ki_c_scale,
                 void* stream);

/*
 * csa_index_topk — Lightning Indexer scores, then per-query top-k.
 * [P1] 混合注意力機制: a light indexer picks the important compressed blocks
 * and each query attends only k of them (k = 512..1024); [P1] FP4 量化: the
 * indexer's QK path runs in FP4. Form taken (the pages give none):
 *   I[t, j] = sum_h w_i[t, h] * max(0, <q_i[t, h, :], k_i[j, :]>),  j < n(t),
 * accumulated in float32 (exact for small-integer inputs). Top-k: the key
 * (-I, j) orders entries, so ties go to the lower j; -0 equals +0. The first
 * min(k, n(t)) are written in ascending j, the remaining slots hold -1.
 *
 *   B, Lq, q_pos0  sequences, query rows per sequence, position of row 0
 *   m              compression block of the cache being indexed (>= 1)
 *   N_cap          rows of k_i per sequence; requires n(q_pos0+Lq-1) <= N_cap
 *                  and N_cap * G * 4 < 2^31 bytes, G = 64 / H_i query rows
 *                  scored together (G = 1 for H_i = 128): N_cap < 2^29 for
 *                  H_i >= 64, < 2^25 for H_i = 4
 *   H_i, d_i       indexer heads (4, 8, 16, 32, 64 or 128) and dim
 *                  (32, 64 or 128)
 *   idx_dtype      CSA_F32, CSA_BF16, CSA_FP8_E4M3 or CSA_FP4_E2M1
 *   q_i            [B, Lq, H_i, d_i] (fp4: [B, Lq, H_i, d_i/2] bytes)
 *   q_i_scale      fp4 only: [B, Lq, H_i, d_i/32] e8m0; otherwise NULL
 *   w_i            [B, Lq, H_i] float32 head weights
 *   k_i            [B, N_cap, d_i] (fp4: [B, N_cap, d_i/2] bytes)
 *   k_i_scale      fp4 only: [B, N_cap, d_i/32] e8m0; otherwise NULL
 *   topk           1..2048
 *   idx_out        [B, Lq, topk] int32
 *   ws, ws_bytes   workspace of csa_index_topk_ws_bytes(B, Lq, q_pos0, m,
 *                  N_cap, topk) bytes; needs no initial contents, and its
 *                  contents after the call are unspecified (the scores
 *                  themselves are what csa_index_scores returns).
 *
 * When every indexer workgroup scores a single query (H_i >= 64, or Lq = 1)
 * and topk <= 1024, the top-k runs fused: each workgroup keeps the top k of
 * its chunk of C entries in LDS (C = 2048 for topk <= 512, 4096 for
 * topk <= 1024, so at most a quarter of the scores leave the chip) and only
 * those candidates reach HBM, to be merged per query; the result is the same.
 */
size_t csa_index_topk_ws_bytes(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, int topk);
int csa_index_topk(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap,
                   int H_i, int d_i, int idx_dtype,
                   const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                   const void* k_i, const uint8_t* k_i_scale,
                   int topk, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_index_scores — the indexer step of csa_index_topk alone.
 * Same formula, arguments and limits as csa_index_topk, without the top-k:
 * writes scores [B, Lq, N_cap] float32, I[b, t, j] for j < n(t); entries
 * j >= n(t) are left untouched. No workspace.
 */
int csa_index_scores(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap,
                     int H_i, int d_i, int idx_dtype,
                     const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                     const void* k_i, const uint8_t* k_i_scale, float* scores, void* stream);

/*
 * csa_topk — the top-k step of csa_index_topk alone, on caller scores.
 * [P1] 混合注意力機制 (each query keeps k compressed entries). Same rule as
 * csa_index_topk: key (-score, j), ascending-j output, -1 padding.
 *
 *   scores     [B, Lq, N_cap] float32; row (b, i) is read for j < n(q_pos0+i)
 *              only, and those values must be finite.
 *   idx_out    [B, Lq, topk] int32
 *   ws, ws_bytes  workspace of csa_topk_ws_bytes(B, Lq, q_pos0, m, topk) bytes
 *              (candidate lists of rows longer than 32768 entries).
 */
size_t csa_topk_ws_bytes(int B, int Lq, int64_t q_pos0, int m, int topk);
int csa_topk(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap, const float* scores,
             int topk, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_index_candidates, csa_topk_merge — the two launches of csa_index_topk
 * when it runs fused, callable alone; in sequence they return what
 * csa_index_topk returns.
 *
 * csa_index_candidates: the indexer of csa_index_topk with the top k of each
 * chunk of C entries of a row kept on chip (C = 2048 for topk <= 512, 4096
 * for topk <= 1024). For every query row (b, i) and chunk
 * c < nc = ceil(n(q_pos0+Lq-1) / C) it writes a list of topk pairs: keys
 * (uint32, order-preserving images of the scores: a larger score has a
 * larger key, -0 and +0 share one) at cand[(((b*Lq + i) * nc + c) * topk]
 * and the entry indices at the same offset past the rows * nc * topk keys,
 * in ascending index, padded with key 0 / index -1. Arguments and limits of
 * csa_index_topk, plus H_i >= 64 or Lq == 1, and topk <= 1024
 * (else CSA_ERR_SHAPE).
 * csa_topk_merge: the top k of each row's lists by (key descending, index
 * ascending) into idx_out [B, Lq, topk] int32, ascending index, -1 padding.
 * The rest of `cand` past the lists is its scratch.
 *
 *   cand, cand_bytes  csa_index_candidates_bytes(B, Lq, q_pos0, m, topk) bytes,
 *                     no initial contents needed
 */
size_t csa_index_candidates_bytes(int B, int Lq, int64_t q_pos0, int m, int topk);
int csa_index_candidates(int B, int Lq, int64_t q_pos0, int m, int64_t N_cap,
                         int H_i, int d_i, int idx_dtype,
                         const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                         const void* k_i, const uint8_t* k_i_scale,
                         int topk, void* cand, size_t cand_bytes, void* stream);
int csa_topk_merge(int B, int Lq, int64_t q_pos0, int m, int topk, void* cand, size_t cand_bytes,
                   int32_t* idx_out, void* stream);

/*
 * csa_sparse_attn — CSA attention over the selected compressed entries plus
 * the sliding window, with attention sink.
 * [P1] 混合注意力機制: each query attends its k selected entries; RoPE on the
 * last 64 dims; a sliding-window branch over raw recent tokens; an attention
 * sink lets the weights add up to less than one. Form taken: one softmax over
 *   compressed rows {idx[t, :] >= 0} (keys stored rotated) and
 *   window rows s = max(0, t-W+1) .. t (raw keys rotated at s),
 *   logits <RoPE(q, t), key> / sqrt(D), sink z_h joining the denominator only:
 *   out = sum_r e^(l_r - M) v_r / (e^(z_h - M) + sum_r e^(l_r - M)),
 *   lse = M + ln(denominator). No source and no sink: out = 0, lse = -inf.
 *
 *   B, Lq, q_pos0  as above; H query heads (1..128), D head dim (128 or 512)
 *   kv_dtype       CSA_F32 or CSA_BF16: q, k_c, v_c, k_raw, v_raw and out
 *   q              [B, Lq, H, D] unrotated
 *   N_cap, k_c, v_c  [B, N_cap, D] compressed cache (keys rotated)
 *   topk, idx      [B, Lq, topk] int32; entries outside [0, N_cap) are ignored
 *   T_raw, raw_pos0, k_raw, v_raw  [B, T_raw, D] raw rows at absolute
 *                  positions raw_pos0 ..; must cover every window row:
 *                  raw_pos0 <= max(0, q_pos0-W+1), q_pos0+Lq-1 < raw_pos0+T_raw
 *   W              window, 0..1024
 *   sink           [H] float32 or NULL (no sink)
 *   out            [B, Lq, H, D] in kv_dtype;  lse [B, Lq, H] float32 or NULL
 *   ws, ws_bytes   workspace of csa_sparse_attn_ws_bytes(B, Lq, H, D, topk, W)
 */
size_t csa_sparse_attn_ws_bytes(int B, int Lq, int H, int D, int topk, int W);
int csa_sparse_attn(int B, int Lq, int64_t q_pos0, int H, int D, int kv_dtype,
                    const void* q, int64_t N_cap, const void* k_c, const void* v_c,
                    int topk, const int32_t* idx,
                    int T_raw, int64_t raw_pos0, const void* k_raw, const void* v_raw, int W,
                    const float* sink, void* out, float* lse,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * csa_sparse_attn_noalloc — csa_sparse_attn for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments, computation and results as
 * csa_sparse_attn, without ws / ws_bytes: the workspace is a library-owned
 * device array of CSA_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held until the
 * process ends; its address is looked up once per device on the first call
 * with that device current. The call allocates nothing.
 * Every call on one GPU shares that GPU's array (its contents are whatever
 * the last call left; nothing needs to start at zero), so calls that overlap
 * on one GPU (concurrent streams, or host threads without ordering between
 * their streams) race and must not be made.
 * Errors: as csa_sparse_attn, plus CSA_ERR_WORKSPACE when
 * csa_sparse_attn_ws_bytes(B, Lq, H, D, topk, W) exceeds the array (checked
 * before anything is enqueued) and CSA_ERR_LAUNCH when the array's address
 * cannot be obtained.
 */
#define CSA_NOALLOC_SCRATCH_BYTES (32u << 20)
int csa_sparse_attn_noalloc(int B, int Lq, int64_t q_pos0, int H, int D, int kv_dtype,
                            const void* q, int64_t N_cap, const void* k_c, const void* v_c,
                            int topk, const int32_t* idx,
                            int T_raw, int64_t raw_pos0, const void* k_raw, const void* v_raw, int W,
                            const float* sink, void* out, float* lse, void* stream);

/*
 * hca_dense_attn — HCA attention: every visible compressed entry plus the
 * sliding window, with attention sink.
 * [P1] 混合注意力機制: HCA compresses 128 tokens into one entry and keeps
 * dense attention. Same formula as csa_sparse_attn with the compressed rows
 * j = 0 .. n(t)-1 of a cache built with block m. Requires n(q_pos0+Lq-1) <= N_cap.
 * Arguments as in csa_sparse_attn; ws of hca_dense_attn_ws_bytes(B, Lq,
 * q_pos0, m, H, D, W) bytes.
 */
size_t hca_dense_attn_ws_bytes(int B, int Lq, int64_t q_pos0, int m, int H, int D, int W);
int hca_dense_attn(int B, int Lq, int64_t q_pos0, int m, int H, int D, int kv_dtype,
                   const void* q, int64_t N_cap, const void* k_c, const void* v_c,
                   int T_raw, int64_t raw_pos0, const void* k_raw, const void* v_raw, int W,
                   const float* sink, void* out, float* lse,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Decode state cache and per-sequence positions.
 * [P1] 框架層優化 (heterogeneous KV cache management): a state cache holding
 * the sliding-window tokens and the tokens whose block is not yet compressed,
 * kept apart from the classic cache of compressed entries; [P3] section 01,
 * 异构缓存设计: the same heterogeneous KV cache layout for inference.
 * [P1] 混合注意力機制: an entry exists once its block of m tokens is complete.
 * Layout taken (the pages give none): per sequence a ring of R raw rows, the
 * token at absolute position s in slot s % R, for K and V ([B, R, D], KV
 * dtype) and optionally the indexer's raw key ([B, R, d_i], KV dtype).
 *
 * csa_state_append — one decode step: for each sequence b with t = pos[b] >= 0
 * (a negative position marks an inactive slot: nothing is written), the rows
 * k_new[b], v_new[b] (and ki_new[b]) go to slot t % R of the rings; when t+1
 * is a multiple of m, the block t-m+1 .. t is folded from the ring into
 * entry j = (t+1)/m - 1 exactly as csa_compress folds a block (gate
 * <w_gate, K_raw[s]>, softmax weights alpha, K_c = RoPE(sum alpha K, t),
 * V_c = sum alpha V), and, when d_i > 0, ki_c[b, j] = sum alpha KI (unrotated)
 * stored in idx_dtype: f32; bf16 (nearest even); e4m3fn (nearest even,
 * magnitudes above 448 saturate to 448); MXFP4 (per 32 elements the e8m0 code
 * floor(log2 amax) - 2 + 127 clamped to 0..254, 0 for an all-zero block;
 * elements nearest e2m1, ties to the even code, saturating at 6; sign bits
 * copied). An entry with j >= N_cap is not written. The rows of
 * t-m+1 .. t-1 must be in the ring (appended by earlier steps).
 *
 *   B, D, m, R     sequences, head dim (128 or 512), block (1..4096), ring
 *                  slots (m <= R <= 2^24)
 *   kv_dtype       CSA_F32 or CSA_BF16 (new rows, rings, k_c, v_c)
 *   pos            [B] int64 device positions of the appended tokens
 *   k_new, v_new   [B, D]; w_gate [D] float32
 *   k_ring, v_ring [B, R, D]; k_c, v_c [B, N_cap, D]
 *   d_i            0 (no indexer key) or 32, 64, 128
 *   idx_dtype      storage of ki_c (any csa_dtype)
 *   ki_new [B, d_i], ki_ring [B, R, d_i] (KV dtype); ki_c [B, N_cap, d_i]
 *   (fp4: [B, N_cap, d_i/2] bytes) and ki_c_scale [B, N_cap, d_i/32] (fp4 only)
 * A step reads the ring rows of earlier steps, so steps of one cache must be
 * ordered on one stream. pos must be 8-byte aligned.
 */
int csa_state_append(int B, int D, int m, int R, int kv_dtype, const int64_t* pos,
                     const void* k_new, const void* v_new, const float* w_gate,
                     void* k_ring, void* v_ring, void* k_c, void* v_c, int64_t N_cap,
                     int d_i, int idx_dtype, const void* ki_new, void* ki_ring, void* ki_c,
                     uint8_t* ki_c_scale, void* stream);

/*
 * csa_index_topk_varlen, csa_sparse_attn_varlen, hca_dense_attn_varlen — the
 * calls above with a position per sequence: query row i of sequence b is at
 * t = min(max(q_pos[b], 0), q_pos_max) + i (q_pos [B] int64 device memory;
 * q_pos_max, a host bound of the positions, sizes the grids and takes the
 * place of q_pos0 in the limits and the *_ws_bytes queries). The attention
 * calls read the window rows from the state cache's rings (R slots, position
 * s in slot s % R; requires W + Lq - 1 <= R, and the ring must hold positions
 * max(0, t-W+1) .. t of every query). Everything else is as in the uniform
 * call.
 */
int csa_index_topk_varlen(int B, int Lq, const int64_t* q_pos, int64_t q_pos_max, int m, int64_t N_cap,
                          int H_i, int d_i, int idx_dtype,
                          const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                          const void* k_i, const uint8_t* k_i_scale,
                          int topk, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);
int csa_sparse_attn_varlen(int B, int Lq, const int64_t* q_pos, int64_t q_pos_max, int H, int D, int kv_dtype,
                           const void* q, int64_t N_cap, const void* k_c, const void* v_c,
                           int topk, const int32_t* idx,
                           int R, const void* k_ring, const void* v_ring, int W,
                           const float* sink, void* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream);
int hca_dense_attn_varlen(int B, int Lq, const int64_t* q_pos, int64_t q_pos_max, int m, int H, int D,
                          int kv_dtype, const void* q, int64_t N_cap, const void* k_c, const void* v_c,
                          int R, const void* k_ring, const void* v_ring, int W,
                          const float* sink, void* out, float* lse,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * csa_index_topk_ex — csa_index_topk with optional per-sequence positions and
 * the precision of the indexer scores as arguments.
 * [P1] FP4 量化: rounding the indexer scores from FP32 to BF16 doubles the
 * speed while keeping 99.7% recall. With score_dtype = CSA_BF16 every score
 * I[t, j] (computed in float32 as in csa_index_topk) is rounded to bfloat16
 * (nearest even) before the top-k, and the top-k rule applies to the rounded
 * scores: key (-bf16(I), j), so entries whose scores round alike go to the
 * lower j. Scores that leave the chip (the unfused path) are stored as
 * bfloat16, half the bytes. score_dtype = CSA_F32 is csa_index_topk.
 *
 *   q_pos       NULL: row 0 of every sequence at q_pos0 (csa_index_topk);
 *               else [B] int64 device positions, bounded by q_pos0 (as
 *               q_pos_max of csa_index_topk_varlen)
 *   score_dtype CSA_F32 or CSA_BF16 (else CSA_ERR_DTYPE)
 *   ws          csa_index_topk_ws_bytes(B, Lq, q_pos0, m, N_cap, topk) bytes
 * Everything else as in csa_index_topk.
 */
int csa_index_topk_ex(int B, int Lq, const int64_t* q_pos, int64_t q_pos0, int m, int64_t N_cap,
                      int H_i, int d_i, int idx_dtype,
                      const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                      const void* k_i, const uint8_t* k_i_scale,
                      int topk, int score_dtype, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_index_scores_ex — the indexer step of csa_index_topk_ex alone: the
 * scores of csa_index_scores, with optional per-sequence positions (q_pos as
 * in csa_index_topk_ex) and stored as float32 (score_dtype = CSA_F32, rows of
 * N_cap entries) or as bfloat16 bits rounded to nearest even (CSA_BF16, rows
 * of N_cap rounded up to even entries: scores [B, Lq, (N_cap+1)/2*2]
 * uint16). Entries j >= n(t) of a row are unspecified for bf16 (a bf16 word
 * pairs entries j and j+1) and untouched for f32. No workspace.
 */
int csa_index_scores_ex(int B, int Lq, const int64_t* q_pos, int64_t q_pos0, int m, int64_t N_cap,
                        int H_i, int d_i, int idx_dtype,
                        const void* q_i, const uint8_t* q_i_scale, const float* w_i,
                        const void* k_i, const uint8_t* k_i_scale, int score_dtype, void* scores, void* stream);

/*
 * csa_sparse_attn_bwd, hca_dense_attn_bwd — gradients of csa_sparse_attn /
 * hca_dense_attn for training.
 * [P1] 確定性內核: the attention backward is deterministic (no split-KV; a
 * fixed result whatever the order of work) and batch-invariant. With P_hr =
 * exp(l_hr - lse_h) the forward's weights (l_hr the scaled logit of head h
 * and source row r, lse from the forward), dO = dout:
 *   dP_hr = <dO_h, v_r>, Dl_h = <dO_h, o_h> (o = the forward's out),
 *   dS_hr = P_hr (dP_hr - Dl_h);
 *   dq_h = RoPE^T(sum_r dS_hr k_r, t) / sqrt(D)   (k_r as attended: compressed
 *          keys as stored, window keys rotated at their position s);
 *   dk_r = sum_h dS_hr RoPE(q_h, t) / sqrt(D), rotated back (RoPE^T at s) for
 *          window rows; dv_r = sum_h P_hr dO_h;
 *   dsink_h = -sum over queries of exp(z_h - lse_h) Dl_h.
 * A row used by several queries (an entry selected by many queries of a
 * sequence, a raw row in many windows) receives the sum of their
 * contributions (each one a sum over heads in float32). One workgroup owns
 * each row and adds them in a fixed order: query order for window rows and
 * HCA entries; for a CSA entry its (query, slot) pairs sorted by query row
 * and slot. An entry selected by more than 8192 (query, slot) pairs is
 * summed instead as 64-bit integers in units of 2^-32 (exact, so
 * order-free; contributions clamped to |x| <= 2^30) and rounded once to
 * float32. No atomics touch the gradients: the same bits on every call, and
 * a sequence's gradients do not depend on the rest of the batch.
 *
 * Arguments of the forward call (uniform positions, linear raw rows), plus:
 *   out, lse    the forward's outputs ([B, Lq, H, D] in kv_dtype, [B, Lq, H] f32)
 *   dout        [B, Lq, H, D] in kv_dtype
 *   dq          [B, Lq, H, D] float32
 *   dk_c, dv_c  [B, N_cap, D] float32, every row written (0 where unused)
 *   dk_raw, dv_raw  [B, T_raw, D] float32, every row written (may be NULL
 *               when T_raw = 0)
 *   dsink       [H] float32 (required with a sink, else may be NULL)
 *   ws, ws_bytes  csa_sparse_attn_bwd_ws_bytes(B, Lq, q_pos0, 0, H, D, N_cap,
 *               topk, W) bytes (HCA: m instead of 0, topk 0); no initial
 *               contents needed. It holds, per (query, source slot, head),
 *               the weight P and dS / sqrt(D) (8 bytes; slots: topk + W for
 *               CSA, n(q_pos0 + Lq - 1) + W for HCA), the rotated q, the sink
 *               parts, and for CSA the index of the (query, slot) pairs of
 *               each compressed entry (8 bytes per entry, 8 per pair).
 * Errors: CSA_ERR_SHAPE also when B * Lq * topk >= 2^31 (pairs are indexed
 * in 32 bits).
 * hca_dense_attn_bwd: the same for hca_dense_attn (block m, every visible entry).
 */
size_t csa_sparse_attn_bwd_ws_bytes(int B, int Lq, int64_t q_pos0, int m, int H, int D, int64_t N_cap, int topk,
                                    int W);
int csa_sparse_attn_bwd(int B, int Lq, int64_t q_pos0, int H, int D, int kv_dtype,
                        const void* q, int64_t N_cap, const void* k_c, const void* v_c,
                        int topk, const int32_t* idx,
                        int T_raw, int64_t raw_pos0, const void* k_raw, const void* v_raw, int W,
                        const float* sink, const void* out, const float* lse, const void* dout,
                        float* dq, float* dk_c, float* dv_c, float* dk_raw, float* dv_raw, float* dsink,
                        void* ws, size_t ws_bytes, void* stream);
int hca_dense_attn_bwd(int B, int Lq, int64_t q_pos0, int m, int H, int D, int kv_dtype,
                       const void* q, int64_t N_cap, const void* k_c, const void* v_c,
                       int T_raw, int64_t raw_pos0, const void* k_raw, const void* v_raw, int W,
                       const float* sink, const void* out, const float* lse, const void* dout,
                       float* dq, float* dk_c, float* dv_c, float* dk_raw, float* dv_raw, float* dsink,
                       void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
