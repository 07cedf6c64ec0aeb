// Launcher of the indexer kernel (index_qk.hpp) in fused mode: per-chunk
// top-k candidate lists instead of scores.
#include "index_qk.hpp"

namespace csa {

int launch_index_qk_fused(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int64_t N_cap, int H_i,
                          int d_i, int fmt,
                          const void* q_i, const uint8_t* q_s, const float* w_i, const void* k_i,
                          const uint8_t* k_s, int topk, int sbf, uint32_t* cand_key, int32_t* cand_idx,
                          hipStream_t stream) {
  const int nchunks = index_fused_nchunks(q_pos0, Lq, m, topk);
  if (nchunks == 0 || B == 0 || Lq == 0) return 0;
  IdxArgs a = idx_args(B, Lq, q_pos0, q_pos, m, N_cap, H_i, q_i, q_s, w_i, k_i, k_s, stream, nchunks);
  a.topk = topk; a.sbf = sbf; a.ck = cand_key; a.ci = cand_idx;
  // chunks of 2048 entries for k <= 512, of 4096 for k <= 1024 (16 or 32 tiles per wave)
  if (index_fused_cols(topk) == kIdxColsPerWG) {
    switch (fmt) {
      case 0: idx_dispatch<0, true, 16>(H_i, d_i, a); break;
      case 1: idx_dispatch<1, true, 16>(H_i, d_i, a); break;
      case 2: idx_dispatch<2, true, 16>(H_i, d_i, a); break;
      default: idx_dispatch<3, true, 16>(H_i, d_i, a); break;
    }
  } else {
    switch (fmt) {
      case 0: idx_dispatch<0, true, 32>(H_i, d_i, a); break;
      case 1: idx_dispatch<1, true, 32>(H_i, d_i, a); break;
      case 2: idx_dispatch<2, true, 32>(H_i, d_i, a); break;
      default: idx_dispatch<3, true, 32>(H_i, d_i, a); break;
    }
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
