// Launchers of the indexer kernel (index_qk.hpp): scores to HBM.
#include "index_qk.hpp"

namespace csa {

int index_qk_queries_per_group(int H_i) { return H_i == 128 ? 1 : 64 / H_i; }

int index_qk_nchunks(int64_t q_pos0, int Lq, int m) {
  const int64_t n_max = (q_pos0 + Lq) / m;
  return (int)((n_max + kIdxColsPerWG - 1) / kIdxColsPerWG);
}

int index_fused_cols(int topk) {
  return topk <= kIdxColsPerWG / 4 ? kIdxColsPerWG : topk <= kIdxColsPerWG / 2 ? 2 * kIdxColsPerWG : 0;
}

int index_fused_nchunks(int64_t q_pos0, int Lq, int m, int topk) {
  const int64_t n_max = (q_pos0 + Lq) / m;
  const int cols = index_fused_cols(topk);
  return cols ? (int)((n_max + cols - 1) / cols) : 0;
}

int launch_index_qk(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int64_t N_cap, int H_i,
                    int d_i, int fmt, const void* q_i, const uint8_t* q_s, const float* w_i,
                    const void* k_i, const uint8_t* k_s, float* scores, int sbf, hipStream_t stream) {
  if (index_qk_nchunks(q_pos0, Lq, m) == 0 || B == 0 || Lq == 0) return 0;
  if (index_qk_prefill_eligible(fmt, H_i, d_i, Lq))
    return launch_index_qk_prefill(B, Lq, q_pos0, q_pos, m, N_cap, q_i, w_i, k_i, scores, sbf, stream);
  // Score-store offsets within one group are 32-bit.
  if ((int64_t)index_qk_queries_per_group(H_i) * N_cap * 4 >= 0x7FFFFFF0LL) return 1;
  IdxArgs a = idx_args(B, Lq, q_pos0, q_pos, m, N_cap, H_i, q_i, q_s, w_i, k_i, k_s, stream,
                       index_qk_nchunks(q_pos0, Lq, m));
  a.sc = scores;
  a.sbf = sbf;
  switch (fmt) {
    case 0: idx_dispatch<0, false>(H_i, d_i, a); break;
    case 1: idx_dispatch<1, false>(H_i, d_i, a); break;
    case 2: idx_dispatch<2, false>(H_i, d_i, a); break;
    default: idx_dispatch<3, false>(H_i, d_i, a); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}


}  // namespace csa
