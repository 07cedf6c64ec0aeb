// K4 for many query heads — CSA attention in two launches with no split
// combine, for one shared KV head of dim 512 in bf16 and H a multiple of 16
// (the decode shape: 64 heads over k + W gathered rows).
// Workspace: P' [rows][H][slots] bf16, chunk statistics [rows][chunks][H]
// (max, sum) and the slots' V row offsets [rows][slots] (written by phase A).
//
// Source: "DeepSeek V4 重磅開源！…" (InfoQ), section 混合注意力機制 (the
// selected compressed entries plus a sliding window over raw tokens, RoPE on
// the last 64 dims, an attention sink). Same formula as the general kernel in
// attn.hip: one softmax over the compressed and window rows, logits
// <RoPE(q, t), key> / sqrt(D), the sink logit joining the denominator only.
//
// Why two launches: splitting a query's rows over workgroups forces every
// split to write a partial output of H x D values (64 KB at H = 64, D = 512)
// for a combine step, as much traffic as the rows themselves. Here
//  * phase A, one workgroup per (query, chunk of 64 source rows), gathers the
//    chunk's K rows into LDS, computes the logits of all H heads on MFMA and
//    writes P' = 2^(l - m_c) in bf16 with the chunk's (m_c, sum P') per head;
//  * phase B, one workgroup per (query, slice of 64 dims, or of 32 when a
//    call has few query rows), folds the chunk statistics and the sink into
//    per-chunk factors 2^(m_c - M) / den, gathers the V slices of all rows and
//    accumulates O = sum_r P_r V_r on MFMA, already normalized.
// P' carries no more rounding than the PV product needs anyway (P enters the
// MFMA in bf16). Every reduction runs in a fixed order, so results are
// deterministic and independent of the batch.
#include "attn_decode.hpp"

namespace csa {

namespace {
using namespace dec;

// Workgroup index -> (query row, unit): all units of a query on one XCD
// (workgroups are dealt to the 8 XCDs by block index modulo 8), so the
// query's Q rows, P' rows and statistics are read from that XCD's L2.
template <int NW>
__global__ __launch_bounds__(NW * kWave) void attn_dec_qk_kernel(AttnArgs p, int nchunk, int spad,
                                                                  uint16_t* __restrict__ pp, float* __restrict__ ml,
                                                                  int64_t* __restrict__ rowsrc) {
  __shared__ DecAShared L;
  const int rows = gridDim.x / nchunk;
  dec_a_body<NW>(L, p, blockIdx.x % rows, blockIdx.x / rows, nchunk, spad, pp, ml, rowsrc);
}

template <int NW, int DSL, int BR>
__global__ __launch_bounds__(NW * kWave) void attn_dec_pv_kernel(AttnArgs p, int nchunk, int spad,
                                                                  const uint16_t* __restrict__ pp,
                                                                  const float* __restrict__ ml,
                                                                  const int64_t* __restrict__ rowsrc) {
  __shared__ DecBShared<NW, BR, DSL> L;
  const int rows = gridDim.x / (kDecD / DSL);
  dec_b_body<NW, BR, DSL>(L, p, blockIdx.x % rows, blockIdx.x / rows, nchunk, spad, pp, ml, rowsrc);
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

}  // namespace

// Sources per query must also fit phase B's table of chunk statistics
// (kMaxChunks chunks); the API allows more (W up to 1024), and such calls run
// the general split kernel.
using dec::kDecD;
using dec::kArows;
using dec::kMaxChunks;

bool attn_decode_eligible(int kv_dtype, bool hca, int H, int D, int topk, int W) {
  return !hca && kv_dtype == 1 && D == kDecD && H % 16 == 0 && H >= 16 && H <= 128 && topk + W > 0 &&
         topk + W <= kMaxChunks * kArows;
}

int attn_decode_chunks(int topk, int W) { return (topk + W + kArows - 1) / kArows; }

size_t attn_decode_ws(int B, int Lq, int H, int topk, int W) {
  const int nc = attn_decode_chunks(topk, W);
  const size_t rows = (size_t)B * Lq;
  const size_t pbytes = (rows * H * nc * kArows * 2 + 255) / 256 * 256;
  const size_t mbytes = (rows * nc * H * 2 * 4 + 255) / 256 * 256;
  return pbytes + mbytes + rows * nc * kArows * 8;
}

int launch_attn_decode(const AttnArgs& a, void* ws, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.Lq;
  if (rows == 0) return 0;
  const int nc = attn_decode_chunks(a.topk, a.W);
  const int spad = nc * kArows;
  uint16_t* pp = (uint16_t*)ws;
  float* ml = (float*)((char*)ws + ((size_t)rows * a.H * spad * 2 + 255) / 256 * 256);
  int64_t* rowsrc = (int64_t*)((char*)ml + ((size_t)rows * nc * a.H * 8 + 255) / 256 * 256);
  if (nc == 0) return 1;
  // phase B: 64-dim slices when 8 per query row fill the chip, else 32-dim
  // slices (twice the workgroups); staging 640 rows at a time, or, when the
  // 32-dim workgroups fit one per CU and a list is longer, 1152 (one block
  // for k = 1024 and W = 128, in LDS that leaves room for one workgroup per CU)
  const int cus = device_cus();
  const int kind = rows * (kDecD / 64) >= cus ? 0 : spad > kBrowsMax && rows * (kDecD / 32) <= cus ? 2 : 1;
#define CSA_DEC_B(NW, DSL, BR)                                                                                \
  hipLaunchKernelGGL((attn_dec_pv_kernel<NW, DSL, BR>), dim3((unsigned)(rows * (kDecD / DSL))),               \
                     dim3(NW * kWave), 0, st, a, nc, spad, (const uint16_t*)pp, (const float*)ml,            \
                     (const int64_t*)rowsrc)
#define CSA_DEC(NW)                                                                                           \
  hipLaunchKernelGGL(attn_dec_qk_kernel<NW>, dim3((unsigned)(rows * nc)), dim3(NW * kWave), 0, st, a, nc,      \
                     spad, pp, ml, rowsrc);                                                                   \
  if (kind == 0)                                                                                              \
    CSA_DEC_B(NW, 64, kBrowsMax);                                                                             \
  else if (kind == 1)                                                                                         \
    CSA_DEC_B(NW, 32, kBrowsMax);                                                                             \
  else                                                                                                        \
    CSA_DEC_B(NW, 32, kBrowsNarrow)
  switch (a.H / 16) {
    case 1: CSA_DEC(1); break;
    case 2: CSA_DEC(2); break;
    case 3: CSA_DEC(3); break;
    case 4: CSA_DEC(4); break;
    case 5: CSA_DEC(5); break;
    case 6: CSA_DEC(6); break;
    case 7: CSA_DEC(7); break;
    default: CSA_DEC(8); break;
  }
#undef CSA_DEC
#undef CSA_DEC_B
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
