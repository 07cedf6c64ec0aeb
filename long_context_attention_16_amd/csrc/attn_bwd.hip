// Backward pass of the CSA / HCA attention (gradients for q, the compressed
// keys and values, the raw window keys and values, and the sinks).
//
// Source: "DeepSeek V4 重磅開源！…" (InfoQ), section 確定性內核: training needs
// a deterministic attention backward (the pages drop split-KV and keep a
// fixed accumulation order) and batch-invariant outputs. Formula (the
// gradient of the forward of attn.hip, which is one softmax over the
// selected compressed rows, the window rows and the sink):
//   P_hr = exp(l_hr - lse_h), l_hr = <RoPE(q_h, t), k_r> / sqrt(D);
//   dP_hr = <dO_h, v_r>, Dl_h = <dO_h, o_h>, dS_hr = P_hr (dP_hr - Dl_h);
//   dq_h = RoPE^T(sum_r dS_hr k_r, t) / sqrt(D);
//   dk_r = sum_h dS_hr RoPE(q_h, t) / sqrt(D)  (window rows: RoPE^T at s);
//   dv_r = sum_h P_hr dO_h;  dz_h = -exp(z_h - lse_h) Dl_h.
//
// Design. Workgroup = (query row, group of 4 heads): the query's source rows
// go through LDS in tiles of 8 (f32, window keys rotated in LDS), logits and
// dP by 4 threads per dot product, dq accumulated in registers. A row's key
// and value gradients receive contributions from every query (and head
// group) that uses it; they are added as 64-bit fixed-point integers
// (units of 2^-32) with atomics, so the sums are exact and the result is the
// same bits whatever the order of the additions: deterministic without a
// split-free ordering pass. A last kernel converts them to f32; the sinks'
// per-query parts are summed in query order.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdHeads = 4;   // heads per workgroup
constexpr int kBwdRows = 8;    // source rows per tile
constexpr float kFixScale = 4294967296.f;  // 2^32: fixed-point unit 2^-32

struct AttnBwdArgs {
  AttnArgs a;
  const void* dout;
  float* dq;
  long long *acc_kc, *acc_vc, *acc_kr, *acc_vr;
  float* dsink_part;  // [B*Lq][H]
};

__device__ __forceinline__ long long to_fix(float x) {
  x = fminf(fmaxf(x, -1073741824.f), 1073741824.f);  // |x| <= 2^30: no overflow of the 64-bit units
  return __float2ll_rn(x * kFixScale);
}

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) {
  return Elem<T>::load(p + i);
}

// Source row sp of query row qrow: kind 0 masked, 1 compressed entry j, 2
// window row at absolute position *pos; *row = the row's index in k_c / v_c
// (kind 1: b * N_cap + j) or k_raw / v_raw (kind 2: b * T_raw + s - raw_pos0).
template <bool HCA>
__device__ __forceinline__ int bwd_source(const AttnArgs& p, int b, int64_t qrow, int n_c, int64_t lo, int n_w, int sp,
                                          int64_t* row, int64_t* pos) {
  *row = 0;
  *pos = 0;
  if (sp < n_c) {
    const int64_t j = HCA ? sp : (int64_t)p.idx[qrow * p.topk + sp];
    if (j < 0 || j >= p.N_cap) return 0;
    *row = (int64_t)b * p.N_cap + j;
    return 1;
  }
  const int w = sp - n_c;
  if (w >= n_w) return 0;
  *pos = lo + w;
  *row = (int64_t)b * p.T_raw + (lo + w - p.raw_pos0);
  return 2;
}

template <typename T, int D, bool HCA>
__global__ __launch_bounds__(kBwdThreads) void attn_bwd_kernel(AttnBwdArgs g) {
  const AttnArgs& p = g.a;
  constexpr int NT = kBwdThreads, HG = kBwdHeads, R = kBwdRows;
  constexpr int EPT = HG * D / NT;  // (head, d) elements of a thread: e = tid + NT * k
  static_assert(EPT >= 1 && HG * D % NT == 0, "whole elements per thread");
  __shared__ float s_q[HG][D], s_do[HG][D];
  __shared__ float s_k[R][D], s_v[R][D];
  __shared__ float s_l[HG][R], s_dp[HG][R], s_p[HG][R], s_ds[HG][R];
  __shared__ float s_lse[HG], s_dl[HG];
  __shared__ int s_kind[R];
  __shared__ int64_t s_row[R], s_pos[R];

  const int tid = threadIdx.x;
  const int ngroups = (p.H + HG - 1) / HG;
  const int64_t qrow = blockIdx.x / ngroups;
  const int h0 = (int)(blockIdx.x % ngroups) * HG;
  const int b = (int)(qrow / p.Lq);
  const int64_t t = p.q_pos0 + qrow % p.Lq;
  const int n_c = HCA ? (int)((t + 1) / p.m) : p.topk;
  const int64_t lo = t - p.W + 1 > 0 ? t - p.W + 1 : 0;
  const int n_w = p.W > 0 ? (int)(t - lo + 1) : 0;
  const int S = n_c + p.W;
  const float rs = 1.f / sqrtf((float)D);

  // q (rotated at t), dO, and Dl_h = <dO_h, o_h> for the group's heads
  const T* qb = (const T*)p.q + (qrow * p.H) * D;
  const T* ob = (const T*)p.out + (qrow * p.H) * D;
  const T* db = (const T*)g.dout + (qrow * p.H) * D;
  for (int e = tid; e < HG * D; e += NT) {
    const int hh = e / D, d = e % D, h = h0 + hh;
    const bool hok = h < p.H;
    s_q[hh][d] = hok ? ld(qb, (int64_t)h * D + d) : 0.f;
    s_do[hh][d] = hok ? ld(db, (int64_t)h * D + d) : 0.f;
  }
  if (tid < HG) s_lse[tid] = h0 + tid < p.H ? p.lse[qrow * p.H + h0 + tid] : 0.f;
  __syncthreads();
  for (int e = tid; e < HG * kRopePairs; e += NT) {
    const int hh = e / kRopePairs, pr = e % kRopePairs, d = D - kRopeDims + 2 * pr;
    float c, sn;
    rope_cos_sin(t, pr, &c, &sn);
    const float x0 = s_q[hh][d], x1 = s_q[hh][d + 1];
    s_q[hh][d] = x0 * c - x1 * sn;
    s_q[hh][d + 1] = x0 * sn + x1 * c;
  }
  // Dl: thread group of NT / HG threads per head, strided over d, then a reduction
  {
    constexpr int TPH = NT / HG;
    const int hh = tid / TPH, part = tid % TPH, h = h0 + hh;
    float acc = 0.f;
    if (h < p.H)
      for (int d = part; d < D; d += TPH) acc = fmaf(s_do[hh][d], ld(ob, (int64_t)h * D + d), acc);
#pragma unroll
    for (int o = TPH / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, kWave);
    if (part == 0) s_dl[hh] = acc;
  }
  __syncthreads();

  float dq[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) dq[k] = 0.f;

  for (int r0 = 0; r0 < S; r0 += R) {
    // the tile's rows: sources, then K (window rows rotated at their position) and V
    if (tid < R) {
      int64_t row, pos;
      s_kind[tid] = r0 + tid < S ? bwd_source<HCA>(p, b, qrow, n_c, lo, n_w, r0 + tid, &row, &pos) : 0;
      s_row[tid] = row;
      s_pos[tid] = pos;
    }
    __syncthreads();
    for (int e = tid; e < R * D; e += NT) {
      const int r = e / D, d = e % D, kd = s_kind[r];
      const T* kp = (const T*)(kd == 2 ? p.k_raw : p.k_c);
      const T* vp = (const T*)(kd == 2 ? p.v_raw : p.v_c);
      s_k[r][d] = kd ? ld(kp, s_row[r] * D + d) : 0.f;
      s_v[r][d] = kd ? ld(vp, s_row[r] * D + d) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < R * kRopePairs; e += NT) {
      const int r = e / kRopePairs, pr = e % kRopePairs, d = D - kRopeDims + 2 * pr;
      if (s_kind[r] != 2) continue;
      float c, sn;
      rope_cos_sin(s_pos[r], pr, &c, &sn);
      const float x0 = s_k[r][d], x1 = s_k[r][d + 1];
      s_k[r][d] = x0 * c - x1 * sn;
      s_k[r][d + 1] = x0 * sn + x1 * c;
    }
    __syncthreads();
    // logits (dot < HG*R) and dP (the rest): 4 threads per dot product
    {
      const int dot = tid / 4, part = tid % 4;
      const int hh = (dot % (HG * R)) / R, r = dot % R;
      const bool is_l = dot < HG * R;
      float acc = 0.f;
      for (int d = part; d < D; d += 4)
        acc = fmaf(is_l ? s_q[hh][d] : s_do[hh][d], is_l ? s_k[r][d] : s_v[r][d], acc);
      acc += __shfl_xor(acc, 1, kWave);
      acc += __shfl_xor(acc, 2, kWave);
      if (part == 0) {
        if (is_l) s_l[hh][r] = acc * rs;
        else s_dp[hh][r] = acc;
      }
    }
    __syncthreads();
    if (tid < HG * R) {
      const int hh = tid / R, r = tid % R;
      const bool ok = s_kind[r] != 0 && h0 + hh < p.H;
      const float pv = ok ? __expf(s_l[hh][r] - s_lse[hh]) : 0.f;
      s_p[hh][r] = pv;
      s_ds[hh][r] = ok ? pv * (s_dp[hh][r] - s_dl[hh]) : 0.f;
    }
    __syncthreads();
    // dq += dS k (unscaled; 1/sqrt(D) at the end)
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = tid + NT * k, hh = e / D, d = e % D;
#pragma unroll
      for (int r = 0; r < R; ++r) dq[k] = fmaf(s_ds[hh][r], s_k[r][d], dq[k]);
    }
    __syncthreads();  // every thread is done with s_k: reuse it for the key gradients
    for (int e = tid; e < R * D; e += NT) {
      const int r = e / D, d = e % D;
      float u = 0.f, w = 0.f;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        u = fmaf(s_ds[hh][r], s_q[hh][d], u);
        w = fmaf(s_p[hh][r], s_do[hh][d], w);
      }
      s_k[r][d] = u * rs;
      s_v[r][d] = w;
    }
    __syncthreads();
    for (int e = tid; e < R * kRopePairs; e += NT) {  // window rows: back to the unrotated frame
      const int r = e / kRopePairs, pr = e % kRopePairs, d = D - kRopeDims + 2 * pr;
      if (s_kind[r] != 2) continue;
      float c, sn;
      rope_cos_sin(s_pos[r], pr, &c, &sn);
      const float x0 = s_k[r][d], x1 = s_k[r][d + 1];
      s_k[r][d] = x0 * c + x1 * sn;
      s_k[r][d + 1] = -x0 * sn + x1 * c;
    }
    __syncthreads();
    for (int e = tid; e < R * D; e += NT) {
      const int r = e / D, d = e % D, kd = s_kind[r];
      if (!kd) continue;
      long long* ak = kd == 2 ? g.acc_kr : g.acc_kc;
      long long* av = kd == 2 ? g.acc_vr : g.acc_vc;
      atomicAdd((unsigned long long*)(ak + s_row[r] * D + d), (unsigned long long)to_fix(s_k[r][d]));
      atomicAdd((unsigned long long*)(av + s_row[r] * D + d), (unsigned long long)to_fix(s_v[r][d]));
    }
    __syncthreads();  // the tile's LDS is reused by the next tile
  }

  // dq: back to the unrotated frame (pairs in LDS), scaled by 1/sqrt(D)
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + NT * k;
    s_q[e / D][e % D] = dq[k] * rs;
  }
  __syncthreads();
  for (int e = tid; e < HG * kRopePairs; e += NT) {
    const int hh = e / kRopePairs, pr = e % kRopePairs, d = D - kRopeDims + 2 * pr;
    float c, sn;
    rope_cos_sin(t, pr, &c, &sn);
    const float x0 = s_q[hh][d], x1 = s_q[hh][d + 1];
    s_q[hh][d] = x0 * c + x1 * sn;
    s_q[hh][d + 1] = -x0 * sn + x1 * c;
  }
  __syncthreads();
  for (int e = tid; e < HG * D; e += NT) {
    const int hh = e / D, d = e % D, h = h0 + hh;
    if (h < p.H) g.dq[(qrow * p.H + h) * D + d] = s_q[hh][d];
  }
  if (tid < HG && h0 + tid < p.H) {
    const int h = h0 + tid;
    g.dsink_part[qrow * p.H + h] = p.sink ? -__expf(p.sink[h] - s_lse[tid]) * s_dl[tid] : 0.f;
  }
}

__global__ void fill_zero_kernel(long long* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

__global__ void fix_to_f32_kernel(const long long* acc, float* out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = (float)((double)acc[i] * (1.0 / 4294967296.0));
}

// dsink[h] = sum over query rows in a fixed order: workgroup h, thread t
// sums rows t, t + 256, ... in order, then a fixed tree over the threads.
__global__ __launch_bounds__(256) void dsink_sum_kernel(const float* part, int64_t rows, int H, float* dsink) {
  __shared__ float red[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  float s = 0.f;
  for (int64_t r = tid; r < rows; r += 256) s += part[r * H + h];
  red[tid] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) dsink[h] = red[0];
}

}  // namespace

size_t attn_bwd_ws_bytes(int B, int Lq, int H, int64_t N_cap, int T_raw, int D) {
  const size_t acc = ((size_t)B * N_cap + (size_t)B * T_raw) * D * 2 * sizeof(long long);
  return acc + ((size_t)B * Lq * H * sizeof(float) + 255) / 256 * 256;
}

int launch_attn_bwd(const AttnArgs& a, bool hca, int kv_dtype, const void* dout, float* dq, float* dk_c, float* dv_c,
                    float* dk_raw, float* dv_raw, float* dsink, void* ws, hipStream_t st) {
  AttnBwdArgs g;
  g.a = a;
  g.dout = dout;
  g.dq = dq;
  const int64_t nc = (int64_t)a.B * a.N_cap * a.D, nr = (int64_t)a.B * a.T_raw * a.D;
  g.acc_kc = (long long*)ws;
  g.acc_vc = g.acc_kc + nc;
  g.acc_kr = g.acc_vc + nc;
  g.acc_vr = g.acc_kr + nr;
  g.dsink_part = (float*)(g.acc_vr + nr);
  const int64_t nacc = 2 * (nc + nr);
  const int fill_blocks = (int)((nacc + 255) / 256 < 4096 ? (nacc + 255) / 256 : 4096);
  if (nacc > 0) hipLaunchKernelGGL(fill_zero_kernel, dim3(fill_blocks), dim3(256), 0, st, g.acc_kc, nacc);
  const int64_t rows = (int64_t)a.B * a.Lq;
  if (rows > 0) {
    const dim3 grid((unsigned)(rows * ((a.H + kBwdHeads - 1) / kBwdHeads)));
#define CSA_BWD(TT, DD)                                                                                    \
  if (hca) hipLaunchKernelGGL((attn_bwd_kernel<TT, DD, true>), grid, dim3(kBwdThreads), 0, st, g);        \
  else hipLaunchKernelGGL((attn_bwd_kernel<TT, DD, false>), grid, dim3(kBwdThreads), 0, st, g)
    if (kv_dtype == 0) {
      if (a.D == 128) { CSA_BWD(float, 128); } else { CSA_BWD(float, 512); }
    } else {
      if (a.D == 128) { CSA_BWD(uint16_t, 128); } else { CSA_BWD(uint16_t, 512); }
    }
#undef CSA_BWD
  }
  if (nc > 0) {
    const int nb = (int)((nc + 255) / 256 < 4096 ? (nc + 255) / 256 : 4096);
    hipLaunchKernelGGL(fix_to_f32_kernel, dim3(nb), dim3(256), 0, st, g.acc_kc, dk_c, nc);
    hipLaunchKernelGGL(fix_to_f32_kernel, dim3(nb), dim3(256), 0, st, g.acc_vc, dv_c, nc);
  }
  if (nr > 0) {
    const int nb = (int)((nr + 255) / 256 < 4096 ? (nr + 255) / 256 : 4096);
    hipLaunchKernelGGL(fix_to_f32_kernel, dim3(nb), dim3(256), 0, st, g.acc_kr, dk_raw, nr);
    hipLaunchKernelGGL(fix_to_f32_kernel, dim3(nb), dim3(256), 0, st, g.acc_vr, dv_raw, nr);
  }
  if (dsink) hipLaunchKernelGGL(dsink_sum_kernel, dim3(a.H), dim3(256), 0, st, g.dsink_part, rows, a.H, dsink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
