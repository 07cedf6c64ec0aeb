// K2 for many query rows at once (prefill chunks): the fp8 e4m3 indexer with
// 64 heads of dim 128, I[t, j] = sum_h w[t, h] * max(0, <q_I[t, h], k_I[j]>).
//
// Source: "DeepSeek V4 重磅開源！…" (InfoQ), section 混合注意力機制 (the light
// indexer scores every compressed block for each query) and section FP4 量化
// (low-precision QK path of the indexer). Same reading as the general kernel
// in index_qk.hpp: ReLU'd per-head dot products mixed by per-query head
// weights, f32 result.
//
// At decode each query streams the whole k_I once and the work is HBM-bound;
// in a prefill chunk thousands of queries share the same k_I, so the work is a
// dense fp8 GEMM (M = query x head, N = entries, K = d_I = 128) plus an
// epilogue of two VALU operations per (query, head, entry): the ReLU and the
// weighted head sum. Design:
//  * a workgroup of 8 waves owns 16 consecutive queries (two per wave) and a
//    chunk of 8192 entries; a wave keeps its two queries' q_I operand
//    fragments (64 VGPRs) and the head weights its lanes need (64 VGPRs) in
//    registers for the whole chunk;
//  * the A operand pairs the wave's two queries inside every 32-row M tile:
//    row p of tile mt is head 16mt + 4(p/8) + p%4 of query (p/4)%2. In the
//    32x32 result layout the rows a lane holds are then exactly heads
//    16mt .. 16mt+15 of ONE query (query = the lane's half-wave), so across the
//    4 tiles a lane holds all 64 heads of its query for its entry and sums
//    them alone: no cross-lane step. Lanes 0-31 end with query 0's scores of
//    the 32 entries, lanes 32-63 with query 1's;
//  * k_I streams HBM -> LDS in blocks of 256 rows (32 KB) through a ring of
//    three buffers with direct global-to-LDS loads, two blocks ahead; a block
//    is read from L2 / HBM once per workgroup and used by its 16 queries.
//    Within a row the 16-byte chunks are XOR-swizzled by bits 1..3 of the row
//    index: a 16-byte LDS read serves 16 lanes (256 bytes) per cycle, and the
//    B-fragment reads of 16 consecutive rows at one logical chunk then cover
//    all 64 banks once (no bank conflicts, measured);
//  * per step a wave multiplies 32 entries (one N tile, read from LDS once)
//    by 4 M tiles: 8 MFMA 32x32x64 fp8; the next step's LDS reads are issued
//    right after and land while this step's epilogue runs, and the block
//    hand-over (barrier, next copy) sits between a block's last MFMAs and
//    its last epilogue, so the pipeline never drains at block ends.
// LDS reads, not MFMA or VALU throughput, limited the earlier one-query-per-
// wave form (every B fragment read fed 4 MFMAs and each step needed a
// cross-half exchange through LDS); here each read feeds 8. Measured on
// MI355X: two waves per SIMD, each overlapping the other's MFMAs with its
// epilogue, beat one wave per SIMD with a lagged epilogue (512 registers,
// two accumulator sets) by about 7%.
// Entries past a query's visible count n(t) are stored through a buffer
// resource with an offset past its end, which the hardware drops, so no store
// is conditional.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

namespace {

constexpr int kPfWaves = 8;
constexpr int kPfQ = 2 * kPfWaves;           // queries per workgroup, two per wave
constexpr int kPfHeads = 64;
constexpr int kPfDim = 128;                  // fp8 bytes per row
constexpr int kPfBlk = 256;                  // k_I rows per LDS block
constexpr int kPfChunk = 8192;               // entries per workgroup
constexpr int kPfSteps = kPfBlk / 32;        // wave steps (32 entries each) per block
constexpr int kPfLoads = kPfBlk * kPfDim / 1024 / kPfWaves;  // 1 KB LDS loads per wave per block
constexpr int kPfStores = kPfSteps;          // score stores per wave per block
static_assert(kPfLoads * kPfWaves * 1024 == kPfBlk * kPfDim, "block splits evenly over the waves");
static_assert(kPfChunk % kPfBlk == 0, "whole blocks per chunk");

__device__ __forceinline__ void pf_lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt immediate: at most n vector-memory operations outstanding.
__device__ __forceinline__ constexpr int pf_vmcnt(int n) {
  return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 0x3) << 14);
}

// SBF: bf16 scores (a template parameter: the f32 epilogue stays as short as
// before, the kernel being bound by its step latency).
template <bool SBF>
__global__ __launch_bounds__(kPfWaves * kWave) void index_qk_prefill_kernel(
    int Lq, int64_t q_pos0, const int64_t* __restrict__ q_pos, int m, int64_t N_cap, int ngroups, int nchunks,
    const uint8_t* __restrict__ q_i, const float* __restrict__ w_i, const uint8_t* __restrict__ k_i,
    float* __restrict__ scores) {
  constexpr int sbf = SBF ? 1 : 0;
  // Three separate arrays rather than one indexed by block: the compiler
  // then knows which ring buffer an LDS read touches and waits only for the
  // copies into that buffer, not for the blocks still in flight.
  __shared__ __attribute__((aligned(16))) uint8_t s_k0[kPfBlk * kPfDim];
  __shared__ __attribute__((aligned(16))) uint8_t s_k1[kPfBlk * kPfDim];
  __shared__ __attribute__((aligned(16))) uint8_t s_k2[kPfBlk * kPfDim];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int half = lane / 32;
  const int n32 = lane % 32;
  const int c = blockIdx.x % nchunks;
  const int gg = blockIdx.x / nchunks;
  const int b = gg / ngroups;
  q_pos0 = seq_pos(q_pos, q_pos0, b);  // from here on: this sequence's row-0 position
  const int i0 = (gg % ngroups) * kPfQ;
  const int nq = min(kPfQ, Lq - i0);
  const int64_t n_last = (q_pos0 + i0 + nq) / m;  // visible entries of the group's last query
  const int64_t j0 = (int64_t)c * kPfChunk;
  if (j0 >= n_last) return;  // uniform over the workgroup
  const int nvis = (int)min<int64_t>(kPfChunk, n_last - j0);
  const int nblk = (nvis + kPfBlk - 1) / kPfBlk;

  // LDS layout of a block: row r at r * 128 bytes; its physical 16-byte
  // chunk p holds logical chunk p ^ swz(r).
  auto swz = [](int r) { return (r >> 1) & 7; };
  // Block loads: load u of wave w covers block rows 8(w*L + u) .. +7; lane l
  // writes row 8(..) + l/8, physical chunk l%8. Rows past N_cap re-read the
  // last row (their scores are never stored).
  const uint8_t* kchunk = k_i + ((int64_t)b * N_cap + j0) * kPfDim;
  const int last_row = (int)min<int64_t>(N_cap - 1 - j0, (int64_t)kPfChunk - 1);
  auto issue = [&](int blk, uint8_t* dst) {
#pragma unroll
    for (int u = 0; u < kPfLoads; ++u) {
      const int lam = wave * kPfLoads + u;
      const int r = 8 * lam + lane / 8;
      const int row = min(blk * kPfBlk + r, last_row);
      const uint8_t* src = kchunk + (uint32_t)(row * kPfDim + 16 * ((lane % 8) ^ swz(r)));
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (__attribute__((address_space(3))) void*)(dst + lam * 1024), 16, 0, 0);
    }
  };
  issue(0, s_k0);
  if (nblk > 1) issue(1, s_k1);

  // The wave's queries i0 + 2*wave + {0, 1} (past Lq: the group's first
  // query, never stored). A operand of tile mt, k-step s: lane l gives row
  // p = l%32 (query (p/4)%2, head 16mt + 4(p/8) + p%4), bytes 64s + 32(l/32).
  auto qrow_of = [&](int qq) {
    const int i = 2 * wave + qq;
    return (int64_t)b * Lq + i0 + (i < nq ? i : 0);
  };
  i32x8 qa[4][2];
  {
    const int p = n32;
    const int64_t qr = qrow_of((p / 4) % 2);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int h = 16 * mt + 4 * (p / 8) + p % 4;
        const uint8_t* src = q_i + (qr * kPfHeads + h) * kPfDim + 64 * s + 32 * half;
        const uint4 x0 = *reinterpret_cast<const uint4*>(src);
        const uint4 x1 = *reinterpret_cast<const uint4*>(src + 16);
        qa[mt][s] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      }
  }
  // Accumulator register e of tile mt holds row 8(e/4) + 4*half + e%4, which
  // is head 16mt + e of the lane's own query (= half).
  float wr[4][16];
  {
    const int64_t qr = qrow_of(half);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 w4 = *reinterpret_cast<const float4*>(w_i + qr * kPfHeads + 16 * mt + 4 * a4);
        wr[mt][4 * a4] = w4.x; wr[mt][4 * a4 + 1] = w4.y; wr[mt][4 * a4 + 2] = w4.z; wr[mt][4 * a4 + 3] = w4.w;
      }
  }
  const int my_q = 2 * wave + half;
  const int lim = my_q < nq ? (int)min<int64_t>((q_pos0 + i0 + my_q + 1) / m - j0, (int64_t)kPfChunk) : -1;
  const uint32_t ulim = (uint32_t)max(lim, 0);

  // Score stores relative to (row i0 + 2*wave, entry j0); the lane's row is
  // that + half. Offsets past the resource's end are dropped.
  // bf16 scores (sbf): rows of score_stride(N_cap, 1) entries, each lane
  // pair's word stored by its even lane; every lane still issues one store.
  const int esz = sbf ? 2 : 4;
  const int64_t sstride = score_stride(N_cap, sbf);
  const uint64_t sbase = (uint64_t)((uint8_t*)scores + (((int64_t)b * Lq + i0 + 2 * wave) * sstride + j0) * esz);
  const uint32_t slo = __builtin_amdgcn_readfirstlane((uint32_t)sbase);
  const uint32_t shi = __builtin_amdgcn_readfirstlane((uint32_t)(sbase >> 32));
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(((uint64_t)shi << 32) | slo), 0, (int)((sstride + kPfChunk) * esz), 0x00020000);
  constexpr int kDrop = 0x7FFFFFF0;
  const int row_off = half ? (int)(sstride * esz) : 0;
  const bool s_lane = !sbf || (lane & 1) == 0;

  // B fragments of step st of an LDS block (two k-steps, entries 32st..+31).
  auto frags = [&](const uint8_t* kt, int st, i32x8 (&kf)[2]) {
    const int r = 32 * st + n32;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int p0 = (4 * s + 2 * half) ^ swz(r);
      const uint4 x0 = *reinterpret_cast<const uint4*>(kt + r * kPfDim + 16 * p0);
      const uint4 x1 = *reinterpret_cast<const uint4*>(kt + r * kPfDim + 16 * (p0 ^ 1));
      kf[s] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
  };
  auto mma = [&](const i32x8 (&kf)[2], f32x16 (&acc)[4]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][e] = 0.f;
#pragma unroll
      for (int s = 0; s < 2; ++s)
        acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mt][s], kf[s], acc[mt], 0, 0, 0, 127, 0,
                                                                    127);
    }
  };
  // ReLU + weights + sum over the lane's 64 heads in four independent
  // chains, and one store of 2 x 32 scores (step g of the chunk).
  auto epi = [&](const f32x16 (&acc)[4], int g) {
    float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) p[e % 4] = fmaf(wr[mt][e], relu_bits(acc[mt][e]), p[e % 4]);
    const float tot = (p[0] + p[1]) + (p[2] + p[3]);
    const int jrel = g * 32 + n32;
    const uint32_t word = score_word(tot, sbf);
    const int off = (uint32_t)jrel < ulim && s_lane ? row_off + jrel * esz : kDrop;
    __builtin_amdgcn_raw_buffer_store_b32(word, srsrc, off, 0, 0);
  };

  // Step order: MFMAs of step g, LDS reads of step g+1 into the same
  // fragment registers (the MFMAs have read them), epilogue of step g while
  // those reads land. Between the MFMAs and the epilogue of a block's last
  // step sits the hand-over to the next block: wait for its copies, barrier,
  // start the copy of the block three ahead into the buffer just finished,
  // read the next block's first fragments. The issue order after block x's
  // copies is: 8 stores, the copies of block x+1, 8 more stores, so waiting
  // down to kPfLoads + kPfStores outstanding operations covers block x and
  // leaves x+1 in flight. Copies, waits and the hand-over are unconditional
  // (past the last block the copy repeats it into a free buffer and the
  // fragment read is unused), so the compiler's own wait analysis sees the
  // same counts on every path and adds none.
  // The two waves of a SIMD (waves w and w + 4) run half a step apart: the
  // second half of the waves does its block hand-over after the last
  // epilogue instead of before it, so right after every barrier one wave of
  // each pair runs an epilogue (VALU) while the other runs MFMAs, and the
  // two stay in alternation through the block instead of contending for the
  // same unit at the same time.
  auto run = [&](auto late_c) {
    constexpr bool late = decltype(late_c)::value;
    i32x8 kf[2];
    f32x16 acc[4];
    auto handover = [&](int blk, const uint8_t* kt, const uint8_t* kt_next) {
      __builtin_amdgcn_s_waitcnt(pf_vmcnt(kPfLoads + kPfStores));
      pf_lds_barrier();  // block blk+1 is in LDS; every wave is done with block blk
      issue(min(blk + 3, nblk - 1), const_cast<uint8_t*>(kt));
      frags(kt_next, 0, kf);
    };
    auto block = [&](int blk, const uint8_t* kt, const uint8_t* kt_next) {
#pragma unroll
      for (int st = 0; st < kPfSteps; ++st) {
        mma(kf, acc);
        if (st + 1 < kPfSteps)
          frags(kt, st + 1, kf);
        else if (!late)
          handover(blk, kt, kt_next);
        // Nothing crosses these points: the reads stay right behind the MFMAs
        // (the scheduler would sink them to the end of the epilogue and expose
        // their latency), and the next step's MFMAs stay behind this epilogue
        // (hoisted above it they would need a second accumulator set).
        __builtin_amdgcn_sched_barrier(0);
        epi(acc, blk * kPfSteps + st);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    __builtin_amdgcn_s_waitcnt(0);
    pf_lds_barrier();  // blocks 0 and 1 are in LDS
    issue(min(2, nblk - 1), s_k2);
    frags(s_k0, 0, kf);
    if constexpr (!late) {
      for (int blk = 0;;) {
        block(blk, s_k0, s_k1);
        if (++blk >= nblk) break;
        block(blk, s_k1, s_k2);
        if (++blk >= nblk) break;
        block(blk, s_k2, s_k0);
        if (++blk >= nblk) break;
      }
    } else {
      // the hand-over of block blk - 1 opens block blk (the loop's back edge
      // then follows an epilogue's store, as in the other order), and a last
      // barrier matches the other waves' count
      block(0, s_k0, s_k1);
      for (int blk = 1; blk < nblk;) {
        handover(blk - 1, s_k0, s_k1);
        block(blk, s_k1, s_k2);
        if (++blk >= nblk) break;
        handover(blk - 1, s_k1, s_k2);
        block(blk, s_k2, s_k0);
        if (++blk >= nblk) break;
        handover(blk - 1, s_k2, s_k0);
        block(blk, s_k0, s_k1);
        ++blk;
      }
      pf_lds_barrier();
    }
  };
  if (wave < kPfWaves / 2)
    run(std::false_type{});
  else
    run(std::true_type{});
  __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS outlives the workgroup
}

}  // namespace

bool index_qk_prefill_eligible(int fmt, int H_i, int d_i, int Lq) {
  return fmt == 2 && H_i == kPfHeads && d_i == kPfDim && Lq >= kPfQ;
}

int launch_index_qk_prefill(int B, int Lq, int64_t q_pos0, const int64_t* q_pos, int m, int64_t N_cap,
                            const void* q_i, const float* w_i, const void* k_i, float* scores, int sbf,
                            hipStream_t stream) {
  const int64_t n_max = (q_pos0 + Lq) / m;
  const int nchunks = (int)((n_max + kPfChunk - 1) / kPfChunk);
  const int ngroups = (Lq + kPfQ - 1) / kPfQ;
  if (nchunks == 0 || B == 0 || Lq == 0) return 0;
  const dim3 grid((unsigned)((int64_t)B * ngroups * nchunks));
  if (sbf)
    hipLaunchKernelGGL(index_qk_prefill_kernel<true>, grid, dim3(kPfWaves * kWave), 0, stream, Lq, q_pos0, q_pos, m,
                       N_cap, ngroups, nchunks, (const uint8_t*)q_i, w_i, (const uint8_t*)k_i, scores);
  else
    hipLaunchKernelGGL(index_qk_prefill_kernel<false>, grid, dim3(kPfWaves * kWave), 0, stream, Lq, q_pos0, q_pos, m,
                       N_cap, ngroups, nchunks, (const uint8_t*)q_i, w_i, (const uint8_t*)k_i, scores);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace csa
