// finalize.hip -- EP finalize, rank combine and expert-TP finalize (gfx950).
//
// The arithmetic is the MoE tail's ([tail] = the Muse Spark moe.tail page:
// module docstring formulas; _TpTailKernel with its helpers gains,
// warp_sum_of_squares and normalized; _TailReduceKernel):
//
//   g   = fp32(gamma) + gain_center                      (FP32 add)
//   s   = x * g  with weight_before_norm, else x
//   ss  = sum of squares of s in the fixed tree below
//   inv = 1 / sqrt(ss * fp32(1/P) + eps)
//   n   = s * inv  with weight_before_norm, else (x * inv) * g
//   p   = n * w    (each product rounded on its own)
//   sum p over routes in ascending order from +0.0, BF16 round-to-nearest-
//   even, -0 written as +0; ranks combined in rank order from +0.0.
//
// Sum-of-squares tree (one band of the pages' warp tree, widened to wave64):
// a row is cut into blocks of 512 columns; within a block, lane l owns the
// 8 columns 512 j + 8 l .. + 7 and adds their squares one by one from 0;
// a wave-wide xor butterfly gives every lane the block total; block totals
// are added in ascending block order from 0.
//
// Everything here is HBM-bound streaming: 16-byte loads, each wave-wide load
// instruction reading 1 KB of one row contiguously.
#include "common.h"
#include "kernels.h"
#include "finalize_device.h"
#include "norm_device.h"

namespace moetail {

namespace {

// ------------------------------------------------------- finalize kernel -
//
// One block per token t, one wave per 512-column block of the row (P <= 8192:
// at most 16 waves); lane l of wave j owns columns 512 j + 8 l .. + 7.
//
//  1. Wave 0 lists the token's local (rank, route) pairs in rank order and,
//     within a rank, in ascending route order, with their row and weight, in
//     LDS (all index loads in flight at once, one ballot per 64 entries).
//  2. The pairs are taken in batches of kSlots (one LDS read hands lane s
//     pair s; the rest are lane reads): every wave loads its chunk of
//     every row of the batch at once (one memory round trip per batch), adds
//     its squares (the gains first with weight_before_norm) and reduces them
//     across the wave; the block shares meet in LDS.
//  3. After a barrier each pair's inverse RMS is the in-order sum of its
//     block shares; the waves walk the batch's pairs in order, adding the
//     weighted normalized products into the current rank's FP32 partial.
//     When the walk passes the last route of a rank, that rank's partial is
//     rounded to BF16 (-0 as +0), stored if asked, and added in rank order
//     into the combined row; ranks without local routes give +0 partials.
constexpr int kMaxPairs = MOETAIL_KMAX_PAIRS;

struct FinArgs {
  const uint16_t* rows;
  int64_t R;            // rows per rank (EP)
  const int32_t* idx;   // [tp][b][K]
  int64_t idx_limit;    // a route is present when 0 <= idx < idx_limit
  const void* w;        // [b][K]
  const uint16_t* gamma;
  float gain_center, eps;
  int b, K, P, tp;
  uint16_t* partials;   // [tp][b][P] or null
  uint16_t* out;        // [b][P] or null
  int wpq;              // waves per column group: block (t, q) forms the
                        // products of waves [q * wpq, (q + 1) * wpq)
};

struct Pair {
  long long row;  // row index into `rows` (units of P elements)
  float w;
  int rank;
};

// kSlots rows in flight per lane: 16 when the block has at most 8 waves
// (256 VGPRs per lane), 8 for wider rows (up to 16 waves, 128 VGPRs).
template <int MODE, bool WBF16, int kSlots, int kMaxThreads>
__global__ void __launch_bounds__(kMaxThreads) finalize_kernel(FinArgs a) {
  __shared__ Pair pairs[kMaxPairs];
  __shared__ float block_ss[kSlots][16];
  __shared__ int pair_count;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nwaves = (a.P + kBlockCols - 1) / kBlockCols;  // the block: a wave per 512 columns
  const int t = blockIdx.x;
  const int P = a.P;
  // Every block of token t takes the whole row's sums of squares; only the
  // waves of its column group go on to the products.
  const bool prod = wave / a.wpq == (int)blockIdx.y;  // wave-uniform

  // Wave 0 lists the local (rank, route) pairs.  Entry e = d * K + k (rank
  // major, route minor: the order of the sums); lane l holds entries l,
  // l + 64, ...; every index load is in flight at once, and a ballot per
  // group of 64 entries places each local pair.
  const int col = (wave * kWave + lane) * kChunk;
  const bool has = col < P;
  const int colc = has ? col : P - kChunk;  // lanes past the row read a valid chunk
  const uint4 gq = MODE != kNoNorm ? load16(a.gamma + colc) : make_uint4(0, 0, 0, 0);
  if (wave == 0) {
    const int nent = a.tp * a.K;
    const int ngroups = (nent + kWave - 1) / kWave;
    const float wk = lane < a.K ? load_weight<WBF16>(a.w, (int64_t)t * a.K + lane) : 0.0f;
    int rr[kMaxPairs / kWave];
#pragma unroll
    for (int q = 0; q < kMaxPairs / kWave; ++q) {
      rr[q] = -1;
      const int e = kWave * q + lane;
      if (q < ngroups && e < nent) {
        const int d = e / a.K, k = e - d * a.K;
        rr[q] = a.idx[((int64_t)d * a.b + t) * a.K + k];
      }
    }
    int base = 0;
#pragma unroll
    for (int q = 0; q < kMaxPairs / kWave; ++q) {
      if (q < ngroups) {
        const int e = min(kWave * q + lane, nent - 1);
        const int d = e / a.K, k = e - d * a.K;
        const float wsel = __shfl(wk, k, kWave);
        const bool local = kWave * q + lane < nent && rr[q] >= 0 && (int64_t)rr[q] < a.idx_limit;
        const uint64_t m = __ballot(local);
        if (local) {
          const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
          const long long row = (long long)d * a.R + rr[q];
          pairs[pos] = Pair{row, wsel, d};
        }
        base += __popcll(m);
      }
    }
    if (lane == 0) pair_count = base;
  }
  __syncthreads();
  const int np = __builtin_amdgcn_readfirstlane(pair_count);

  float g[8];
  unpack8(gq, g);
#pragma unroll
  for (int c = 0; c < 8; ++c) g[c] = g[c] + a.gain_center;
  const float inv_width = (float)(1.0 / (double)P);

  float acc[8], comb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = comb[e] = 0.0f;
  int next_rank = 0;  // ranks below this one have been emitted
  auto emit_through = [&](int end_rank) {
    while (next_rank < end_rank) {
      const uint4 q = pack8_pz(acc);
      if (has && a.partials) store16(a.partials + ((int64_t)next_rank * a.b + t) * P + col, q);
      float v[8];
      unpack8(q, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        comb[e] = comb[e] + v[e];
        acc[e] = 0.0f;
      }
      ++next_rank;
    }
  };

  for (int base = 0; base < np; base += kSlots) {
    const int nb = min(kSlots, np - base);
    // Lane s < kSlots holds pair base + s (one LDS read for the batch).
    Pair mine = Pair{0, 0.0f, 0};
    if (lane < kSlots) mine = pairs[base + min(lane, nb - 1)];
    const int row_lo = (int)(mine.row & 0xffffffffll), row_hi = (int)(mine.row >> 32);
    uint4 xq[kSlots];
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      const long long row =
          (long long)(((uint64_t)(uint32_t)readlane_i(row_hi, s) << 32) | (uint32_t)readlane_i(row_lo, s));
      xq[s] = load16(a.rows + row * P + colc);
    }
    // All slots reduce without branches (slots past nb repeat the last
    // pair and are never used), so the slots' butterflies interleave.
    float my_inv = 0.0f;
    if (MODE != kNoNorm) {
      float ss[kSlots];
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        ss[s] = has ? chunk_ss<MODE>(xq[s], g) : 0.0f;
        ss[s] = wave_butterfly_sum(ss[s]);
      }
      if (lane == 0) {
#pragma unroll
        for (int s = 0; s < kSlots; ++s)
          if (s < nb) block_ss[s][wave] = ss[s];
      }
      __syncthreads();
      if (lane < nb) {
        float total = 0.0f;
        for (int j = 0; j < nwaves; ++j) total = total + block_ss[lane][j];
        my_inv = inv_rms(total, inv_width, a.eps);
      }
    }
    if (prod) {
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        if (s < nb) {
          emit_through(readlane_i(mine.rank, s));
          const float inv = readlane_f(my_inv, s);
          add_products<MODE>(xq[s], g, inv, readlane_f(mine.w, s), acc);
        }
      }
    }
    if (MODE != kNoNorm) __syncthreads();  // block_ss is refilled by the next batch
  }
  if (!prod) return;
  emit_through(a.tp);
  if (has && a.out) store16(a.out + (int64_t)t * P + col, pack8_pz(comb));
}

// Column groups per token: enough blocks for one per CU (a block holds
// a CU: up to 16 waves of up to 209 VGPRs), at most one group per wave.
template <int MODE, bool WBF16>
hipError_t finalize_launch(FinArgs a, hipStream_t s) {
  const int nwaves = (a.P + kBlockCols - 1) / kBlockCols;
  const int want = (device_cu_count() + a.b - 1) / a.b;
  const int groups = want < 1 ? 1 : want > nwaves ? nwaves : want;
  a.wpq = (nwaves + groups - 1) / groups;
  const dim3 grid(a.b, (nwaves + a.wpq - 1) / a.wpq);
  if (nwaves <= 8)
    hipLaunchKernelGGL((finalize_kernel<MODE, WBF16, 16, 512>), grid, dim3(kWave * nwaves), 0, s,
                       a);
  else
    hipLaunchKernelGGL((finalize_kernel<MODE, WBF16, 8, 1024>), grid, dim3(kWave * nwaves), 0, s,
                       a);
  return hipGetLastError();
}

hipError_t finalize_dispatch(const FinArgs& a, int mode, bool w_bf16, hipStream_t s) {
  switch (mode * 2 + (w_bf16 ? 1 : 0)) {
    case 0: return finalize_launch<kGainAfter, false>(a, s);
    case 1: return finalize_launch<kGainAfter, true>(a, s);
    case 2: return finalize_launch<kGainFirst, false>(a, s);
    case 3: return finalize_launch<kGainFirst, true>(a, s);
    case 4: return finalize_launch<kNoNorm, false>(a, s);
    case 5: return finalize_launch<kNoNorm, true>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------ per-rank finalize -----
//
// The same arithmetic when only the rank partials are asked for: one block
// per (token t, rank d), one wave per 512-column block.  Each wave lists the
// rank's local routes itself (lane k < K reads idx[d][t][k]; one ballot;
// the set bits in ascending order are the routes in the order of the sum),
// so no LDS pass or barrier precedes the row loads.  A block reads only its
// rank's rows, so a token's rows spread over tp blocks.  The partial is the
// fused kernel's bit for bit: the same chunks, tree, inverse and route order.
template <int MODE, bool WBF16, int kSlots, int kMaxThreads>
__global__ void __launch_bounds__(kMaxThreads) rank_finalize_kernel(FinArgs a) {
  __shared__ float block_ss[kSlots][16];
  const RankUnit u{a.rows, a.R, a.idx, a.idx_limit, a.w, a.gamma, a.gain_center, a.eps,
                   a.b, a.K, a.P, a.partials};
  rank_partial<MODE, WBF16, kSlots>(u, blockIdx.x, blockIdx.y, block_ss);
}

// out[t] = bf16(sum over ranks, in rank order from +0, of partials[d][t]),
// -0 as +0; one thread per 8 columns of a token, every rank's load in
// flight at once.
__global__ void __launch_bounds__(256) rank_combine_kernel(const uint16_t* partials, int tp, int b,
                                                           int P, uint16_t* out) {
  const int per_tok = P / kChunk;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // blocks of 256
  if (i >= (int64_t)b * per_tok) return;
  const int t = (int)(i / per_tok);
  const int col = (int)(i - (int64_t)t * per_tok) * kChunk;
  const uint16_t* src = partials + (int64_t)t * P + col;
  const int64_t rank_stride = (int64_t)b * P;
  float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int d0 = 0; d0 < tp; d0 += 8) {
    uint4 q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) q[u] = load16(src + min(d0 + u, tp - 1) * rank_stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (d0 + u < tp) {
        float v[8];
        unpack8(q[u], v);
#pragma unroll
        for (int c = 0; c < 8; ++c) sum[c] = sum[c] + v[c];
      }
    }
  }
  store16(out + (int64_t)t * P + col, pack8_pz(sum));
}

// Rows in flight per batch: the expected local routes of a rank (K / tp),
// as 4, 8 or 16 slots (8 at most for rows wider than 4096 columns, whose
// 16-wave blocks leave 128 VGPRs a lane); a rank holding more takes more
// batches.
template <int MODE, bool WBF16>
hipError_t rank_finalize_launch(const FinArgs& a, hipStream_t s) {
  const int nwaves = (a.P + kBlockCols - 1) / kBlockCols;
  const int expect = (a.K + a.tp - 1) / a.tp;
  const dim3 grid(a.b, a.tp), block(kWave * nwaves);
  if (nwaves <= 8) {
    if (expect <= 4)
      hipLaunchKernelGGL((rank_finalize_kernel<MODE, WBF16, 4, 512>), grid, block, 0, s, a);
    else if (expect <= 8)
      hipLaunchKernelGGL((rank_finalize_kernel<MODE, WBF16, 8, 512>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((rank_finalize_kernel<MODE, WBF16, 16, 512>), grid, block, 0, s, a);
  } else {
    if (expect <= 4)
      hipLaunchKernelGGL((rank_finalize_kernel<MODE, WBF16, 4, 1024>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((rank_finalize_kernel<MODE, WBF16, 8, 1024>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t rank_finalize_dispatch(const FinArgs& a, int mode, bool w_bf16, hipStream_t s) {
  switch (mode * 2 + (w_bf16 ? 1 : 0)) {
    case 0: return rank_finalize_launch<kGainAfter, false>(a, s);
    case 1: return rank_finalize_launch<kGainAfter, true>(a, s);
    case 2: return rank_finalize_launch<kGainFirst, false>(a, s);
    case 3: return rank_finalize_launch<kGainFirst, true>(a, s);
    case 4: return rank_finalize_launch<kNoNorm, false>(a, s);
    case 5: return rank_finalize_launch<kNoNorm, true>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// --------------------------------------------------- expert-TP rank sum --
//
// The K-partials are read once: non-temporal loads (streamed past the
// caches), which keep the rank-summed rows cached for the second pass
// (measured at b=128, P=7168: 61.3 -> 59.0 us).
// x_r = bf16(sum over ranks, in rank order from +0, of the route's
// K-partials), one wave per (route, 512-column block): pure streaming with
// every rank's chunk in flight at once.  The wave also forms its block's
// share of the route's sum of squares -- lane l adds the squares of its 8
// columns of s (x_r, or x_r * g with the gain first) from 0, a wave
// butterfly gives the block total: the tree's first two levels, so the
// second pass adds 512-column block totals only.  Absent routes are skipped
// (the second pass never reads them).
__global__ void __launch_bounds__(256) tp_rank_sum_kernel(const uint16_t* kpart, int64_t num_rows,
                                                          const int32_t* idx, int routes, int P,
                                                          int tp, uint16_t* xr,
                                                          const uint16_t* gamma, float gain_center,
                                                          int gain_first, float* block_total) {
  const int nbk = (P + kBlockCols - 1) / kBlockCols;
  const int64_t wid = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;  // blocks of 4 waves
  if (wid >= (int64_t)routes * nbk) return;
  const int route = (int)(wid / nbk);
  const int j = (int)(wid - (int64_t)route * nbk);
  const int r = idx[route];
  if (r < 0 || (int64_t)r >= num_rows) return;  // wave-uniform
  const int lane = threadIdx.x & (kWave - 1);
  const int col = (j * kWave + lane) * kChunk;
  const bool has = col < P;
  const int colc = has ? col : P - kChunk;  // lanes past the row read a valid chunk
  const uint16_t* src = kpart + (int64_t)r * P + colc;
  const int64_t rank_stride = num_rows * (int64_t)P;
  float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  int d = 0;
  for (; d + 8 <= tp; d += 8) {
    uint4 q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) q[u] = load16_stream(src + (d + u) * rank_stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float v[8];
      unpack8(q[u], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
    }
  }
  for (; d < tp; ++d) {
    float v[8];
    unpack8(load16_stream(src + d * rank_stride), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
  }
  const uint4 q = pack8(sum);
  if (has) store16(xr + (int64_t)route * P + col, q);
  float g[8];
  unpack8(load16(gamma + colc), g);
#pragma unroll
  for (int c = 0; c < 8; ++c) g[c] = g[c] + gain_center;
  float ss = 0.0f;
  if (has) ss = gain_first ? chunk_ss<kGainFirst>(q, g) : chunk_ss<kGainAfter>(q, g);
  ss = wave_butterfly_sum(ss);
  if (lane == 0) block_total[(int64_t)route * nbk + j] = ss;
}

// The expert-TP finalize's second pass: one thread per 8 columns of a
// token, blocks of 256 threads over one token's columns.  Every thread first
// loads its chunk of every route row (the rank-summed rows sit at fixed
// places in the workspace, absent routes included, so the loads need no
// index); meanwhile wave 0's lane k forms route k's inverse RMS from the
// route's block totals (added in column order from 0).  Then the weighted
// normalized products of the present routes are added in route order from
// +0.
template <int MODE, bool WBF16>
__global__ void __launch_bounds__(256) tp_norm_kernel(const uint16_t* xr, const int32_t* idx,
                                                      int64_t num_rows, const void* w,
                                                      const uint16_t* gamma, float gain_center,
                                                      float eps, int K, int P,
                                                      const float* block_total, uint16_t* out) {
  __shared__ float inv_s[MOETAIL_MAX_ROUTES];
  __shared__ float w_s[MOETAIL_MAX_ROUTES];
  __shared__ int present_s[MOETAIL_MAX_ROUTES];
  const int t = blockIdx.y;
  const int nbk = (P + kBlockCols - 1) / kBlockCols;
  const int col = (blockIdx.x * 256 + threadIdx.x) * kChunk;
  const bool has = col < P;
  const int colc = has ? col : P - kChunk;  // threads past the row read a valid chunk
  const uint16_t* src = xr + (int64_t)t * K * P + colc;
  uint4 q[MOETAIL_MAX_ROUTES];
#pragma unroll
  for (int k = 0; k < MOETAIL_MAX_ROUTES; ++k)
    if (k < K) q[k] = load16(src + (int64_t)k * P);
  const uint4 gq = load16(gamma + colc);
  if (threadIdx.x < (unsigned)K) {
    const int k = threadIdx.x;
    // The route's index, its block totals (P <= 8192: at most 16) and its
    // weight are loaded at once: the totals sit at a fixed place whether or
    // not the route is present (an absent route's are never used).
    const int r = idx[(int64_t)t * K + k];
    const float* bt = block_total + ((int64_t)t * K + k) * nbk;
    float v[MOETAIL_MAX_WIDTH / kBlockCols];
#pragma unroll
    for (int j = 0; j < MOETAIL_MAX_WIDTH / kBlockCols; ++j) v[j] = j < nbk ? bt[j] : 0.0f;
    const float wk = load_weight<WBF16>(w, (int64_t)t * K + k);
    const bool present = r >= 0 && (int64_t)r < num_rows;
    float inv = 0.0f;
    if (present) {
      float total = 0.0f;  // in column order from 0
#pragma unroll
      for (int j = 0; j < MOETAIL_MAX_WIDTH / kBlockCols; ++j)
        if (j < nbk) total = total + v[j];
      inv = inv_rms(total, (float)(1.0 / (double)P), eps);
    }
    inv_s[k] = inv;
    w_s[k] = wk;
    present_s[k] = present;
  }
  __syncthreads();
  if (!has) return;
  float g[8];
  unpack8(gq, g);
#pragma unroll
  for (int c = 0; c < 8; ++c) g[c] = g[c] + gain_center;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < MOETAIL_MAX_ROUTES; ++k)
    if (k < K && present_s[k]) add_products<MODE>(q[k], g, inv_s[k], w_s[k], acc);
  store16(out + (int64_t)t * P + col, pack8_pz(acc));
}

// ------------------------------------------------ expert-TP in one pass --
//
// Two blocks per token (its columns in two halves of 512-column blocks),
// one wave per 512 columns, so that the 235 MB of K-partials stream through
// every CU (measured: a plain read of that size reaches 6.4 TB/s with 256
// blocks of 7 waves, 5.4 TB/s with 128 blocks of 14).  x_r never leaves the
// chip: a wave streams the routes in order, two routes' loads ahead, and
// holds each route's rank sums only until that route's products are added.
//
// A route's inverse RMS needs the whole row's sum of squares, i.e. the
// 512-column block totals of every wave of both blocks.  Each wave writes its
// block total of route k, as soon as it has it, to a mailbox slot: one 64-bit
// word (tag << 32 | FP32 bits), written and read whole, so no fence orders
// it.  Two routes later the wave polls the row's slots of route k (the poll
// issued before the next stream loads, read one route after), adds the totals
// in column order from 0 (the same tree and bits as the two-pass path), and
// adds route k's weighted normalized products.  The exchange overlaps the
// stream instead of following it.
//
// The tag is the token's generation (read at the start, plus one); every
// wave raises the generation to its tag at the end, so a later call's tag is
// above every slot an earlier call left (the workspace is zero before its
// first use).  A wait is bounded: a wave whose slots are not all there
// within the limit forms the missing block totals itself from the
// K-partials (slower, the same bits), and from then on waits no more.  No
// barrier and no fence: no result depends on two blocks running at once.
struct TpMailArgs {
  const uint16_t* kpart;  // [tp][num_rows][P]
  int64_t num_rows;
  const int32_t* idx;     // [b][K]
  const void* w;          // [b][K]
  const uint16_t* gamma;  // [P]
  float gain_center, eps;
  int K, P, tp;
  uint16_t* out;          // [b][P]
  unsigned* gen;          // [b]: each token's generation
  uint64_t* slots;        // [b][KMAX][ceil(P/512)]: (tag << 32) | FP32 block total
                          // (KMAX = 16 for K <= 16, else 32; every slot written each call)
  int wpb;                // waves per block: block x takes column blocks x * wpb ..
  long long wait_ticks;   // wait limit in 100 MHz ticks; < 0: do not wait
};

// A row of zeros as wide as the widest row: the chunks of the ranks past tp.
__device__ uint4 tp_zero_row[MOETAIL_MAX_WIDTH / kChunk];

// One route's K-partial chunks of the 8 columns at colc, every rank's load
// in flight (tp <= 8; ranks past tp read zeros, whose +0 changes no sum:
// the sums start at +0 and are never -0).  Issued whether or not the route
// is there -- an absent one reads the gamma chunk instead, a cache hit -- so
// the loads in flight stay countable and the wait for one route never
// drains the loads ahead of it.
__device__ __forceinline__ void tp_issue(const TpMailArgs& a, bool there, int r, int colc,
                                         uint4 (&q)[8]) {
  const uint16_t* src = there ? a.kpart + (int64_t)r * a.P + colc : a.gamma + colc;
  const int64_t rank_stride = there ? a.num_rows * (int64_t)a.P : 0;
  const uint16_t* zeros = reinterpret_cast<const uint16_t*>(tp_zero_row) + colc;
#pragma unroll
  for (int u = 0; u < 8; ++u) q[u] = load16_stream(u < a.tp ? src + u * rank_stride : zeros);
}

// x_r = bf16(sum over ranks, in rank order from +0).
__device__ __forceinline__ uint4 tp_rank_sum(const uint4 (&q)[8]) {
  float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float v[8];
    unpack8(q[u], v);
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
  }
  return pack8(sum);
}

// The 512-column block total of route row r over column block jj, formed by
// one wave from the K-partials (for a block total whose slot did not come).
template <int MODE>
__device__ __forceinline__ float tp_block_total(const TpMailArgs& a, int r, int jj) {
  const int lane = threadIdx.x & (kWave - 1);
  const int col = (jj * kWave + lane) * kChunk;
  const bool has = col < a.P;
  const int colc = has ? col : a.P - kChunk;
  uint4 q[8];
  tp_issue(a, true, r, colc, q);
  float g[8];
  unpack8(load16(a.gamma + colc), g);
#pragma unroll
  for (int c = 0; c < 8; ++c) g[c] = g[c] + a.gain_center;
  const uint4 x = tp_rank_sum(q);
  return wave_butterfly_sum(has ? chunk_ss<MODE>(x, g) : 0.0f);
}

// The slow path of a poll: the slots of one route (ms[0 .. nbk)) that are
// not there are read again until `limit` ticks have passed (then `limit`
// becomes -1: no more waiting), and any still missing are formed from the
// K-partials of route row r.  v: this lane's read of slot `lane`; returns
// the lane's slot as a complete read has it.
template <int MODE>
__device__ __forceinline__ uint64_t tp_wait_slots(const TpMailArgs& a, const uint64_t* ms,
                                                  int nbk, unsigned tag, int r, uint64_t v,
                                                  long long& limit) {
  const int lane = threadIdx.x & (kWave - 1);
  bool ready = lane >= nbk || (unsigned)(v >> 32) == tag;
  if (limit >= 0) {
    const long long t0 = wall_clock64();
    while (__ballot(!ready)) {
      if (wall_clock64() - t0 > limit) {
        limit = -1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      if (!ready) {
        v = __hip_atomic_load(ms + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ready = (unsigned)(v >> 32) == tag;
      }
    }
  }
  uint64_t missing = __ballot(!ready);
  while (missing) {
    const int jj = __builtin_ctzll(missing);
    missing &= missing - 1;
    const float tot = tp_block_total<MODE>(a, r, jj);
    if (lane == jj) v = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(tot);
  }
  return v;
}

constexpr int kTpMaxAhead = 4;  // most routes a wave's loads run ahead

// A wave's state through the stream: route k's loads in q[k % (ahead + 1)], its rank
// sums in xr[k] until its products are added, the FP32 sums, and the slot
// read polled last.
template <int KMAX>
struct TpWave {
  int lane, j, col, colc, nbk, e;
  bool has;
  float wk;
  uint64_t present;
  unsigned tag;
  uint64_t* tslots;
  long long limit;
  float g[8];
  uint4 q[kTpMaxAhead + 1][8];  // route k's loads in q[k % (ahead + 1)]
  uint4 xr[KMAX];
  float acc[8];
  uint64_t poll;
};

// Step k of the stream (template recursion, so every k is a constant and the
// state stays in registers): poll route k - kLag, issue route k + kAhead's
// loads, add route k's ranks and publish its block total, then add route
// k - kLag - 1's products (its poll came in with route k's loads).
template <int MODE, int KMAX, int kAhead, int k>
__device__ __forceinline__ void tp_step(const TpMailArgs& a, TpWave<KMAX>& w) {
  constexpr int kLag = 2;    // routes between a slot's write and its poll
  // Every memory operation below is issued on every path (routes that are
  // not there use stand-in data and a slot of their own): only arithmetic
  // depends on which routes are there.
  constexpr int mp = k - kLag;
  uint64_t next_poll = 0;
  if (mp >= 0 && mp < KMAX)
    next_poll = __hip_atomic_load(w.tslots + (int64_t)(mp < 0 ? 0 : mp) * w.nbk +
                                      min(w.lane, w.nbk - 1),
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (k + kAhead < KMAX) {
    constexpr int kn = k + kAhead < KMAX ? k + kAhead : 0;
    tp_issue(a, (w.present >> kn) & 1ull, readlane_i(w.e, kn), w.colc, w.q[kn % (kAhead + 1)]);
  }
  if (k < KMAX) {
    constexpr int kk = k < KMAX ? k : 0;
    const uint4 x = tp_rank_sum(w.q[kk % (kAhead + 1)]);
    w.xr[kk] = x;
    const float tot = wave_butterfly_sum(w.has ? chunk_ss<MODE>(x, w.g) : 0.0f);
    // lane 0 stores the wave's total (64 lanes writing one word would be 64
    // writes; one lane's store under the exec mask is still counted)
    if (w.lane == 0)
      __hip_atomic_store(w.tslots + (int64_t)kk * w.nbk + w.j,
                         ((uint64_t)w.tag << 32) | (uint64_t)__float_as_uint(tot),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  constexpr int m = k - kLag - 1;
  if (m >= 0 && m < KMAX && ((w.present >> (m < 0 ? 0 : m)) & 1ull)) {
    constexpr int mm = m < 0 ? 0 : m;
    uint64_t v = w.poll;
    const bool ready = (unsigned)(v >> 32) == w.tag;
    if (__ballot(!ready))
      v = tp_wait_slots<MODE>(a, w.tslots + (int64_t)mm * w.nbk, w.nbk, w.tag,
                              readlane_i(w.e, mm), v, w.limit);
    const float mine = __uint_as_float((unsigned)v);
    float total = 0.0f;  // block totals in column order from 0
#pragma unroll
    for (int jj = 0; jj < MOETAIL_MAX_WIDTH / kBlockCols; ++jj)
      if (jj < w.nbk) total = total + readlane_f(mine, jj);
    const float inv = inv_rms(total, (float)(1.0 / (double)a.P), a.eps);
    add_products<MODE>(w.xr[mm], w.g, inv, readlane_f(w.wk, mm), w.acc);
  }
  w.poll = next_poll;
  if constexpr (k + 1 < KMAX + kLag + 1) tp_step<MODE, KMAX, kAhead, k + 1>(a, w);
}

template <int MODE, bool WBF16, int KMAX, int kAhead>
__global__ void __launch_bounds__(512) tp_mail_kernel(TpMailArgs a) {
  TpWave<KMAX> w;
  w.lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = blockIdx.y;
  w.nbk = (a.P + kBlockCols - 1) / kBlockCols;
  w.j = blockIdx.x * a.wpb + wave;
  if (w.j >= w.nbk) return;  // a spare wave of the last block (nothing below waits for it)
  w.col = (w.j * kWave + w.lane) * kChunk;
  w.has = w.col < a.P;
  w.colc = w.has ? w.col : a.P - kChunk;  // lanes past the row read a valid chunk

  // First loads: the route list (lane k < K: route k's row and weight) and
  // the token's generation.  Absent routes have no bit in `present`.
  w.e = -1;
  w.wk = 0.0f;
  if (w.lane < a.K) {
    w.e = a.idx[(int64_t)t * a.K + w.lane];
    w.wk = load_weight<WBF16>(a.w, (int64_t)t * a.K + w.lane);
  }
  unsigned g0 = 0;
  if (w.lane == 0) g0 = __hip_atomic_load(a.gen + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  w.present = __ballot(w.lane < a.K && w.e >= 0 && (int64_t)w.e < a.num_rows);
  unpack8(load16(a.gamma + w.colc), w.g);
#pragma unroll
  for (int c = 0; c < 8; ++c) w.g[c] = w.g[c] + a.gain_center;
  w.tag = (unsigned)__builtin_amdgcn_readfirstlane((int)g0) + 1u;
  w.tslots = a.slots + (int64_t)t * KMAX * w.nbk;
  w.limit = a.wait_ticks;
  w.poll = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) w.acc[c] = 0.0f;
#pragma unroll
  for (int k = 0; k < kAhead; ++k)
    tp_issue(a, (w.present >> k) & 1ull, readlane_i(w.e, k), w.colc, w.q[k]);
  tp_step<MODE, KMAX, kAhead, 0>(a, w);
  if (w.has) store16(a.out + (int64_t)t * a.P + w.col, pack8_pz(w.acc));
  if (w.lane == 0)
    __hip_atomic_fetch_max(a.gen + t, w.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------ latent combine ---
//
// One block per token (latent_norm_body in norm_device.h).
__global__ void __launch_bounds__(1024) latent_norm_kernel(const uint16_t* lat, int tp, int b,
                                                           int L, const uint16_t* gamma,
                                                           float eps, uint16_t* y) {
  __shared__ float block_ss[16];
  latent_norm_body(lat, tp, b, L, gamma, eps, y, blockIdx.x, block_ss);
}

}  // namespace

// With the partials asked for, the per-rank kernel writes them and (when
// out is asked for too) a combine pass adds them in rank order; with out
// only, the fused kernel keeps the partials on chip.
hipError_t launch_ep_finalize(const EpArgs& a, hipStream_t s) {
  FinArgs f{a.rows, a.R, a.idx, a.R, a.w, a.gamma, a.gain_center, a.eps,
            a.b, a.K, a.P, a.tp, a.partials, a.out, 1};
  if (!a.partials) return finalize_dispatch(f, a.wbn, a.w_bf16 != 0, s);
  hipError_t e = rank_finalize_dispatch(f, a.wbn, a.w_bf16 != 0, s);
  if (e != hipSuccess || !a.out) return e;
  const int64_t threads = (int64_t)a.b * (a.P / kChunk);
  hipLaunchKernelGGL(rank_combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     a.partials, a.tp, a.b, a.P, a.out);
  return hipGetLastError();
}

template <int MODE, bool WBF16>
hipError_t tp_norm_launch(const TpArgs& a, hipStream_t s) {
  const dim3 grid((a.P / kChunk + 255) / 256, a.b);
  hipLaunchKernelGGL((tp_norm_kernel<MODE, WBF16>), grid, dim3(256), 0, s, a.xr, a.idx,
                     a.num_rows, a.w, a.gamma, a.gain_center, a.eps, a.K, a.P, a.block_total,
                     a.out);
  return hipGetLastError();
}

// Waves per block and routes in flight ahead of the one being added.
constexpr int kTpWavesPerBlock = 7;
constexpr int kTpAhead = 1;

template <int MODE, bool WBF16, int KMAX>
hipError_t tp_mail_launch(const TpMailArgs& p, int b, hipStream_t s) {
  const int nbk = (p.P + kBlockCols - 1) / kBlockCols;
  const int blocks = (nbk + p.wpb - 1) / p.wpb;
  hipLaunchKernelGGL((tp_mail_kernel<MODE, WBF16, KMAX, kTpAhead>), dim3(blocks, b),
                     dim3(kWave * p.wpb), 0, s, p);
  return hipGetLastError();
}

template <int MODE, bool WBF16>
hipError_t tp_mail_dispatch_k(const TpMailArgs& p, int b, hipStream_t s) {
  return p.K <= 16 ? tp_mail_launch<MODE, WBF16, 16>(p, b, s)
                   : tp_mail_launch<MODE, WBF16, 32>(p, b, s);
}

hipError_t launch_tp_finalize(const TpArgs& a, hipStream_t s) {
  if (a.tp <= kTpOnePassMaxRanks) {
    // one pass: a wave per 512 columns, blocks of kTpWavesPerBlock waves
    const int nbk = (a.P + kBlockCols - 1) / kBlockCols;
    const int wpb = nbk < kTpWavesPerBlock ? nbk : kTpWavesPerBlock;
    TpMailArgs p{a.kpart, a.num_rows, a.idx, a.w, a.gamma, a.gain_center, a.eps, a.K, a.P, a.tp,
                 a.out, a.gen, a.slots, wpb, a.wait_ticks};
    switch ((a.wbn != 0 ? 2 : 0) + (a.w_bf16 != 0 ? 1 : 0)) {
      case 0: return tp_mail_dispatch_k<kGainAfter, false>(p, a.b, s);
      case 1: return tp_mail_dispatch_k<kGainAfter, true>(p, a.b, s);
      case 2: return tp_mail_dispatch_k<kGainFirst, false>(p, a.b, s);
      default: return tp_mail_dispatch_k<kGainFirst, true>(p, a.b, s);
    }
  }
  const int routes = a.b * a.K;
  const int nbk = (a.P + kBlockCols - 1) / kBlockCols;
  const int64_t waves = (int64_t)routes * nbk;
  hipLaunchKernelGGL(tp_rank_sum_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s,
                     a.kpart, a.num_rows, a.idx, routes, a.P, a.tp, a.xr, a.gamma, a.gain_center,
                     a.wbn != 0 ? 1 : 0, a.block_total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch ((a.wbn != 0 ? 2 : 0) + (a.w_bf16 != 0 ? 1 : 0)) {
    case 0: return tp_norm_launch<kGainAfter, false>(a, s);
    case 1: return tp_norm_launch<kGainAfter, true>(a, s);
    case 2: return tp_norm_launch<kGainFirst, false>(a, s);
    default: return tp_norm_launch<kGainFirst, true>(a, s);
  }
}

hipError_t launch_latent_norm(const uint16_t* lat, int tp, int b, int L, const uint16_t* gamma,
                              float eps, uint16_t* y, hipStream_t s) {
  const int nwaves = (L + kBlockCols - 1) / kBlockCols;
  hipLaunchKernelGGL(latent_norm_kernel, dim3(b), dim3(kWave * nwaves), 0, s, lat, tp, b, L,
                     gamma, eps, y);
  return hipGetLastError();
}

}  // namespace moetail
