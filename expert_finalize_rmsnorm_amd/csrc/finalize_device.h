// finalize_device.h -- the per-rank EP finalize of one (token, rank) as a
// device function, in phases (the unit's first loads, a batch of rows in
// flight, the arithmetic) that a caller can interleave with other work.
//
// [tail] module docstring and _TpTailKernel (gains, warp_sum_of_squares,
// normalized): for the routes k of token t local to rank d, in ascending
// order,
//   g   = fp32(gamma) + gain_center
//   s   = x * g  with weight_before_norm, else x
//   inv = 1 / sqrt(ss(s) * fp32(1/P) + eps)        (ss: the fixed tree)
//   n   = s * inv  with weight_before_norm, else (x * inv) * g
//   partial[d][t] = bf16(sum_k n * w_k) from +0, -0 written as +0.
#pragma once

#include "common.h"

namespace moetail {

template <bool WBF16>
__device__ __forceinline__ float load_weight(const void* w, int64_t i) {
  if (WBF16) return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(w)[i]) << 16);
  return reinterpret_cast<const float*>(w)[i];
}

// Norm modes: kGainAfter (the gain multiplies the normalized row), kGainFirst
// (weight_before_norm: the gain multiplies before the statistic) and kNoNorm
// ([tail_runtime] module docstring, the Kimi finalize: the route-weighted
// row itself, no statistic).
enum { kGainAfter = 0, kGainFirst = 1, kNoNorm = 2 };

// Route-weighted products of one chunk (normalized unless kNoNorm), added
// into acc.
template <int MODE>
__device__ __forceinline__ void add_products(const uint4& xq, const float (&g)[8], float inv,
                                             float w, float (&acc)[8]) {
  float x[8];
  unpack8(xq, x);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float n;
    if (MODE == kGainFirst) {
      float s = x[c] * g[c];
      n = s * inv;
    } else if (MODE == kGainAfter) {
      float u = x[c] * inv;
      n = u * g[c];
    } else {
      n = x[c];
    }
    float p = n * w;
    acc[c] = acc[c] + p;
  }
}

// Lane's share of a chunk's sum of squares (the gains first with kGainFirst).
template <int MODE>
__device__ __forceinline__ float chunk_ss(const uint4& xq, const float (&g)[8]) {
  float v[8];
  unpack8(xq, v);
  if (MODE == kGainFirst) {
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = v[c] * g[c];
  }
  return chunk_sum_of_squares(v);
}

// One (token, rank) unit's inputs.
struct RankUnit {
  const uint16_t* rows;   // [tp][R][P]
  int64_t R;
  const int32_t* idx;     // [tp][b][K]
  int64_t idx_limit;      // a route is present when 0 <= idx < idx_limit
  const void* w;          // [b][K]
  const uint16_t* gamma;  // [P] (unused with kNoNorm)
  float gain_center, eps;
  int b, K, P;
  uint16_t* partials;     // [tp][b][P]
};

// LDS-only block barrier: this wave's LDS accesses complete, then s_barrier
// (__syncthreads() would also wait for every global load in flight).
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The block's waves 0 .. ceil(P / 512) - 1 own 512-column blocks of the row
// (lane l of wave j: columns 512 j + 8 l .. + 7); any further wave of the
// block runs along with no columns.  Each wave lists the rank's local routes
// itself (lane k < K reads idx[d][t][k]; one ballot; the set bits in
// ascending order are the routes in the order of the sum), then takes them
// in batches of kSlots: every row of a batch is loaded at once, the squares
// reduced across the wave, the block shares met in LDS (block_ss), and the
// weighted products added in route order.  Every wave of the block must
// call this (it holds block barriers).
// A unit's first loads (its route indices and weights, lane k < K holding
// route k's, and the lane's gamma chunk), which the rows' addresses wait for.
struct RankHead {
  int e;
  float wk;
  uint4 gq;
};
template <int MODE, bool WBF16>
__device__ __forceinline__ RankHead rank_head(const RankUnit& a, int t, int d) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = (wave * kWave + lane) * kChunk;
  const int colc = col < a.P ? col : a.P - kChunk;
  RankHead h{-1, 0.0f, make_uint4(0, 0, 0, 0)};
  if (MODE != kNoNorm) h.gq = load16(a.gamma + colc);
  if (lane < a.K) {
    h.e = a.idx[((int64_t)d * a.b + t) * a.K + lane];
    h.wk = load_weight<WBF16>(a.w, (int64_t)t * a.K + lane);
  }
  return h;
}

// A batch of up to kSlots local routes with this lane's chunk of each row
// in flight: slot s holds the s-th of the routes still to add (slots past
// the batch repeat its last route).
template <int kSlots>
struct RankBatch {
  uint64_t rest;  // routes after this batch
  int nb;         // routes in this batch
  int ks[kSlots];
  uint4 xq[kSlots];
};

template <int kSlots>
__device__ __forceinline__ RankBatch<kSlots> rank_batch(const RankUnit& a, int d, int e,
                                                        uint64_t mask) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = (wave * kWave + lane) * kChunk;
  const int colc = col < a.P ? col : a.P - kChunk;
  const uint16_t* rank_rows = a.rows + (int64_t)d * a.R * a.P;
  RankBatch<kSlots> r;
  r.nb = min(kSlots, __popcll(mask));
  uint64_t m = mask;
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    r.ks[s] = m ? (int)__builtin_ctzll(m) : (s > 0 ? r.ks[s - 1] : 0);
    if (m) m &= m - 1;
    // with no local route at all the slots read row 0 (never added): an
    // absent index may lie outside the rank's rows
    const int row = mask ? readlane_i(e, r.ks[s]) : 0;
    r.xq[s] = load16(rank_rows + (int64_t)row * a.P + colc);
  }
  r.rest = m;
  return r;
}

// The rank's local routes: the set bits, in ascending order, of the ballot
// of lanes k < K whose index is present.
__device__ __forceinline__ uint64_t rank_mask(const RankUnit& a, const RankHead& head) {
  const int lane = threadIdx.x & (kWave - 1);
  return __ballot(lane < a.K && head.e >= 0 && (int64_t)head.e < a.idx_limit);
}

// The unit from its head and its first batch (rows already in flight).
template <int MODE, bool WBF16, int kSlots>
__device__ __forceinline__ void rank_finish(const RankUnit& a, int t, int d,
                                            float (*block_ss)[16], const RankHead& head,
                                            RankBatch<kSlots> batch) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int P = a.P;
  const int nwaves = (P + kBlockCols - 1) / kBlockCols;
  const int col = (wave * kWave + lane) * kChunk;
  const bool has = col < P;
  float g[8];
  unpack8(head.gq, g);
#pragma unroll
  for (int c = 0; c < 8; ++c) g[c] = g[c] + a.gain_center;
  const float inv_width = (float)(1.0 / (double)P);
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;

  while (batch.nb > 0) {
    const int nb = batch.nb;
    float my_inv = 0.0f;
    if (MODE != kNoNorm) {
      float ss[kSlots];
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        ss[s] = has ? chunk_ss<MODE>(batch.xq[s], g) : 0.0f;
        ss[s] = wave_butterfly_sum(ss[s]);
      }
      if (lane == 0 && wave < nwaves) {
#pragma unroll
        for (int s = 0; s < kSlots; ++s)
          if (s < nb) block_ss[s][wave] = ss[s];
      }
      lds_sync();
      if (lane < nb) {
        float total = 0.0f;
        for (int j = 0; j < nwaves; ++j) total = total + block_ss[lane][j];
        my_inv = inv_rms(total, inv_width, a.eps);
      }
    }
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      if (s < nb)
        add_products<MODE>(batch.xq[s], g, readlane_f(my_inv, s), readlane_f(head.wk, batch.ks[s]),
                           acc);
    }
    if (MODE != kNoNorm) lds_sync();  // block_ss is refilled by the next batch
    if (batch.rest == 0) break;
    batch = rank_batch<kSlots>(a, d, head.e, batch.rest);
  }
  if (has) store16(a.partials + ((int64_t)d * a.b + t) * P + col, pack8_pz(acc));
}

template <int MODE, bool WBF16, int kSlots>
__device__ __forceinline__ void rank_partial(const RankUnit& a, int t, int d,
                                             float (*block_ss)[16], const RankHead& head) {
  rank_finish<MODE, WBF16, kSlots>(a, t, d, block_ss, head,
                                   rank_batch<kSlots>(a, d, head.e, rank_mask(a, head)));
}

template <int MODE, bool WBF16, int kSlots>
__device__ __forceinline__ void rank_partial(const RankUnit& a, int t, int d,
                                             float (*block_ss)[16]) {
  rank_partial<MODE, WBF16, kSlots>(a, t, d, block_ss, rank_head<MODE, WBF16>(a, t, d));
}

}  // namespace moetail
