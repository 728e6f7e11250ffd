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

namespace moetail {

namespace {

template <bool WBF16>
__device__ __forceinline__ float load_weight(const void* w, int64_t i) {
  if (WBF16) return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(w)[i]) << 16);
  return reinterpret_cast<const float*>(w)[i];
}

// Gains of one 8-column chunk.
__device__ __forceinline__ void load_gains(const uint16_t* gamma, int col, float gc,
                                           float (&g)[8]) {
  unpack8(load16(gamma + col), g);
#pragma unroll
  for (int c = 0; c < 8; ++c) g[c] = g[c] + gc;
}

// Normalized, route-weighted products of one chunk, added into acc.
template <bool WBN>
__device__ __forceinline__ void add_products(const uint4& xq, const float (&g)[8], float inv,
                                             float w, float (&acc)[8]) {
  float x[8];
  unpack8(xq, x);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float n;
    if (WBN) {
      float s = x[c] * g[c];
      n = s * inv;
    } else {
      float u = x[c] * inv;
      n = u * g[c];
    }
    float p = n * w;
    acc[c] = acc[c] + p;
  }
}

// Lane's share of a chunk's sum of squares (the gains first with WBN).
template <bool WBN>
__device__ __forceinline__ float chunk_ss(const uint4& xq, const float (&g)[8]) {
  float v[8];
  unpack8(xq, v);
  if (WBN) {
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = v[c] * g[c];
  }
  return chunk_sum_of_squares(v);
}

// ------------------------------------------------------------ EP finalize -
//
// One wavefront per (rank d, token t).  Lane k < K holds route k's row index
// and weight; a ballot gives the wave-uniform mask of the rank's local
// routes, walked in ascending order.  The row of the next local route is
// loaded before the current one is reduced, so two rows are in flight.
// Lane l holds columns 512 j + 8 l .. + 7 of every block j in registers.
//
// FUSE: the block is the tp waves of one token; each wave also leaves its
// BF16 partial in LDS and, after one barrier, the block adds the tp
// partials in rank order and writes the combined row (no second launch and
// no re-read of the partials from memory).
template <int NB, bool WBN, bool WBF16, bool FUSE>
__global__ void __launch_bounds__(512) ep_finalize_kernel(EpArgs a) {
  extern __shared__ uint4 staged[];  // FUSE: [tp][P / 8]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int d, t;
  if (FUSE) {
    t = blockIdx.x;
    d = wave;
  } else {
    const int pair = blockIdx.x * (blockDim.x / kWave) + wave;
    if (pair >= a.tp * a.b) return;  // whole wave leaves together
    d = pair / a.b;
    t = pair - d * a.b;
  }
  const int P = a.P;

  int my_row = -1;
  float my_w = 0.0f;
  if (lane < a.K) {
    my_row = a.idx[((int64_t)d * a.b + t) * a.K + lane];
    my_w = load_weight<WBF16>(a.w, (int64_t)t * a.K + lane);
  }
  const bool local = lane < a.K && my_row >= 0 && (int64_t)my_row < a.R;
  uint64_t routes = __ballot(local);

  float g[NB][8];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int col = j * kBlockCols + lane * kChunk;
    if (col < P) load_gains(a.gamma, col, a.gain_center, g[j]);
  }

  const uint16_t* rank_rows = a.rows + (int64_t)d * a.R * P;
  auto load_row = [&](int r, uint4 (&dst)[NB]) {
    const uint16_t* row = rank_rows + (int64_t)r * P;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = j * kBlockCols + lane * kChunk;
      if (col < P) dst[j] = load16(row + col);
    }
  };

  float acc[NB][8];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[j][c] = 0.0f;

  const float inv_width = (float)(1.0 / (double)P);
  uint4 cur[NB];
  int k = -1;
  if (routes) {
    k = __builtin_ctzll(routes);
    routes &= routes - 1;
    load_row(readlane_i(my_row, k), cur);
  }
  while (k >= 0) {
    int kn = -1;
    uint4 nxt[NB];
    if (routes) {
      kn = __builtin_ctzll(routes);
      routes &= routes - 1;
      load_row(readlane_i(my_row, kn), nxt);
    }
    const float wk = readlane_f(my_w, k);
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = j * kBlockCols + lane * kChunk;
      float s = 0.0f;
      if (col < P) s = chunk_ss<WBN>(cur[j], g[j]);
      s = wave_butterfly_sum(s);
      ss = ss + s;
    }
    const float inv = inv_rms(ss, inv_width, a.eps);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = j * kBlockCols + lane * kChunk;
      if (col < P) add_products<WBN>(cur[j], g[j], inv, wk, acc[j]);
    }
    k = kn;
#pragma unroll
    for (int j = 0; j < NB; ++j) cur[j] = nxt[j];
  }

  const int nchunks = P / kChunk;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int col = j * kBlockCols + lane * kChunk;
    if (col < P) {
      const uint4 q = pack8_pz(acc[j]);
      if (a.partials) store16(a.partials + ((int64_t)d * a.b + t) * P + col, q);
      if (FUSE) staged[d * nchunks + col / kChunk] = q;
    }
  }
  if (FUSE) {
    __syncthreads();
    for (int c = threadIdx.x; c < nchunks; c += blockDim.x) {
      float s[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      for (int r = 0; r < a.tp; ++r) {
        float v[8];
        unpack8(staged[r * nchunks + c], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = s[e] + v[e];
      }
      store16(a.out + (int64_t)t * P + c * kChunk, pack8_pz(s));
    }
  }
}

// Rank combine from memory: one thread per 8-column chunk of a token.
__global__ void __launch_bounds__(256) rank_combine_kernel(const uint16_t* partials, int tp,
                                                           int b, int P, uint16_t* out) {
  const int nchunks = P / kChunk;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)b * nchunks) return;
  const int t = (int)(i / nchunks);
  const int c = (int)(i - (int64_t)t * nchunks);
  float s[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int r = 0; r < tp; ++r) {
    float v[8];
    unpack8(load16(partials + ((int64_t)r * b + t) * P + c * kChunk), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = s[e] + v[e];
  }
  store16(out + (int64_t)t * P + c * kChunk, pack8_pz(s));
}

template <int NB, bool WBN, bool WBF16, bool FUSE>
hipError_t ep_launch(const EpArgs& a, hipStream_t stream) {
  if (FUSE) {
    const size_t lds = (size_t)a.tp * a.P * sizeof(uint16_t);
    hipLaunchKernelGGL((ep_finalize_kernel<NB, WBN, WBF16, true>), dim3(a.b), dim3(kWave * a.tp),
                       lds, stream, a);
  } else {
    const int waves = a.tp * a.b;
    const int per_block = 4;
    hipLaunchKernelGGL((ep_finalize_kernel<NB, WBN, WBF16, false>),
                       dim3((waves + per_block - 1) / per_block), dim3(kWave * per_block), 0,
                       stream, a);
  }
  return hipGetLastError();
}

template <int NB>
hipError_t ep_dispatch_nb(const EpArgs& a, bool fuse, hipStream_t s) {
  const int key = (a.wbn ? 4 : 0) | (a.w_bf16 ? 2 : 0) | (fuse ? 1 : 0);
  switch (key) {
    case 0: return ep_launch<NB, false, false, false>(a, s);
    case 1: return ep_launch<NB, false, false, true>(a, s);
    case 2: return ep_launch<NB, false, true, false>(a, s);
    case 3: return ep_launch<NB, false, true, true>(a, s);
    case 4: return ep_launch<NB, true, false, false>(a, s);
    case 5: return ep_launch<NB, true, false, true>(a, s);
    case 6: return ep_launch<NB, true, true, false>(a, s);
    default: return ep_launch<NB, true, true, true>(a, s);
  }
}

// --------------------------------------------------------- expert-TP ----
//
// One block per token, one wave per 512-column block of the row (P <= 8192:
// at most 16 waves).  Pass 1, routes in order: every lane sums its chunk of
// the route's tp K-partials in rank order (FP32 from 0), rounds the sum to
// BF16 (kept in registers) and adds its squares; the wave butterfly gives
// the block's share, left in LDS.  After one barrier every wave folds the
// block shares of each route in block order into inv, and pass 2 adds the
// weighted, normalized products of the routes in order from 0.
template <bool WBN, bool WBF16, int KMAX>
__global__ void __launch_bounds__(1024) tp_finalize_kernel(TpArgs a) {
  __shared__ float block_ss[KMAX][16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const int t = blockIdx.x;
  const int P = a.P;
  const int col = (wave * kWave + lane) * kChunk;
  const bool has = col < P;

  int my_row = -1;
  float my_w = 0.0f;
  if (lane < a.K) {
    my_row = a.idx[(int64_t)t * a.K + lane];
    my_w = load_weight<WBF16>(a.w, (int64_t)t * a.K + lane);
  }
  float g[8];
  if (has) load_gains(a.gamma, col, a.gain_center, g);

  const int64_t rank_stride = a.num_rows * (int64_t)P;
  uint4 xr[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < a.K) {
      const int r = readlane_i(my_row, k);
      if (r >= 0 && (int64_t)r < a.num_rows) {
        float s = 0.0f;
        if (has) {
          const uint16_t* src = a.kpart + (int64_t)r * P + col;
          float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
          for (int rank = 0; rank < a.tp; ++rank) {
            float v[8];
            unpack8(load16(src + rank * rank_stride), v);
#pragma unroll
            for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
          }
          xr[k] = pack8(sum);
          s = chunk_ss<WBN>(xr[k], g);
        }
        s = wave_butterfly_sum(s);
        if (lane == 0) block_ss[k][wave] = s;
      }
    }
  }
  __syncthreads();

  const float inv_width = (float)(1.0 / (double)P);
  float my_inv = 0.0f;
  if (lane < a.K) {
    float total = 0.0f;
    for (int j = 0; j < nwaves; ++j) total = total + block_ss[lane][j];
    my_inv = inv_rms(total, inv_width, a.eps);
  }

  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < a.K) {
      const int r = readlane_i(my_row, k);
      const float inv = readlane_f(my_inv, k);
      const float wk = readlane_f(my_w, k);
      if (r >= 0 && (int64_t)r < a.num_rows && has) add_products<WBN>(xr[k], g, inv, wk, acc);
    }
  }
  if (has) store16(a.out + (int64_t)t * P + col, pack8_pz(acc));
}

template <bool WBN, bool WBF16>
hipError_t tp_launch(const TpArgs& a, hipStream_t s) {
  const int nwaves = (a.P + kBlockCols - 1) / kBlockCols;
  if (a.K <= 16)
    hipLaunchKernelGGL((tp_finalize_kernel<WBN, WBF16, 16>), dim3(a.b), dim3(kWave * nwaves), 0, s, a);
  else
    hipLaunchKernelGGL((tp_finalize_kernel<WBN, WBF16, 32>), dim3(a.b), dim3(kWave * nwaves), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------ latent combine ---
//
// One block per token, one wave per 512-column block: the tp latent
// partials are added in rank order from 0 and rounded to BF16 (l), the
// sum of squares of l is taken in the tree above, and
// y = bf16((l * inv) * fp32(gamma)) with -0 as +0.
__global__ void __launch_bounds__(1024) latent_norm_kernel(const uint16_t* lat, int tp, int b,
                                                           int L, const uint16_t* gamma,
                                                           float eps, uint16_t* y) {
  __shared__ float block_ss[16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const int t = blockIdx.x;
  const int col = (wave * kWave + lane) * kChunk;
  const bool has = col < L;
  uint4 lq = make_uint4(0, 0, 0, 0);
  float s = 0.0f;
  if (has) {
    float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
    for (int r = 0; r < tp; ++r) {
      float v[8];
      unpack8(load16(lat + ((int64_t)r * b + t) * L + col), v);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
    }
    lq = pack8(sum);
    float lv[8];
    unpack8(lq, lv);
    s = chunk_sum_of_squares(lv);
  }
  s = wave_butterfly_sum(s);
  if (lane == 0) block_ss[wave] = s;
  __syncthreads();
  float total = 0.0f;
  for (int j = 0; j < nwaves; ++j) total = total + block_ss[j];
  const float inv = inv_rms(total, (float)(1.0 / (double)L), eps);
  if (has) {
    float lv[8], gv[8], out[8];
    unpack8(lq, lv);
    unpack8(load16(gamma + col), gv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float n = lv[e] * inv;
      out[e] = n * gv[e];
    }
    store16(y + (int64_t)t * L + col, pack8_pz(out));
  }
}

}  // namespace

hipError_t launch_ep_finalize(const EpArgs& a, hipStream_t s) {
  const int nb = (a.P + kBlockCols - 1) / kBlockCols;
  // Fused combine when one block can hold the token's tp partials in LDS.
  const bool fuse = a.out != nullptr && a.tp <= 8 &&
                    (size_t)a.tp * a.P * sizeof(uint16_t) <= 64 * 1024;
  hipError_t e;
  switch (nb) {
    case 1: e = ep_dispatch_nb<1>(a, fuse, s); break;
    case 2: e = ep_dispatch_nb<2>(a, fuse, s); break;
    case 3: e = ep_dispatch_nb<3>(a, fuse, s); break;
    case 4: e = ep_dispatch_nb<4>(a, fuse, s); break;
    case 5: e = ep_dispatch_nb<5>(a, fuse, s); break;
    case 6: e = ep_dispatch_nb<6>(a, fuse, s); break;
    case 7: e = ep_dispatch_nb<7>(a, fuse, s); break;
    case 8: e = ep_dispatch_nb<8>(a, fuse, s); break;
    case 9: e = ep_dispatch_nb<9>(a, fuse, s); break;
    case 10: e = ep_dispatch_nb<10>(a, fuse, s); break;
    case 11: e = ep_dispatch_nb<11>(a, fuse, s); break;
    case 12: e = ep_dispatch_nb<12>(a, fuse, s); break;
    case 13: e = ep_dispatch_nb<13>(a, fuse, s); break;
    case 14: e = ep_dispatch_nb<14>(a, fuse, s); break;
    case 15: e = ep_dispatch_nb<15>(a, fuse, s); break;
    default: e = ep_dispatch_nb<16>(a, fuse, s); break;
  }
  if (e != hipSuccess || fuse || a.out == nullptr) return e;
  const int64_t chunks = (int64_t)a.b * (a.P / kChunk);
  hipLaunchKernelGGL(rank_combine_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     a.partials, a.tp, a.b, a.P, a.out);
  return hipGetLastError();
}

hipError_t launch_tp_finalize(const TpArgs& a, hipStream_t s) {
  const int key = (a.wbn ? 2 : 0) | (a.w_bf16 ? 1 : 0);
  switch (key) {
    case 0: return tp_launch<false, false>(a, s);
    case 1: return tp_launch<false, true>(a, s);
    case 2: return tp_launch<true, false>(a, s);
    default: return tp_launch<true, true>(a, s);
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
