// norm_device.h -- the latent combine + RMSNorm of one token, as a device
// function shared by its own kernel and the fused tail's middle launch.
//
// [tail_runtime] module docstring: the tp latent partials of a token are
// added in rank order from +0 in FP32 and rounded to BF16 (l); the RMS
// statistic spans the full row (sum of squares of l in the fixed tree of
// common.h, times fp32(1/L), plus eps); y = bf16((l * inv) * fp32(gamma)),
// -0 written as +0.
#pragma once

#include "common.h"

namespace moetail {

// Block of kWave * ceil(L / 512) threads, one wave per 512-column block;
// block_ss holds one float per wave.  Every rank's load is in flight at once
// (batches of 8; indices past the last rank re-read it and are not added).
__device__ __forceinline__ void latent_norm_body(const uint16_t* lat, int tp, int b, int L,
                                                 const uint16_t* gamma, float eps, uint16_t* y,
                                                 int t, float* block_ss) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = (L + kBlockCols - 1) / kBlockCols;  // the block: a wave per 512 columns
  const int col = (wave * kWave + lane) * kChunk;
  const bool has = col < L;
  const int colc = has ? col : L - kChunk;
  const uint4 gq = load16(gamma + colc);  // in flight across the barrier
  const uint16_t* src = lat + (int64_t)t * L + colc;
  const int64_t rank_stride = (int64_t)b * L;
  float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int r0 = 0; r0 < tp; r0 += 8) {
    uint4 q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) q[u] = load16(src + min(r0 + u, tp - 1) * rank_stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (r0 + u < tp) {
        float v[8];
        unpack8(q[u], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] = sum[e] + v[e];
      }
    }
  }
  const uint4 lq = pack8(sum);
  float lv[8];
  unpack8(lq, lv);
  float s = has ? chunk_sum_of_squares(lv) : 0.0f;
  s = wave_butterfly_sum(s);
  if (lane == 0) block_ss[wave] = s;
  __syncthreads();
  float total = 0.0f;
  for (int j = 0; j < nwaves; ++j) total = total + block_ss[j];
  const float inv = inv_rms(total, (float)(1.0 / (double)L), eps);
  if (has) {
    float gv[8], out[8];
    unpack8(gq, gv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float n = lv[e] * inv;
      out[e] = n * gv[e];
    }
    store16(y + (int64_t)t * L + col, pack8_pz(out));
  }
}

}  // namespace moetail
