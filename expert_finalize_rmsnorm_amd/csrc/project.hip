// project.hip -- the skinny projections of the MoE tail on the gfx950 matrix
// cores: the 3584 -> 7168 up projection ([tail_runtime] module docstring:
// "the K-split up projection") and the shared expert's gate/up and down
// ([shared] module docstring and SharedUmma.owned_h).
//
// At decode batch sizes (b <= 256 tokens) these are bound by streaming the
// weights from HBM: every weight element is used b times.  Weight rows go
// on the M side of v_mfma_f32_16x16x32_bf16 and tokens on N, so one 16-byte
// load per lane feeds a 16 x 32 weight tile and the FP32 accumulators stay
// in registers for the whole K range of a wave.
//
// Work split: a block is WK waves on one tile of 16*MR weight rows; the
// waves take interleaved 32-wide k steps and add their accumulators in
// wave order through LDS (fixed order, so the result does not depend on
// timing).  When the row tiles alone give too few waves to keep enough
// loads in flight, K is also cut into `splits` slices whose FP32 partials
// go to the workspace and are added in slice order by a second kernel.
// Either way the FP32 result is rounded to BF16 once, -0 written as +0.
#include "common.h"
#include "kernels.h"

namespace moetail {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWK = 4;      // waves per block
constexpr int kKStep = 32;  // k per MFMA

enum { kLinear = 0, kGateUp = 1 };

struct ProjArgs {
  const uint16_t* A0;  // [N][K] (gate rows for kGateUp)
  const uint16_t* A1;  // [N][K] up rows (kGateUp) or null
  int N, K;
  const uint16_t* X;   // [b][K]
  int b;
  int k_per_split;
  float* partials;     // [splits][b][n_out] or null
  const uint16_t* rs;  // [b][N] or null (kLinear)
  uint16_t* out;       // [b][N] (kLinear) or h [b][N] (kGateUp)
};

__device__ __forceinline__ float silu(float z) {
  const float e = expf(-z);
  const float den = 1.0f + e;
  return z / den;
}

// h word pair of one (gate, up) FP32 result pair.
__device__ __forceinline__ float gated(float gate, float up) {
  const float gs = __uint_as_float(bf16_bits(gate) << 16);
  const float us = __uint_as_float(bf16_bits(up) << 16);
  const float a = silu(gs);
  return a * us;
}

__device__ __forceinline__ uint2 pack4_pz(float a, float b, float c, float d) {
  return make_uint2(pack2_rn_pz(a, b), pack2_rn_pz(c, d));
}

template <int MR, int NT, int PF, int MODE>
__global__ void __launch_bounds__(kWave * kWK) proj_kernel(ProjArgs a) {
  extern __shared__ f32x4_t red[];  // [kWK][MR][NT][64 lanes]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int lrow = lane & 15;
  const int kq = lane >> 4;
  const int K = a.K;
  const int kb = blockIdx.y * a.k_per_split;
  const int ke = min(K, kb + a.k_per_split);
  const int nsteps = (ke - kb) / kKStep;

  // Weight rows of the MR tiles.
  const int row0 = (MODE == kGateUp) ? blockIdx.x * 16 : blockIdx.x * 16 * MR;
  const uint16_t* pa[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const uint16_t* base = (MODE == kGateUp) ? (m == 0 ? a.A0 : a.A1) : a.A0;
    const int r = (MODE == kGateUp) ? row0 + lrow : row0 + 16 * m + lrow;
    pa[m] = base + (int64_t)r * K + kb + 8 * kq;
  }
  const uint16_t* pb[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int tok = min(16 * nt + lrow, a.b - 1);  // padded tokens read a valid row
    pb[nt] = a.X + (int64_t)tok * K + kb + 8 * kq;
  }

  f32x4_t acc[MR][NT];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[m][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Register ring of PF k steps; wave w takes steps w, w + WK, ...
  uint4 ra[PF][MR], rb[PF][NT];
  auto load_step = [&](int step, uint4 (&da)[MR], uint4 (&db)[NT]) {
    const int off = step * kKStep;
#pragma unroll
    for (int m = 0; m < MR; ++m) da[m] = load16(pa[m] + off);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) db[nt] = load16(pb[nt] + off);
  };
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int step = wave + i * kWK;
    if (step < nsteps) load_step(step, ra[i], rb[i]);
  }
  for (int base = 0;; base += PF) {
    bool done = false;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int step = wave + (base + i) * kWK;
      if (step >= nsteps) {
        done = true;
        break;
      }
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, ra[i][m]), __builtin_bit_cast(bf16x8_t, rb[i][nt]),
              acc[m][nt], 0, 0, 0);
      const int next = step + PF * kWK;
      if (next < nsteps) load_step(next, ra[i], rb[i]);
    }
    if (done) break;
  }

  // Waves' accumulators added in wave order.
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[((wave * MR + m) * NT + nt) * kWave + lane] = acc[m][nt];
  __syncthreads();

  // Accumulator lane layout: rows 4 * (lane / 16) + v, token lane % 16.
  const int rsub = 4 * kq;
  for (int q = wave; q < NT * (MODE == kGateUp ? 1 : MR); q += kWK) {
    const int nt = (MODE == kGateUp) ? q : q % NT;
    const int m = (MODE == kGateUp) ? 0 : q / NT;
    const int tok = 16 * nt + lrow;
    f32x4_t s0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    f32x4_t s1 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int w = 0; w < kWK; ++w) {
      s0 = s0 + red[((w * MR + m) * NT + nt) * kWave + lane];
      if (MODE == kGateUp) s1 = s1 + red[((w * MR + 1) * NT + nt) * kWave + lane];
    }
    if (tok >= a.b) continue;
    if (MODE == kLinear) {
      const int r = row0 + 16 * m + rsub;
      if (a.partials) {
        *reinterpret_cast<f32x4_t*>(a.partials + ((int64_t)blockIdx.y * a.b + tok) * a.N + r) = s0;
      } else {
        float o[4] = {s0[0], s0[1], s0[2], s0[3]};
        if (a.rs) {
          const uint2 q2 = *reinterpret_cast<const uint2*>(a.rs + (int64_t)tok * a.N + r);
          o[0] = o[0] + bf16_lo(q2.x);
          o[1] = o[1] + bf16_hi(q2.x);
          o[2] = o[2] + bf16_lo(q2.y);
          o[3] = o[3] + bf16_hi(q2.y);
        }
        *reinterpret_cast<uint2*>(a.out + (int64_t)tok * a.N + r) = pack4_pz(o[0], o[1], o[2], o[3]);
      }
    } else {
      const int r = row0 + rsub;
      if (a.partials) {
        float* p = a.partials + ((int64_t)blockIdx.y * a.b + tok) * (2 * (int64_t)a.N);
        *reinterpret_cast<f32x4_t*>(p + r) = s0;
        *reinterpret_cast<f32x4_t*>(p + a.N + r) = s1;
      } else {
        *reinterpret_cast<uint2*>(a.out + (int64_t)tok * a.N + r) =
            pack4_pz(gated(s0[0], s1[0]), gated(s0[1], s1[1]), gated(s0[2], s1[2]),
                     gated(s0[3], s1[3]));
      }
    }
  }
}

// Slice partials added in slice order, then the epilogue: one thread per
// 4 output rows of a token.
template <int MODE>
__global__ void __launch_bounds__(256) split_reduce_kernel(const float* partials, int splits, int b,
                                                          int N, const uint16_t* rs,
                                                          uint16_t* out) {
  const int quads = N / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)b * quads) return;
  const int tok = (int)(i / quads);
  const int r = (int)(i - (int64_t)tok * quads) * 4;
  const int64_t width = (MODE == kGateUp) ? 2 * (int64_t)N : N;
  f32x4_t s0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  f32x4_t s1 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < splits; ++s) {
    const float* p = partials + ((int64_t)s * b + tok) * width;
    s0 = s0 + *reinterpret_cast<const f32x4_t*>(p + r);
    if (MODE == kGateUp) s1 = s1 + *reinterpret_cast<const f32x4_t*>(p + N + r);
  }
  if (MODE == kLinear) {
    float o[4] = {s0[0], s0[1], s0[2], s0[3]};
    if (rs) {
      const uint2 q2 = *reinterpret_cast<const uint2*>(rs + (int64_t)tok * N + r);
      o[0] = o[0] + bf16_lo(q2.x);
      o[1] = o[1] + bf16_hi(q2.x);
      o[2] = o[2] + bf16_lo(q2.y);
      o[3] = o[3] + bf16_hi(q2.y);
    }
    *reinterpret_cast<uint2*>(out + (int64_t)tok * N + r) = pack4_pz(o[0], o[1], o[2], o[3]);
  } else {
    *reinterpret_cast<uint2*>(out + (int64_t)tok * N + r) =
        pack4_pz(gated(s0[0], s1[0]), gated(s0[1], s1[1]), gated(s0[2], s1[2]),
                 gated(s0[3], s1[3]));
  }
}

int token_blocks(int b) {
  const int nt = (b + 15) / 16;
  return nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : nt <= 8 ? 8 : 16;
}

// Rows per tile for the linear mode.
int linear_mr(int nt) { return nt <= 2 ? 1 : 2; }

template <int MR, int NT, int MODE>
hipError_t proj_launch_mr_nt(const ProjArgs& a, int row_tiles, int splits, hipStream_t s) {
  constexpr int kLoads = MR + NT;
  constexpr int PF = kLoads <= 3 ? 8 : kLoads <= 4 ? 6 : kLoads <= 6 ? 4 : kLoads <= 10 ? 2 : 1;
  const size_t lds = sizeof(f32x4_t) * kWK * MR * NT * kWave;
  hipLaunchKernelGGL((proj_kernel<MR, NT, PF, MODE>), dim3(row_tiles, splits), dim3(kWave * kWK),
                     lds, s, a);
  return hipGetLastError();
}

template <int MODE, int MR>
hipError_t proj_launch_mr(const ProjArgs& a, int nt, int row_tiles, int splits, hipStream_t s) {
  switch (nt) {
    case 1: return proj_launch_mr_nt<MR, 1, MODE>(a, row_tiles, splits, s);
    case 2: return proj_launch_mr_nt<MR, 2, MODE>(a, row_tiles, splits, s);
    case 4: return proj_launch_mr_nt<MR, 4, MODE>(a, row_tiles, splits, s);
    case 8: return proj_launch_mr_nt<MR, 8, MODE>(a, row_tiles, splits, s);
    default: return proj_launch_mr_nt<MR, 16, MODE>(a, row_tiles, splits, s);
  }
}

// Splits so that the grid holds about 2048 waves (8 per CU) without cutting
// a slice below 4 k steps per wave.
ProjPlan make_plan(int b, int row_tiles, int K) {
  const int waves = row_tiles * kWK;
  int splits = 1;
  while (splits < 8 && waves * splits < 2048 && K / (2 * splits) >= kKStep * kWK * 4) splits *= 2;
  int kps = (K + splits - 1) / splits;
  kps = (kps + kKStep - 1) / kKStep * kKStep;
  splits = (K + kps - 1) / kps;
  return ProjPlan{splits, kps};
}

}  // namespace

ProjPlan plan_upproj(int b, int N, int L) {
  const int nt = token_blocks(b);
  return make_plan(b, N / (16 * linear_mr(nt)), L);
}
ProjPlan plan_down(int b, int H, int I) { return plan_upproj(b, H, I); }
ProjPlan plan_gate_up(int b, int I, int H) { return make_plan(b, I / 16, H); }

size_t proj_partial_bytes(const ProjPlan& p, int b, int n_out) {
  return p.splits > 1 ? sizeof(float) * (size_t)p.splits * b * n_out : 0;
}

hipError_t launch_linear(const uint16_t* W, int N, int K, const uint16_t* X, int b,
                         const uint16_t* rs, uint16_t* out, const ProjPlan& plan,
                         float* partials, hipStream_t s) {
  ProjArgs a{W, nullptr, N, K, X, b, plan.k_per_split, plan.splits > 1 ? partials : nullptr,
             rs, out};
  const int nt = token_blocks(b);
  const int mr = linear_mr(nt);
  hipError_t e = mr == 1 ? proj_launch_mr<kLinear, 1>(a, nt, N / 16, plan.splits, s)
                         : proj_launch_mr<kLinear, 2>(a, nt, N / 32, plan.splits, s);
  if (e != hipSuccess || plan.splits == 1) return e;
  const int64_t threads = (int64_t)b * (N / 4);
  hipLaunchKernelGGL(split_reduce_kernel<kLinear>, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     0, s, partials, plan.splits, b, N, rs, out);
  return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t* Wg, const uint16_t* Wu, int I, int H, const uint16_t* X,
                          int b, uint16_t* h, const ProjPlan& plan, float* partials,
                          hipStream_t s) {
  ProjArgs a{Wg, Wu, I, H, X, b, plan.k_per_split, plan.splits > 1 ? partials : nullptr, nullptr,
             h};
  const int nt = token_blocks(b);
  hipError_t e = proj_launch_mr<kGateUp, 2>(a, nt, I / 16, plan.splits, s);
  if (e != hipSuccess || plan.splits == 1) return e;
  const int64_t threads = (int64_t)b * (I / 4);
  hipLaunchKernelGGL(split_reduce_kernel<kGateUp>, dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, s, partials, plan.splits, b, I, nullptr, h);
  return hipGetLastError();
}

}  // namespace moetail
