// project.hip -- the skinny projections of the MoE tail on the gfx950 matrix
// cores: the 3584 -> 7168 up projection ([tail_runtime] module docstring:
// "the K-split up projection") and the shared expert's gate/up and down
// ([shared] module docstring and SharedUmma.owned_h).
//
// At decode batch sizes (b <= 128 tokens) these are bound by streaming the
// weights from HBM: every weight element is used b times, every activation
// element by every weight row.  Weight rows go on the M side of
// v_mfma_f32_16x16x32_bf16 and tokens on N.
//
// Design (measured on MI355X): what costs bandwidth is not the weight
// stream's access pattern but every other vector-memory instruction a wave
// issues beside it; activation fragments loaded from L2 next to each weight
// load halve the weight stream.  So a block stages the activations of its K
// slice, X[16*NT tokens][k slice], in LDS once (gfx950 gives a block up to
// 160 KB), and then each of its 8 waves streams 16 weight rows over the
// slice with nothing but weight loads (a PF-deep register ring, issued
// unconditionally so the loads in flight stay countable), LDS reads and
// MFMAs.  The K slices are sized to fit the LDS and to give the grid at
// least one block per CU; their FP32 partials are added in slice order by a
// small second kernel, which also applies the epilogue (rs add, or SiLU for
// gate/up) and the single BF16 rounding, -0 written as +0.  Results are
// deterministic: the slice sum order is fixed and each slice is one wave's
// in-order MFMA chain.
#include "common.h"
#include "kernels.h"

namespace moetail {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKStep = 32;              // k per MFMA
constexpr int kLdsBytes = 160 * 1024;   // gfx950 LDS available to one block
constexpr int kPF = 8;                  // k steps in flight per wave

enum { kLinear = 0, kGateUp = 1 };

struct FxArgs {
  const uint16_t* A0;  // rows [0, n0)
  const uint16_t* A1;  // rows [n0, N) (the up matrix for gate/up), or null
  int n0, N, K;
  const uint16_t* X;   // [b][K]
  int b;
  int k_per_split;
  int pitch;           // LDS row pitch of the staged activations (elements)
  float* partials;     // [splits][b][N], or null for the direct epilogue
  const uint16_t* rs;  // direct epilogue only: [b][N] or null
  uint16_t* out;       // direct epilogue only: [b][N]
};

__device__ __forceinline__ float silu(float z) {
  const float e = expf(-z);
  const float den = 1.0f + e;
  return z / den;
}

// h of one (gate, up) FP32 pair: both rounded to BF16 first.
__device__ __forceinline__ float gated(float gate, float up) {
  const float gs = __uint_as_float(bf16_bits(gate) << 16);
  const float us = __uint_as_float(bf16_bits(up) << 16);
  const float a = silu(gs);
  return a * us;
}

__device__ __forceinline__ uint2 pack4_pz(float a, float b, float c, float d) {
  return make_uint2(pack2_rn_pz(a, b), pack2_rn_pz(c, d));
}

// kWaves waves per block, 16 weight rows each.
template <int NT, int kWaves>
__global__ void __launch_bounds__(kWave * kWaves) fx_kernel(FxArgs a) {
  extern __shared__ uint16_t xs[];  // [16 * NT][pitch]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lrow = lane & 15;
  const int kq = lane >> 4;
  const int K = a.K;
  const int kb = blockIdx.y * a.k_per_split;
  const int ke = min(K, kb + a.k_per_split);
  const int nsteps = (ke - kb) / kKStep;
  const int row0 = (blockIdx.x * kWaves + wave) * 16;
  const bool active = row0 < a.N;  // wave-uniform

  // The wave's 16 weight rows lie in one matrix (n0 % 16 == 0).
  const uint16_t* pa = nullptr;
  if (active) {
    const uint16_t* base = row0 < a.n0 ? a.A0 + (int64_t)row0 * K
                                       : a.A1 + (int64_t)(row0 - a.n0) * K;
    pa = base + (int64_t)lrow * K + kb + 8 * kq;
  }
  uint4 ra[kPF];
  const int last = nsteps - 1;
  auto load_a = [&](int j) { return load16(pa + min(j, last) * kKStep); };
  if (active) {
#pragma unroll
    for (int i = 0; i < kPF; ++i) ra[i] = load_a(i);
  }

  // Stage X[16*NT][kb, ke) in LDS; padded tokens repeat the last real one.
  const int cpt = (ke - kb) / 8;  // 16-byte pieces per token
  const int pieces = 16 * NT * cpt;
  for (int p = threadIdx.x; p < pieces; p += blockDim.x) {
    const int tok = p / cpt;
    const int pc = p - tok * cpt;
    const int src = min(tok, a.b - 1);
    *reinterpret_cast<uint4*>(xs + tok * a.pitch + pc * 8) =
        load16(a.X + (int64_t)src * K + kb + pc * 8);
  }
  __syncthreads();
  if (!active) return;

  f32x4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const uint16_t* xl = xs + lrow * a.pitch + 8 * kq;
  for (int j0 = 0; j0 < nsteps; j0 += kPF) {
#pragma unroll
    for (int i = 0; i < kPF; ++i) {
      const int j = j0 + i;
      if (j < nsteps) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint4 bq = *reinterpret_cast<const uint4*>(xl + 16 * nt * a.pitch + j * kKStep);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ra[i]),
                                                            __builtin_bit_cast(bf16x8_t, bq),
                                                            acc[nt], 0, 0, 0);
        }
      }
      ra[i] = load_a(j + kPF);
    }
  }

  // Accumulator lane layout: rows row0 + 4 * (lane / 16) + v, token lane % 16.
  const int r = row0 + 4 * kq;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int tok = 16 * nt + lrow;
    if (tok >= a.b) continue;
    const f32x4_t s = acc[nt];
    if (a.partials) {
      *reinterpret_cast<f32x4_t*>(a.partials + ((int64_t)blockIdx.y * a.b + tok) * a.N + r) = s;
    } else {
      float o[4] = {s[0], s[1], s[2], s[3]};
      if (a.rs) {
        const uint2 q2 = *reinterpret_cast<const uint2*>(a.rs + (int64_t)tok * a.N + r);
        o[0] = o[0] + bf16_lo(q2.x);
        o[1] = o[1] + bf16_hi(q2.x);
        o[2] = o[2] + bf16_lo(q2.y);
        o[3] = o[3] + bf16_hi(q2.y);
      }
      *reinterpret_cast<uint2*>(a.out + (int64_t)tok * a.N + r) = pack4_pz(o[0], o[1], o[2], o[3]);
    }
  }
}

// Slice partials added in slice order, then the epilogue: one thread per 4
// output rows of a token.  kGateUp: partials hold gate rows [0, N) and up
// rows [N, 2N); out is h [b][N].
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
  return nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : 8;
}

int round_up_i(int v, int a) { return (v + a - 1) / a * a; }

// Slices of K: each slice's staged activations fit the LDS (row pitch
// rounded to 128 + 8 elements keeps the LDS reads conflict-free); at least
// `target` blocks when target > 0; forced_splits > 0 asks for that many
// slices (raised to what the LDS needs, capped at 4 k steps per slice).
ProjPlan make_plan(int b, int rows, int K, int waves, int target, int forced_splits) {
  const int tok = 16 * token_blocks(b);
  const int kmax = ((kLdsBytes / (2 * tok)) - 8) / 128 * 128;
  const int row_blocks = (rows + 16 * waves - 1) / (16 * waves);
  const int lds_min = (K + kmax - 1) / kmax;
  int splits = lds_min;
  const int par = target > 0 ? (target + row_blocks - 1) / row_blocks : 1;
  if (par > splits) splits = par;
  if (forced_splits > splits) splits = forced_splits;
  const int max_splits = K / (kKStep * 4);  // at least 4 k steps per slice
  if (splits > max_splits) splits = max_splits > 0 ? max_splits : 1;
  int kps = round_up_i((K + splits - 1) / splits, kKStep);
  while (round_up_i(kps, 128) > kmax && kps > kKStep) kps -= kKStep;  // stay inside LDS
  splits = (K + kps - 1) / kps;
  ProjPlan p;
  p.splits = splits;
  p.k_per_split = kps;
  p.pitch = round_up_i(kps, 128) + 8;
  p.lds = (size_t)tok * p.pitch * sizeof(uint16_t);
  p.waves = waves;
  return p;
}

template <int NT, int W>
hipError_t fx_launch(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  static bool attr_set = false;  // idempotent: every call sets the same maximum
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fx_kernel<NT, W>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int row_blocks = (a.N + 16 * W - 1) / (16 * W);
  hipLaunchKernelGGL((fx_kernel<NT, W>), dim3(row_blocks, p.splits), dim3(kWave * W), p.lds, s, a);
  return hipGetLastError();
}

template <int W>
hipError_t fx_dispatch_w(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  switch (token_blocks(a.b)) {
    case 1: return fx_launch<1, W>(a, p, s);
    case 2: return fx_launch<2, W>(a, p, s);
    case 4: return fx_launch<4, W>(a, p, s);
    default: return fx_launch<8, W>(a, p, s);
  }
}

hipError_t fx_dispatch(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  return p.waves == 16 ? fx_dispatch_w<16>(a, p, s) : fx_dispatch_w<8>(a, p, s);
}

}  // namespace

// Default knobs, from a sweep on MI355X of slices {2,3,4,6,8,12} x waves
// {8,16} at b in {16,32,64,128} for the three projections of the tail
// (gate/up 12288x7168, down 7168x6144, up 7168x3584): four K slices win
// almost everywhere (eight for the long reductions at b = 64), and 16 waves
// per block for the long reductions (gate/up always, down above b = 32)
// and for every projection above b = 64.
ProjTuning default_tuning(int b, int rows, int K) {
  const bool wide = K >= 6144;
  ProjTuning t{4, 8, 0};
  if (wide && (rows >= 12288 || b > 32)) t.waves = 16;
  if (b > 64) t.waves = 16;
  if (wide && b > 32 && b <= 64) t.splits = 8;
  if (b > 64 && !wide) t.splits = 3;
  return t;
}

ProjPlan plan_projection(int b, int rows, int K, const ProjTuning& t) {
  const ProjTuning d = default_tuning(b, rows, K);
  const int splits = t.splits > 0 ? t.splits : d.splits;
  const int waves = (t.waves > 0 ? t.waves : d.waves) == 16 ? 16 : 8;
  const int target = t.target_blocks > 0 ? t.target_blocks : 0;
  return make_plan(b, rows, K, waves, target, splits);
}

size_t proj_partial_bytes(const ProjPlan& p, int b, int n_out, bool always) {
  return (p.splits > 1 || always) ? sizeof(float) * (size_t)p.splits * b * n_out : 0;
}

hipError_t launch_linear(const uint16_t* W, int N, int K, const uint16_t* X, int b,
                         const uint16_t* rs, uint16_t* out, const ProjPlan& plan,
                         float* partials, hipStream_t s) {
  const bool split = plan.splits > 1;
  FxArgs a{W, nullptr, N, N, K, X, b, plan.k_per_split, plan.pitch, split ? partials : nullptr,
           rs, out};
  hipError_t e = fx_dispatch(a, plan, s);
  if (e != hipSuccess || !split) return e;
  const int64_t threads = (int64_t)b * (N / 4);
  hipLaunchKernelGGL(split_reduce_kernel<kLinear>, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     0, s, partials, plan.splits, b, N, rs, out);
  return hipGetLastError();
}

hipError_t launch_gate_up(const uint16_t* Wg, const uint16_t* Wu, int I, int H, const uint16_t* X,
                          int b, uint16_t* h, const ProjPlan& plan, float* partials,
                          hipStream_t s) {
  // Gate rows [0, I) and up rows [I, 2I) in one grid; SiLU in the reduction.
  FxArgs a{Wg, Wu, I, 2 * I, H, X, b, plan.k_per_split, plan.pitch, partials, nullptr, nullptr};
  hipError_t e = fx_dispatch(a, plan, s);
  if (e != hipSuccess) return e;
  const int64_t threads = (int64_t)b * (I / 4);
  hipLaunchKernelGGL(split_reduce_kernel<kGateUp>, dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, s, partials, plan.splits, b, I, nullptr, h);
  return hipGetLastError();
}

}  // namespace moetail
