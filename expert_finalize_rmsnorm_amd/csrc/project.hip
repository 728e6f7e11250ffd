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
// Design (measured on MI355X):
//  * The weight stream's pattern matters: on row-major weights a wave-wide
//    operand load reads 64 B of each of 16 rows, and such a stream reaches
//    4.4 TB/s; on the tiled layout of moetail_pack_weights every such load
//    reads 1 KB of contiguous memory, and the stream reaches 5.9 TB/s, as a
//    linear read does.  The loads are non-temporal (weights are read once).
//  * Every other vector-memory instruction a wave issues beside the weight
//    loads costs stream rate: activation fragments loaded from L2 next to
//    each weight load cut it by 20-60%.  So a block stages the activations
//    of its K slice, X[16*NT tokens][k slice], in LDS once (gfx950 gives a
//    block up to 160 KB), and then each of its waves streams 16 weight rows
//    over the slice with nothing but weight loads (a PF-deep register ring,
//    issued unconditionally so the loads in flight stay countable), LDS
//    reads and MFMAs.
//  * The K slices are sized to fit the LDS and to give the grid at least one
//    block per CU; their FP32 partials are added in slice order by a small
//    second kernel, which also applies the epilogue (rs add, or SiLU for
//    gate/up) and the single BF16 rounding, -0 written as +0.
//  * At 4 token blocks a slice holds at most 1152 of K, so a block may run
//    its K range as two LDS passes with every unit's sum kept in registers
//    across them (px_mp_kernel): half the split partials.  The b=64 gate/up
//    and down projections run that way.
// Results are deterministic: the slice sum order is fixed and each slice is
// one wave's in-order MFMA chain, whichever block runs it.
#include <atomic>

#include "common.h"
#include "kernels.h"
#include "norm_device.h"

namespace moetail {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKStep = 32;              // k per MFMA
constexpr int kLdsBytes = 160 * 1024;   // gfx950 LDS available to one block

enum { kLinear = 0, kGateUp = 1 };

struct FxArgs {
  const uint16_t* A0;  // rows [0, n0)
  const uint16_t* A1;  // rows [n0, N) (the up matrix for gate/up), or null
  int n0, N, K;
  const uint16_t* X;   // [b][K]
  int b;
  int k_per_split;
  int blocks_per_slice;
  int pitch;           // LDS row pitch of the staged activations (elements)
  f32x4_t* partials;   // [splits][N / 16][NT][64] tile-major, or null for the
                       // direct epilogue
  const uint16_t* rs;  // direct epilogue only: [b][N] or null
  uint16_t* out;       // direct epilogue only: [b][N]
  int tiled;           // weights in the tiled layout (moetail_pack_weights)
  int passes;          // LDS slices of k_per_split a block's K range spans
};

// A block barrier for LDS data only: this thread's LDS writes complete,
// then s_barrier.  __syncthreads() also makes global memory visible, which
// waits for every load in flight -- here the weight ring's loads from HBM.
// The memory clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float silu(float z) {
  const float e = expf(-z);
  const float den = 1.0f + e;
  return z / den;
}

// h of one (gate, up) FP32 pair: both rounded to BF16 first.
__device__ __forceinline__ float gated(float gate, float up) {
  const uint32_t q = pack2_rn(gate, up);
  const float gs = bf16_lo(q);
  const float us = bf16_hi(q);
  const float a = silu(gs);
  return a * us;
}

__device__ __forceinline__ uint2 pack4_pz(float a, float b, float c, float d) {
  return make_uint2(pack2_rn_pz(a, b), pack2_rn_pz(c, d));
}

// One block per CU, kWaves waves per block.  Block g works on K slice
// s = g / blocks_per_slice; its waves take units u, u + stride, ... of the
// slice (u = wave index within the slice, stride = waves per slice), a unit
// being MR consecutive 16-row tiles that share every activation fragment
// read from LDS.  The slice's activations are staged in LDS once per block
// and reused for every unit the block streams.  Each wave's (unit, k step)
// sequence is one flat stream: the kPF-deep prefetch ring runs across unit
// boundaries, and a unit's FP32 result leaves as soon as its last step is in.
// With kHold > 0 a wave keeps the FP32 results of its first kHold units in
// registers and stores them after its last k step: partial stores issued in
// the middle of the weight stream hold up the loads behind them (vector
// memory operations complete in issue order), stores after it do not.
template <int NT, int MR, int kPF, int kWaves, int kHold>
__device__ __forceinline__ void px_body(const FxArgs& a, int block) {
  extern __shared__ uint16_t xs[];  // [16 * NT][pitch]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lrow = lane & 15;
  const int kq = lane >> 4;
  const int K = a.K;
  const int slice = block / a.blocks_per_slice;
  const int kb = slice * a.k_per_split;
  const int ke = min(K, kb + a.k_per_split);
  const int nsteps = (ke - kb) / kKStep;
  const int stride = a.blocks_per_slice * kWaves;
  const int u = (block - slice * a.blocks_per_slice) * kWaves + wave;
  const int nunits = a.N / (16 * MR);
  const int my_units = u < nunits ? (nunits - u + stride - 1) / stride : 0;  // wave-uniform
  const int total = my_units * nsteps;

  // Weights are read once per call, so their loads are marked non-temporal
  // (streamed past the caches): measured on the b=64 tail step, 102.1 ->
  // 96.3 us, the split partials written at the end of a launch staying
  // cached for the slice sums that read them.
  // Where this lane's 8 weights of a k step lie.  Row-major: row lrow of
  // the tile, columns 8 kq.. of the step (16 rows x 64 B per wave load).
  // Tiled: the step's 16 x 32 fragment is 1 KB in the accumulator's operand
  // order, lane l at 16 l bytes (one contiguous 1 KB per wave load).  A
  // 16-row tile starts 16 K elements further in both layouts.
  const int64_t lane_off = a.tiled ? 8 * lane : (int64_t)lrow * K + 8 * kq;
  const int k_mul = a.tiled ? 16 : 1;        // elements per k of a slice start
  const int step_stride = a.tiled ? 512 : kKStep;

  // The MR tiles of a unit lie in one matrix (n0 % (16 * MR) == 0).
  auto unit_ptr = [&](int unit) {
    const int row0 = unit * 16 * MR;
    const uint16_t* base = row0 < a.n0 ? a.A0 + (int64_t)row0 * K
                                       : a.A1 + (int64_t)(row0 - a.n0) * K;
    return base + lane_off + (int64_t)kb * k_mul;
  };

  // Load cursor: (unit, step); past the wave's last step it stays on it
  // (cache hits), so every ring slot is refilled unconditionally.
  int l_step = 0, l_left = total, l_unit = u;
  const uint16_t* l_ptr = total > 0 ? unit_ptr(u) : a.A0;
  auto next_load = [&](uint4 (&q)[MR]) {
#pragma unroll
    for (int m = 0; m < MR; ++m) q[m] = load16_stream(l_ptr + (int64_t)m * 16 * K + l_step * step_stride);
    if (l_left > 1) {
      --l_left;
      if (++l_step == nsteps) {
        l_step = 0;
        l_unit += stride;
        l_ptr = unit_ptr(l_unit);
      }
    }
  };
  // Stage X[16*NT][kb, ke) in LDS; padded tokens repeat the last real one.
  // A thread's pieces load in batches of kStage, all issued before the
  // first LDS store, and the first batch before the weight ring's first
  // loads: loads complete in issue order, so the activations (L2 hits)
  // never wait behind a weight load from HBM.
  constexpr int kStage = 16;
  constexpr int kThreads = kWave * kWaves;  // (blockDim.x would be a memory load)
  const int cpt = (ke - kb) / 8;  // 16-byte pieces per token
  const int pieces = 16 * NT * cpt;
  auto stage_load = [&](int p) {  // clamped: past the last piece re-reads it
    p = min(p, pieces - 1);
    const int tok = p / cpt;
    const int pc = p - tok * cpt;
    return load16(a.X + (int64_t)min(tok, a.b - 1) * K + kb + pc * 8);
  };
  auto stage_store = [&](int p, const uint4& q) {
    if (p < pieces) {
      const int tok = p / cpt;
      *reinterpret_cast<uint4*>(xs + tok * a.pitch + (p - tok * cpt) * 8) = q;
    }
  };
  uint4 sq[kStage];
#pragma unroll
  for (int j = 0; j < kStage; ++j) sq[j] = stage_load(threadIdx.x + j * kThreads);

  // (unconditional: with no work the cursor rests on the matrix's first
  // element, so the count of loads in flight is the same on every path)
  uint4 ra[kPF][MR];
#pragma unroll
  for (int i = 0; i < kPF; ++i) next_load(ra[i]);

#pragma unroll
  for (int j = 0; j < kStage; ++j) stage_store(threadIdx.x + j * kThreads, sq[j]);
  for (int p0 = threadIdx.x + kStage * kThreads; p0 < pieces; p0 += kStage * kThreads) {
#pragma unroll
    for (int j = 0; j < kStage; ++j) sq[j] = stage_load(p0 + j * kThreads);
#pragma unroll
    for (int j = 0; j < kStage; ++j) stage_store(p0 + j * kThreads, sq[j]);
  }
  lds_barrier();
  if (total == 0) return;

  f32x4_t acc[MR][NT];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[m][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const uint16_t* xl = xs + lrow * a.pitch + 8 * kq;
  int c_unit = u, c_step = 0;

  // Accumulator lane layout: rows 16 * tile + 4 * (lane / 16) + v, token
  // 16 * nt + lane % 16.  Split partials keep exactly that layout, one 1 KB
  // store per (tile, token block); padded tokens are stored too and never read.
  const int ntiles = a.N / 16;
  auto store_partial = [&](const f32x4_t (&v)[MR][NT], int unit) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        a.partials[(((int64_t)slice * ntiles + unit * MR + m) * NT + nt) * kWave + lane] = v[m][nt];
  };
  f32x4_t hold[kHold > 0 ? kHold : 1][MR][NT];
  int held = 0;
  auto emit = [&]() {
    if (a.partials) {
      f32x4_t v[MR][NT];
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          v[m][nt] = acc[m][nt];
          acc[m][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
      if (kHold > 0 && held < kHold) {
        // wave-uniform slot: register moves, no memory operation
#pragma unroll
        for (int j = 0; j < (kHold > 0 ? kHold : 1); ++j)
          if (j == held) {
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) hold[j][m][nt] = v[m][nt];
          }
        ++held;
      } else {
        store_partial(v, c_unit);
      }
      return;
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const int r = (c_unit * MR + m) * 16 + 4 * kq;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int tok = 16 * nt + lrow;
        const f32x4_t s = acc[m][nt];
        acc[m][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if (tok >= a.b) continue;
        float o[4] = {s[0], s[1], s[2], s[3]};
        if (a.rs) {
          const uint2 q2 = *reinterpret_cast<const uint2*>(a.rs + (int64_t)tok * a.N + r);
          o[0] = o[0] + bf16_lo(q2.x);
          o[1] = o[1] + bf16_hi(q2.x);
          o[2] = o[2] + bf16_lo(q2.y);
          o[3] = o[3] + bf16_hi(q2.y);
        }
        *reinterpret_cast<uint2*>(a.out + (int64_t)tok * a.N + r) =
            pack4_pz(o[0], o[1], o[2], o[3]);
      }
    }
  };

  for (int q0 = 0; q0 < total; q0 += kPF) {
#pragma unroll
    for (int i = 0; i < kPF; ++i) {
      if (q0 + i < total) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint4 bq =
              *reinterpret_cast<const uint4*>(xl + 16 * nt * a.pitch + c_step * kKStep);
#pragma unroll
          for (int m = 0; m < MR; ++m)
            acc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, ra[i][m]), __builtin_bit_cast(bf16x8_t, bq),
                acc[m][nt], 0, 0, 0);
        }
        if (++c_step == nsteps) {
          emit();
          c_step = 0;
          c_unit += stride;
        }
      }
      next_load(ra[i]);
    }
  }
  if (kHold > 0) {
#pragma unroll
    for (int j = 0; j < (kHold > 0 ? kHold : 1); ++j)
      if (j < held) store_partial(hold[j], u + j * stride);
  }
}

// Multi-pass: a block's K range is `passes` LDS slices of k_per_split.  It
// stages one slice at a time and streams all of its units over it, each
// wave holding every one of its units' FP32 accumulators in registers
// across the passes (kMaxU units at most), so one split partial covers the
// whole range: fewer partials for the same LDS.  Between passes the block
// meets at an LDS barrier, restages, and meets again; the weight ring runs
// on across the boundary (its loads do not depend on the activations).
// Each unit is still one in-order MFMA chain over its K range.
template <int NT, int kWaves, int kMaxU>
__device__ __forceinline__ void px_body_mp(const FxArgs& a, int block) {
  constexpr int kPF = 8;
  extern __shared__ uint16_t xs[];  // [16 * NT][pitch]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lrow = lane & 15;
  const int kq = lane >> 4;
  const int K = a.K;
  const int passes = a.passes;
  const int split = block / a.blocks_per_slice;
  const int kps = a.k_per_split;
  const int kb0 = split * kps * passes;
  // A multi-pass plan has K == splits * passes * kps; a single-pass plan
  // run here (one pass) may end in a shorter slice.
  const int klen = passes > 1 ? kps : min(kps, K - kb0);
  const int nsteps = klen / kKStep;
  const int stride = a.blocks_per_slice * kWaves;
  const int u = (block - split * a.blocks_per_slice) * kWaves + wave;
  const int nunits = a.N / 16;
  const int my_units = u < nunits ? (nunits - u + stride - 1) / stride : 0;  // <= kMaxU
  const int total = my_units * nsteps * passes;

  const int64_t lane_off = a.tiled ? 8 * lane : (int64_t)lrow * K + 8 * kq;
  const int k_mul = a.tiled ? 16 : 1;
  const int step_stride = a.tiled ? 512 : kKStep;
  auto unit_ptr = [&](int i, int pass) {
    const int row0 = (u + i * stride) * 16;
    const uint16_t* base = row0 < a.n0 ? a.A0 + (int64_t)row0 * K
                                       : a.A1 + (int64_t)(row0 - a.n0) * K;
    return base + lane_off + (int64_t)(kb0 + pass * kps) * k_mul;
  };
  // Load cursor over (pass, unit, step), in the order of the MFMAs; past the
  // wave's last step it stays on it.
  int l_step = 0, l_i = 0, l_pass = 0, l_left = total;
  const uint16_t* l_ptr = total > 0 ? unit_ptr(0, 0) : a.A0;
  auto next_load = [&](uint4& q) {
    q = load16_stream(l_ptr + l_step * step_stride);
    if (l_left > 1) {
      --l_left;
      if (++l_step == nsteps) {
        l_step = 0;
        if (++l_i == my_units) {
          l_i = 0;
          ++l_pass;
        }
        l_ptr = unit_ptr(l_i, l_pass);
      }
    }
  };

  constexpr int kStage = NT >= 8 ? 4 : 16;  // (8 token blocks: the accumulators take 32 registers)
  constexpr int kThreads = kWave * kWaves;
  const int cpt = klen / 8;  // 16-byte pieces per token and pass
  const int pieces = 16 * NT * cpt;
  auto stage_load = [&](int p, int pass) {
    p = min(p, pieces - 1);
    const int tok = p / cpt;
    const int pc = p - tok * cpt;
    return load16(a.X + (int64_t)min(tok, a.b - 1) * K + kb0 + pass * kps + pc * 8);
  };
  auto stage_store = [&](int p, const uint4& q) {
    if (p < pieces) {
      const int tok = p / cpt;
      *reinterpret_cast<uint4*>(xs + tok * a.pitch + (p - tok * cpt) * 8) = q;
    }
  };
  auto stage_rest = [&](int pass, int p_first) {
    uint4 sq[kStage];
    for (int p0 = p_first; p0 < pieces; p0 += kStage * kThreads) {
#pragma unroll
      for (int j = 0; j < kStage; ++j) sq[j] = stage_load(p0 + j * kThreads, pass);
#pragma unroll
      for (int j = 0; j < kStage; ++j) stage_store(p0 + j * kThreads, sq[j]);
    }
  };

  // Pass 0's first staging batch goes out before the weight ring (loads
  // complete in issue order).
  uint4 sq[kStage];
#pragma unroll
  for (int j = 0; j < kStage; ++j) sq[j] = stage_load(threadIdx.x + j * kThreads, 0);
  uint4 ra[kPF];
#pragma unroll
  for (int i = 0; i < kPF; ++i) next_load(ra[i]);
#pragma unroll
  for (int j = 0; j < kStage; ++j) stage_store(threadIdx.x + j * kThreads, sq[j]);
  stage_rest(0, threadIdx.x + kStage * kThreads);
  lds_barrier();

  // Between passes: every wave done with this pass's activations, the next
  // pass's staged, every wave sees them.
  auto restage = [&](int pass) {
    lds_barrier();
    stage_rest(pass, threadIdx.x);
    lds_barrier();
  };
  if (total == 0) {
    for (int p = 1; p < passes; ++p) restage(p);
    return;
  }

  f32x4_t acc[NT];
  f32x4_t hold[kMaxU][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < kMaxU; ++j)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) hold[j][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const uint16_t* xl = xs + lrow * a.pitch + 8 * kq;
  int c_step = 0, c_i = 0, c_pass = 0;

  for (int q0 = 0; q0 < total; q0 += kPF) {
#pragma unroll
    for (int i = 0; i < kPF; ++i) {
      if (q0 + i < total) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint4 bq =
              *reinterpret_cast<const uint4*>(xl + 16 * nt * a.pitch + c_step * kKStep);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, ra[i]), __builtin_bit_cast(bf16x8_t, bq), acc[nt], 0,
              0, 0);
        }
        if (++c_step == nsteps) {
          // park this unit's sum, take up the next one's (register moves:
          // the slot index is wave-uniform)
          c_step = 0;
          const int next_i = c_i + 1 == my_units ? 0 : c_i + 1;
#pragma unroll
          for (int j = 0; j < kMaxU; ++j)
            if (j == c_i)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) hold[j][nt] = acc[nt];
#pragma unroll
          for (int j = 0; j < kMaxU; ++j)
            if (j == next_i)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) acc[nt] = hold[j][nt];
          c_i = next_i;
          if (c_i == 0 && ++c_pass < passes) restage(c_pass);
        }
      }
      next_load(ra[i]);
    }
  }
  // Accumulator lane layout: rows 16 * tile + 4 * (lane / 16) + v, token
  // 16 * nt + lane % 16; one 1 KB store per (tile, token block).
  const int ntiles = a.N / 16;
#pragma unroll
  for (int j = 0; j < kMaxU; ++j)
    if (j < my_units)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        a.partials[(((int64_t)split * ntiles + u + j * stride) * NT + nt) * kWave + lane] =
            hold[j][nt];
}

// Streamed activations.  The block's K range is cut into chunks of
// kStreamCols<NT> columns (32 KB of activations for any token count) and
// wave kW of the block is a producer: it copies chunk after chunk of
// X[16*NT tokens][chunk] into a ring of kRing LDS buffers with direct
// global->LDS loads (no registers, and its loads never sit in a consumer's
// memory queue), up to kRing chunks ahead of the slowest consumer.  Waves
// 0 .. kW-1 are consumers: each streams the weights of its units -- a
// kPF-deep register ring that runs across chunk and unit boundaries -- in
// (chunk, unit, k step) order, every unit's FP32 sum held in registers over
// the whole range.  Nothing makes a consumer stop for the activations
// unless the producer has fallen behind: no pass boundary and no block
// barrier after the first.  Each unit is one in-order MFMA chain over the
// split's K range, so a split gives the same sums as in the other kernels.
//
// LDS: kRing chunk buffers, then the flags: [0] chunks filled, [1 + w]
// chunks consumer w is done with.  Within a chunk, token row t holds its
// 16-byte pieces in the order piece ^ (t % 16): the 16 tokens that one
// operand read takes then sit in 16 different bank groups.
constexpr int kRing = 4;
constexpr int kStreamChunkBytes = 32 * 1024;
constexpr int kStreamLds = kRing * kStreamChunkBytes + 256;
constexpr int kStreamLoads = kStreamChunkBytes / 1024;  // 1 KB direct loads per chunk
constexpr int kSpinLimit = 1 << 20;  // polls before a wait gives up (never reached in practice)
template <int NT>
constexpr int kStreamCols = kStreamChunkBytes / (2 * 16 * NT);

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// The LDS flags are read and written as relaxed workgroup-scope atomics:
// plain LDS reads and writes, which one wave's LDS operations keep in
// order, without the waits for every memory operation in flight that a
// volatile access or an acquire would add (they would drain the weight
// ring).
__device__ __forceinline__ int flag_get(const int* f) {
  return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void flag_set(int* f, int v) {
  __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Waits until at least `need` chunks are filled (consumers) -- a bounded
// poll of the LDS flag; the memory clobber keeps the chunk's reads after it.
__device__ __forceinline__ void wait_filled(int* flags, int need) {
  for (int it = 0; it < kSpinLimit && flag_get(flags) < need; ++it) __builtin_amdgcn_s_sleep(1);
  asm volatile("" ::: "memory");
}

// ------------------------------------------- split sums inside the launch
//
// A streamed launch can form its outputs itself.  Every wave writes its
// units' FP32 partial tiles as before, then counts itself in at the output
// tile's counter.  The wave whose arrival completes the count adds that
// tile's partials of every split in split order from +0, with the adds and
// the single BF16 rounding of split_reduce_kernel / tail_out_kernel, so the
// bits are those of the separate sum launch.  It then writes the tile's BF16
// outputs.  No wave waits for another: which wave is last is known from the
// count alone, whatever order the waves run in.
//
// The splits of a tile run on different XCDs, whose L2 caches are not
// coherent with each other.  So the partial tiles are written and read with
// 16-byte buffer accesses carrying sc1, the cache policy this compiler gives
// device-scope atomic loads and stores on this GPU.  All of a wave's partial
// stores have completed (s_waitcnt vmcnt(0)) before its lane 0 adds to the
// counter with a device-scope atomic.  The compiler's device-scope release is
// that wait plus an L2 write-back for data written with plain stores, and
// no such data is published here.  The last arriver sets its counter back
// to zero, so every counter is zero between calls; the caller zeroes them
// once, before the first call.
enum { kFuseNone = 0, kFuseGateUp = 1, kFusePair = 2 };

struct FuseArgs {
  unsigned* counters;       // one per output tile (null: partials only)
  uint16_t* out;            // gate/up: h [b][n0]; pair: out [b][N]
  uint16_t* rs;             // pair: rs [b][N] (BF16 of the first sum), or null
  int splits0, splits1;     // the two sums' splits (gate/up: the launch's, twice)
  uint32_t bytes0, bytes1;  // the phases' partial regions (bounds of the accesses)
  // The fused gate/up launch's last wave: the latent combine + RMSNorm of
  // one token per block (lat null: none).
  const uint16_t* lat;      // [tp][b][L]
  const uint16_t* gamma;    // [L]
  uint16_t* y;              // [b][L]
  int tp, L;
  float eps;
};

constexpr int kSc1 = 16;  // cache-policy operand of the buffer builtins: sc1

// A raw buffer over [base, base + bytes): accesses past the end read zero
// and write nothing.  The last word is the 32-bit data format of a raw
// buffer on this GPU family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t device_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void store_dev16(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kSc1);
}
__device__ __forceinline__ f32x4_t load_dev16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}

// Byte offset of this lane's f32x4 of partial tile `tile` of split s
// (tile-major: [splits][tiles][NT][64]).
template <int NT>
__device__ __forceinline__ uint32_t partial_off(int s, int tiles, int tile, int nt, int lane) {
  return ((((uint32_t)s * tiles + tile) * NT + nt) * kWave + lane) * 16u;
}

// Counts this wave in at counter c once its partial stores have completed;
// true in the wave whose arrival makes `arrivals` (which sets c back to 0).
__device__ __forceinline__ bool arrive_last(unsigned* c, int arrivals) {
  const int lane = threadIdx.x & (kWave - 1);
  unsigned old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __builtin_amdgcn_readlane(old, 0);
  const bool last = old + 1 == (unsigned)arrivals;
  if (last && lane == 0) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// Two split sums of this lane's f32x4 per token block, each in split order
// from +0: tile ta of region ra (sa splits, tla tiles a split) and tile tb
// of rb.  A batch's loads (both sums) all issue before its adds; indices
// past the last split re-read it and are not added.
template <int NT>
__device__ __forceinline__ void two_split_sums(__amdgpu_buffer_rsrc_t ra, int sa, int tla, int ta,
                                               __amdgpu_buffer_rsrc_t rb, int sb, int tlb, int tb,
                                               f32x4_t (&za)[NT], f32x4_t (&zb)[NT]) {
  constexpr int kB = NT <= 2 ? 8 : (NT == 4 ? 4 : 2);
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    za[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    zb[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const int smax = sa > sb ? sa : sb;
  for (int s0 = 0; s0 < smax; s0 += kB) {
    f32x4_t qa[kB][NT], qb[kB][NT];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int pa = min(s0 + j, sa - 1), pb = min(s0 + j, sb - 1);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        qa[j][nt] = load_dev16(ra, partial_off<NT>(pa, tla, ta, nt, lane));
        qb[j][nt] = load_dev16(rb, partial_off<NT>(pb, tlb, tb, nt, lane));
      }
    }
#pragma unroll
    for (int j = 0; j < kB; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (s0 + j < sa) za[nt] = za[nt] + qa[j][nt];
        if (s0 + j < sb) zb[nt] = zb[nt] + qb[j][nt];
      }
  }
}

// The last arriver's work for output tile t.  Gate/up: h = SiLU(gate sum) *
// up sum (gate tiles [0, n0/16), up tiles [n0/16, N/16) of one region).
// Pair: rs = bf16(down sum), out = bf16(up sum + rs).  -0 leaves as +0.
// Accumulator lane layout: rows 16 t + 4 (lane / 16) + v, token
// 16 nt + lane % 16.
template <int NT, int kFuse>
__device__ __forceinline__ void fuse_tile(const FxArgs& a0, const FxArgs& a1, const FuseArgs& f,
                                          int t) {
  const int lane = threadIdx.x & (kWave - 1);
  f32x4_t za[NT], zb[NT];
  const __amdgpu_buffer_rsrc_t r0 = device_rsrc(a0.partials, f.bytes0);
  if (kFuse == kFuseGateUp) {
    two_split_sums<NT>(r0, f.splits0, a0.N / 16, t, r0, f.splits0, a0.N / 16, t + a0.n0 / 16, za,
                       zb);
  } else {
    const __amdgpu_buffer_rsrc_t r1 = device_rsrc(a1.partials, f.bytes1);
    two_split_sums<NT>(r0, f.splits0, a0.N / 16, t, r1, f.splits1, a1.N / 16, t, za, zb);
  }
  const int row = 16 * t + 4 * (lane >> 4);
  const int nout = kFuse == kFuseGateUp ? a0.n0 : a0.N;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int tok = 16 * nt + (lane & 15);
    if (tok >= a0.b) continue;
    const f32x4_t g = za[nt], u = zb[nt];
    uint2* dst = reinterpret_cast<uint2*>(f.out + (int64_t)tok * nout + row);
    if (kFuse == kFuseGateUp) {
      *dst = pack4_pz(gated(g[0], u[0]), gated(g[1], u[1]), gated(g[2], u[2]), gated(g[3], u[3]));
    } else {
      const uint2 rs2 = pack4_pz(g[0], g[1], g[2], g[3]);
      if (f.rs) *reinterpret_cast<uint2*>(f.rs + (int64_t)tok * nout + row) = rs2;
      *dst = pack4_pz(u[0] + bf16_lo(rs2.x), u[1] + bf16_hi(rs2.x), u[2] + bf16_lo(rs2.y),
                      u[3] + bf16_hi(rs2.y));
    }
  }
}

// One token's latent combine + RMSNorm by a single wave: the arithmetic of
// latent_norm_body, whose block gives each 512-column block its own wave.
// Here the wave takes the column blocks in turn (two blocks' loads in
// flight), adds their butterfly totals in block order from +0 as that
// block does, and then writes y.  L <= 8192: at most 16 column blocks, each
// lane's rounded combine of them kept in registers.
constexpr int kNormMaxBlocks = 16;
__device__ __forceinline__ void latent_norm_wave(const FuseArgs& f, int b, int t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int L = f.L, tp = f.tp;
  const int nblk = (L + kBlockCols - 1) / kBlockCols;
  const uint16_t* src = f.lat + (int64_t)t * L;
  const int64_t rank_stride = (int64_t)b * L;
  uint4 lq[kNormMaxBlocks];
  float total = 0.0f;
#pragma unroll
  for (int j = 0; j < kNormMaxBlocks; j += 2) {
    if (j >= nblk) continue;  // (not break: the loop stays fully unrolled)
    int colc[2];
    bool has[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = ((j + h) * kWave + lane) * kChunk;
      has[h] = j + h < nblk && col < L;
      colc[h] = col < L ? col : L - kChunk;
    }
    float sum[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[h][e] = 0.0f;
    for (int r0 = 0; r0 < tp; r0 += 8) {
      uint4 q[2][8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < 8; ++u) q[h][u] = load16(src + min(r0 + u, tp - 1) * rank_stride + colc[h]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (r0 + u < tp) {
            float v[8];
            unpack8(q[h][u], v);
#pragma unroll
            for (int e = 0; e < 8; ++e) sum[h][e] = sum[h][e] + v[e];
          }
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (j + h < nblk) {
        lq[j + h] = pack8(sum[h]);
        float lv[8];
        unpack8(lq[j + h], lv);
        const float s = wave_butterfly_sum(has[h] ? chunk_sum_of_squares(lv) : 0.0f);
        total = total + s;
      }
    }
  }
  const float inv = inv_rms(total, (float)(1.0 / (double)L), f.eps);
  uint4 gq[kNormMaxBlocks];
#pragma unroll
  for (int j = 0; j < kNormMaxBlocks; ++j) {
    const int col = (j * kWave + lane) * kChunk;
    if (j < nblk) gq[j] = load16(f.gamma + (col < L ? col : L - kChunk));
  }
#pragma unroll
  for (int j = 0; j < kNormMaxBlocks; ++j) {
    const int col = (j * kWave + lane) * kChunk;
    if (j < nblk && col < L) {
      float lv[8], gv[8], o[8];
      unpack8(lq[j], lv);
      unpack8(gq[j], gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float n = lv[e] * inv;
        o[e] = n * gv[e];
      }
      store16(f.y + (int64_t)t * L + col, pack8_pz(o));
    }
  }
}

// One projection's share of a streamed block: its K range (split) and the
// units of it that this wave holds.  With two phases a block runs the
// first projection's chunks, then the second's (the fused tail's down and
// up projections: every wave one unit of each, equal work everywhere).
struct StreamPhase {
  const uint16_t* A0;
  const uint16_t* A1;
  const uint16_t* X;
  f32x4_t* partials;
  int n0, N, K, b, tiled, split;
  int kb0, klen, nchunks, first_chunk;
  int u, stride, units;  // this wave's first unit, unit stride, units held
};

template <int NT, int kW>
__device__ __forceinline__ StreamPhase stream_phase(const FxArgs& a, int block, int first_chunk) {
  constexpr int kC = kStreamCols<NT>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  StreamPhase ph;
  const int split = block / a.blocks_per_slice;
  ph.A0 = a.A0;
  ph.A1 = a.A1;
  ph.X = a.X;
  ph.partials = a.partials;
  ph.n0 = a.n0;
  ph.N = a.N;
  ph.K = a.K;
  ph.b = a.b;
  ph.tiled = a.tiled;
  ph.split = split;
  ph.kb0 = split * a.k_per_split;
  ph.klen = ph.kb0 < a.K ? min(a.k_per_split, a.K - ph.kb0) : 0;  // 0: no split here
  ph.nchunks = (ph.klen + kC - 1) / kC;
  ph.first_chunk = first_chunk;
  ph.stride = a.blocks_per_slice * kW;
  ph.u = (block - split * a.blocks_per_slice) * kW + wave;
  const int nunits = a.N / 16;
  ph.units = (ph.klen > 0 && ph.u < nunits) ? (nunits - ph.u + ph.stride - 1) / ph.stride : 0;
  return ph;
}

// Phase-dependent values are chosen between plain local scalars (q0_f,
// q1_f) by these macros, with no helper function or closure in between: a
// helper that picks one of two fields in memory is simplified, before it
// is inlined, into one load from a selected address, and the structure
// behind it can then never live in registers (it goes to scratch memory).
#define STREAM_FIELD(p, f) ((kPhases > 1 && (p) != 0) ? q1_##f : q0_##f)
#define STREAM_LOCALS(f)           \
  const auto q0_##f = ph0.f;       \
  const auto q1_##f = ph1.f;

// The direct loads of chunk x into its ring buffer (not waited for).
template <int NT, int kPhases>
__device__ __forceinline__ void stream_issue(const StreamPhase& ph0, const StreamPhase& ph1,
                                             uint16_t* xs, int x) {
  constexpr int kC = kStreamCols<NT>;
  constexpr int kChunkElems = kStreamChunkBytes / 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int b = ph0.b;
  STREAM_LOCALS(X)
  STREAM_LOCALS(K)
  STREAM_LOCALS(kb0)
  STREAM_LOCALS(first_chunk)
  const int p = (kPhases > 1 && x >= q1_first_chunk) ? 1 : 0;
  const uint16_t* X = STREAM_FIELD(p, X);
  const int K = STREAM_FIELD(p, K);
  const int col0 = STREAM_FIELD(p, kb0) + (x - STREAM_FIELD(p, first_chunk)) * kC;
  uint16_t* buf = xs + (x % kRing) * kChunkElems;
#pragma unroll
  for (int j = 0; j < kStreamLoads; ++j) {
    const int e = j * 512 + lane * 8;  // element of the chunk this lane fills
    const int t = e / kC;
    const int s = ((e - t * kC) >> 3) ^ (t & 15);
    const int col = min(col0 + 8 * s, K - 8);  // past the range: a valid piece, never read
    const uint16_t* g = X + (int64_t)min(t, b - 1) * K + col;
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)(buf + j * 512), 16, 0, 0);
  }
}

// The producers' LDS flag accesses, each one LDS instruction.  Before any
// LDS access of a wave with direct global->LDS loads in flight, the
// compiler waits for all of them (it cannot tell a flag from the ring
// buffers those loads fill), which would leave one chunk in flight.  The
// producers order these accesses themselves: a chunk's flag is written
// after s_waitcnt vmcnt(kStreamLoads), when that chunk's loads have
// completed (a wave's vector memory operations complete in issue order) and
// only the next chunk's are still in flight; a read waits for its result
// in the same statement.
static_assert(kStreamLoads == 32, "the producers' waits count one chunk's loads");
__device__ __forceinline__ int producer_flag_get(const int* f) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
               : "=v"(v)
               : "v"((unsigned)(size_t)(lds_ptr_t)const_cast<int*>(f))
               : "memory");
  return v;
}
__device__ __forceinline__ void producer_flag_set(int* f, int v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"((unsigned)(size_t)(lds_ptr_t)f), "v"(v) : "memory");
}

// Waits (bounded) until every consumer's flag is at least `need`.
template <int kW>
__device__ __forceinline__ void producer_wait(const int* flags, int need) {
  const int lane = threadIdx.x & (kWave - 1);
  const int* mine = flags + 1 + (lane < kW ? lane : 0);
  for (int it = 0; it < kSpinLimit; ++it) {
    const int v = producer_flag_get(mine);
    if (__ballot(lane < kW && v < need) == 0) break;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Chunk 0 was issued before the block's first barrier.  Two chunks stay in
// flight: chunk x - 1 is published once chunk x's loads are out and x - 1's
// have landed.  Buffer x % kRing is refilled once every consumer is done
// with chunk x - kRing.
template <int NT, int kW, int kPhases>
__device__ __forceinline__ void stream_producer(const StreamPhase& ph0, const StreamPhase& ph1,
                                                uint16_t* xs, int* flags, int nchunks) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int x = 1; x < nchunks; ++x) {
    if (x >= kRing) producer_wait<kW>(flags, x - kRing + 1);
    stream_issue<NT, kPhases>(ph0, ph1, xs, x);
    asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
    if (lane == 0) producer_flag_set(flags, x);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane == 0) producer_flag_set(flags, nchunks);
}

// kPhases (1 or 2) projections in one streamed block: a0's chunks, then
// a1's (a1 unused with one phase); block: the block's position in both
// grids.  kFuse: the split sums formed in the launch (kFuseGateUp: h, and
// the block's wave kW + 1 forms y; kFusePair: rs and out), when f.counters
// is set.
template <int NT, int kW, int kPF, int kMaxU, int kPhases, int kFuse = kFuseNone>
__device__ __forceinline__ void px_body_stream(const FxArgs& a0, const FxArgs& a1, int block,
                                               const FuseArgs& f = FuseArgs{}) {
  constexpr int kC = kStreamCols<NT>;
  constexpr int kChunkElems = kStreamChunkBytes / 2;
  extern __shared__ uint16_t xs[];
  int* flags = reinterpret_cast<int*>(xs + kRing * kChunkElems);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lrow = lane & 15;
  const int kq = lane >> 4;
  const StreamPhase ph0 = stream_phase<NT, kW>(a0, block, 0);
  const StreamPhase ph1 = stream_phase<NT, kW>(kPhases > 1 ? a1 : a0, block, ph0.nchunks);
  const int nchunks = ph0.nchunks + (kPhases > 1 ? ph1.nchunks : 0);
  if (threadIdx.x < 1 + kW) flag_set(flags + threadIdx.x, 0);
  // The first chunk's loads go out before any weight load: the consumers'
  // first ring loads (12 MB over the grid) would otherwise fill the memory
  // queues ahead of them, and every consumer waits for that chunk (measured:
  // it arrived 2.6-3.5 us into the launch).  Issued, then the block meets at
  // an LDS-only barrier (the flags set; no wait for memory).  The producer
  // meets it at a barrier of its own: no code path of the other waves passes
  // its direct loads, which would make the compiler wait for all of their
  // ring loads before their first LDS access.
  if (wave == kW) {
    if (nchunks > 0) stream_issue<NT, kPhases>(ph0, ph1, xs, 0);
    lds_barrier();
    stream_producer<NT, kW, kPhases>(ph0, ph1, xs, flags, nchunks);
    return;
  }
  lds_barrier();
  if (kFuse == kFuseGateUp && wave == kW + 1) {
    if (f.lat)
      for (int t = blockIdx.x; t < a0.b; t += gridDim.x) latent_norm_wave(f, a0.b, t);
    return;
  }
  STREAM_LOCALS(A0)
  STREAM_LOCALS(A1)
  STREAM_LOCALS(n0)
  STREAM_LOCALS(K)
  STREAM_LOCALS(kb0)
  STREAM_LOCALS(klen)
  STREAM_LOCALS(nchunks)
  STREAM_LOCALS(first_chunk)
  STREAM_LOCALS(u)
  STREAM_LOCALS(stride)
  STREAM_LOCALS(units)
  const int tiled = ph0.tiled;  // (every phase has the same layout)

// chunk c's phase; its k steps for each of that phase's units; that
// phase's units held by this wave; the first chunk from c on in which this
// wave has units (nchunks: none); the hold slot of the phase's first unit
#define PHASE_OF(c) ((kPhases > 1 && (c) >= q1_first_chunk) ? 1 : 0)
#define CHUNK_STEPS(c) \
  (min(kC, STREAM_FIELD(PHASE_OF(c), klen) - ((c) - STREAM_FIELD(PHASE_OF(c), first_chunk)) * kC) / kKStep)
#define UNITS_OF(c) STREAM_FIELD(PHASE_OF(c), units)
#define SKIP0(c) ((q0_units == 0 && (c) < q0_nchunks) ? q0_nchunks : (c))
#define WORK_CHUNK(c) \
  ((kPhases > 1 && q1_units == 0 && SKIP0(c) >= q1_first_chunk) ? nchunks : SKIP0(c))
#define SLOT_BASE(c) ((kPhases > 1 && PHASE_OF(c) > 0) ? q0_units : 0)

  const int total =
      q0_units * (q0_klen / kKStep) + (kPhases > 1 ? q1_units * (q1_klen / kKStep) : 0);
  if (total == 0) {
    if (lane == 0) flag_set(flags + 1 + wave, nchunks);
    return;
  }
  const int64_t lane_off0 = tiled ? 8 * lane : (int64_t)lrow * q0_K + 8 * kq;
  const int64_t lane_off1 = tiled ? 8 * lane : (int64_t)lrow * q1_K + 8 * kq;
  const int k_mul = tiled ? 16 : 1;
  const int step_stride = tiled ? 512 : kKStep;
  // where unit i of chunk c starts (the chunk's first k step)
#define UNIT_PTR(c, i, out)                                                                   \
  do {                                                                                        \
    const int p_ = PHASE_OF(c);                                                               \
    const int K_ = STREAM_FIELD(p_, K);                                                       \
    const int n0_ = STREAM_FIELD(p_, n0);                                                     \
    const int row0_ = (STREAM_FIELD(p_, u) + (i) * STREAM_FIELD(p_, stride)) * 16;            \
    const uint16_t* base_ = row0_ < n0_ ? STREAM_FIELD(p_, A0) + (int64_t)row0_ * K_          \
                                        : STREAM_FIELD(p_, A1) + (int64_t)(row0_ - n0_) * K_; \
    (out) = base_ + (p_ ? lane_off1 : lane_off0) +                                            \
            (int64_t)(STREAM_FIELD(p_, kb0) + ((c) - STREAM_FIELD(p_, first_chunk)) * kC) *   \
                k_mul;                                                                        \
  } while (0)

  // Load cursor over (chunk, unit, step), in the order of the MFMAs; past
  // the wave's last step it stays on it (every ring slot refills).
  int l_chunk = WORK_CHUNK(0);
  int l_step = 0, l_i = 0, l_left = total, l_ns = CHUNK_STEPS(l_chunk), l_mu = UNITS_OF(l_chunk);
  const uint16_t* l_ptr;
  UNIT_PTR(l_chunk, 0, l_ptr);
#define NEXT_LOAD(q)                          \
  do {                                        \
    (q) = load16_stream(l_ptr + l_step * step_stride); \
    if (l_left > 1) {                         \
      --l_left;                               \
      if (++l_step == l_ns) {                 \
        l_step = 0;                           \
        if (++l_i == l_mu) {                  \
          l_i = 0;                            \
          l_chunk = WORK_CHUNK(l_chunk + 1);  \
          l_ns = CHUNK_STEPS(l_chunk);        \
          l_mu = UNITS_OF(l_chunk);           \
        }                                     \
        UNIT_PTR(l_chunk, l_i, l_ptr);        \
      }                                       \
    }                                         \
  } while (0)
  uint4 ra[kPF];
#pragma unroll
  for (int i = 0; i < kPF; ++i) NEXT_LOAD(ra[i]);

  // hold slots: phase 0's units first, then phase 1's
  f32x4_t acc[NT];
  f32x4_t hold[kMaxU][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < kMaxU; ++j)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) hold[j][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  int c_chunk = WORK_CHUNK(0);
  int c_step = 0, c_i = 0, c_ns = CHUNK_STEPS(c_chunk), c_mu = UNITS_OF(c_chunk);
  int c_slot0 = SLOT_BASE(c_chunk);
  // operand reads: token row 16 nt + lrow, piece (4 step + kq) ^ lrow
  const uint16_t* xrow = xs + (c_chunk % kRing) * kChunkElems + lrow * kC;
  if (lane == 0) flag_set(flags + 1 + wave, c_chunk);
  wait_filled(flags, c_chunk + 1);

  for (int q0 = 0; q0 < total; q0 += kPF) {
#pragma unroll
    for (int i = 0; i < kPF; ++i) {
      if (q0 + i < total) {
        const uint16_t* xp = xrow + (((4 * c_step + kq) ^ lrow) << 3);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint4 bq = *reinterpret_cast<const uint4*>(xp + 16 * nt * kC);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, ra[i]), __builtin_bit_cast(bf16x8_t, bq), acc[nt], 0,
              0, 0);
        }
        if (++c_step == c_ns) {
          c_step = 0;
          int next_i = c_i + 1;
          int next_chunk = c_chunk;
          if (next_i == c_mu) {
            // this wave is done with the chunk: its buffer may be refilled
            next_i = 0;
            next_chunk = WORK_CHUNK(c_chunk + 1);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane == 0) flag_set(flags + 1 + wave, next_chunk);
          }
          // park this unit's sum, take up the next one's (register moves:
          // the slot indices are wave-uniform)
          const int here = c_slot0 + c_i;
          if (next_chunk < nchunks) {
            c_ns = CHUNK_STEPS(next_chunk);
            c_mu = UNITS_OF(next_chunk);
            c_slot0 = SLOT_BASE(next_chunk);
          }
          const int there = c_slot0 + next_i;
#pragma unroll
          for (int j = 0; j < kMaxU; ++j)
            if (j == here)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) hold[j][nt] = acc[nt];
#pragma unroll
          for (int j = 0; j < kMaxU; ++j)
            if (j == there)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) acc[nt] = hold[j][nt];
          c_i = next_i;
          if (next_chunk != c_chunk) {
            c_chunk = next_chunk;
            if (c_chunk < nchunks) {
              xrow = xs + (c_chunk % kRing) * kChunkElems + lrow * kC;
              wait_filled(flags, c_chunk + 1);
            }
          }
        }
      }
      NEXT_LOAD(ra[i]);
    }
  }
  // Accumulator lane layout: rows 16 * tile + 4 * (lane / 16) + v, token
  // 16 * nt + lane % 16; one 1 KB store per (tile, token block).  Hold slot
  // k is unit k - s0 of its phase (slots visited in a static order: a
  // run-time index into hold would put it in scratch memory).
#define STORE_PHASE(q, s0, bytes)                                                             \
  do {                                                                                        \
    const int ntiles_ = (q).N / 16;                                                           \
    const __amdgpu_buffer_rsrc_t r_ = device_rsrc((q).partials, (bytes));                     \
    _Pragma("unroll") for (int k = 0; k < kMaxU; ++k) {                                       \
      const int j = k - (s0);                                                                 \
      if (j >= 0 && j < (q).units)                                                            \
        _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) {                                   \
          const int tile_ = (q).u + j * (q).stride;                                           \
          if (fused)                                                                          \
            store_dev16(r_, partial_off<NT>((q).split, ntiles_, tile_, nt, lane), hold[k][nt]); \
          else                                                                                \
            (q).partials[(((int64_t)(q).split * ntiles_ + tile_) * NT + nt) * kWave + lane] =  \
                hold[k][nt];                                                                  \
        }                                                                                     \
    }                                                                                         \
  } while (0)
  // (with the sums formed here, the stores are the device-coherent ones)
  const bool fused = kFuse != kFuseNone && f.counters != nullptr;
  STORE_PHASE(ph0, 0, f.bytes0);
  if (kPhases > 1) STORE_PHASE(ph1, q0_units, f.bytes1);
  if (fused) {
    // every lane's partial stores complete, then the arrivals (one per unit
    // held); the wave completing a tile's count forms that tile
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int arrivals = kFuse == kFuseGateUp ? 2 * f.splits0 : f.splits0 + f.splits1;
    const int half = a0.n0 / 16;  // gate/up: up tile i + half pairs with gate tile i
#define FUSE_PHASE(q)                                                                 \
  _Pragma("unroll") for (int j = 0; j < kMaxU; ++j) {                                 \
    if (j < (q).units) {                                                              \
      int t_ = (q).u + j * (q).stride;                                                \
      if (kFuse == kFuseGateUp && t_ >= half) t_ -= half;                             \
      if (arrive_last(f.counters + t_, arrivals)) fuse_tile<NT, kFuse>(a0, a1, f, t_); \
    }                                                                                 \
  }
    FUSE_PHASE(ph0);
    if (kPhases > 1) FUSE_PHASE(ph1);
#undef FUSE_PHASE
  }
#undef PHASE_OF
#undef CHUNK_STEPS
#undef UNITS_OF
#undef SKIP0
#undef WORK_CHUNK
#undef SLOT_BASE
#undef UNIT_PTR
#undef NEXT_LOAD
#undef STORE_PHASE
}
#undef STREAM_FIELD
#undef STREAM_LOCALS

// Blocks reach the 8 XCDs in turn (block g on XCD g % 8), and each XCD has
// its own L2.  The position of block g among the blocks [s, s + m) sorted
// by (XCD, index): consecutive positions share an XCD, so the blocks of one
// K slice -- which stage the same activations -- mostly do too.  Only the
// order in which blocks take their work changes; no sum does.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_position(int g, int s, int m) {
  auto count = [](int lo, int hi, int y) {  // h in [lo, hi) with h % 8 == y
    return (hi - y + kXcds - 1) / kXcds - (lo - y + kXcds - 1) / kXcds;
  };
  const int x = g % kXcds;
  int pos = count(s, g, x);
  for (int y = 0; y < x; ++y) pos += count(s, s + m, y);
  return pos;
}

__device__ __forceinline__ int fx_blocks(const FxArgs& a) {
  const int range = a.k_per_split * (a.passes > 1 ? a.passes : 1);
  return a.blocks_per_slice * ((a.K + range - 1) / range);
}

template <int NT, int MR, int kPF, int kWaves, int kHold>
__global__ void __launch_bounds__(kWave * kWaves) px_kernel(FxArgs a) {
  px_body<NT, MR, kPF, kWaves, kHold>(a, xcd_position(blockIdx.x, 0, fx_blocks(a)));
}

template <int NT, int kWaves, int kMaxU>
__global__ void __launch_bounds__(kWave * kWaves) px_mp_kernel(FxArgs a) {
  px_body_mp<NT, kWaves, kMaxU>(a, xcd_position(blockIdx.x, 0, fx_blocks(a)));
}

// Two independent projections in one persistent grid (the fused tail's down
// and up projections): blocks [0, blocks0) run a0's plan, the rest a1's.
template <int NT, int kWaves, int kHold>
__global__ void __launch_bounds__(kWave * kWaves) px_group_kernel(FxArgs a0, FxArgs a1,
                                                                  int blocks0) {
  if ((int)blockIdx.x < blocks0)
    px_body<NT, 1, 8, kWaves, kHold>(a0, xcd_position(blockIdx.x, 0, blocks0));
  else
    px_body<NT, 1, 8, kWaves, kHold>(a1, xcd_position(blockIdx.x, blocks0, fx_blocks(a1)));
}

// The same two projections, both in the multi-pass form: a single-pass plan
// runs as one pass (the same k-step order into one accumulator, the same
// partial layout, so the same sums as its own launch).
template <int NT, int kWaves, int kMaxU>
__global__ void __launch_bounds__(kWave * kWaves) px_group_mp_kernel(FxArgs a0, FxArgs a1,
                                                                     int blocks0) {
  if ((int)blockIdx.x < blocks0)
    px_body_mp<NT, kWaves, kMaxU>(a0, xcd_position(blockIdx.x, 0, blocks0));
  else
    px_body_mp<NT, kWaves, kMaxU>(a1, xcd_position(blockIdx.x, blocks0, fx_blocks(a1)));
}


template <int NT, int kW, int kPF, int kMaxU>
__global__ void __launch_bounds__(kWave * (kW + 1)) px_stream_kernel(FxArgs a) {
  px_body_stream<NT, kW, kPF, kMaxU, 1>(a, a, xcd_position(blockIdx.x, 0, fx_blocks(a)));
}

// The gate/up projection forming h in the launch, its blocks' last wave
// forming y (the fused tail's first launch after the finalize).
template <int NT, int kW, int kPF>
__global__ void __launch_bounds__(kWave * (kW + 2)) px_gateup_fused_kernel(FxArgs a, FuseArgs f) {
  px_body_stream<NT, kW, kPF, 1, 1, kFuseGateUp>(a, a, xcd_position(blockIdx.x, 0, fx_blocks(a)),
                                                 f);
}

// Two projections (the fused tail's down and up) in one streamed grid:
// block g runs split g / bps of each, one after the other.
template <int NT, int kW, int kPF, int kMaxU>
__global__ void __launch_bounds__(kWave * (kW + 1)) px_pair_stream_kernel(FxArgs a0, FxArgs a1) {
  const int g0 = fx_blocks(a0), g1 = fx_blocks(a1);
  px_body_stream<NT, kW, kPF, kMaxU, 2>(a0, a1, xcd_position(blockIdx.x, 0, g0 > g1 ? g0 : g1));
}

// The same grid forming rs and out in the launch (the fused tail's last).
template <int NT, int kW, int kPF>
__global__ void __launch_bounds__(kWave * (kW + 1)) px_pair_fused_kernel(FxArgs a0, FxArgs a1,
                                                                        FuseArgs f) {
  const int g0 = fx_blocks(a0), g1 = fx_blocks(a1);
  px_body_stream<NT, kW, kPF, 2, 2, kFusePair>(a0, a1,
                                               xcd_position(blockIdx.x, 0, g0 > g1 ? g0 : g1), f);
}

// Slice partials added in slice order, then the epilogue: one thread per
// accumulator lane of a (tile, token block), i.e. 4 output rows of one
// token, reading the tile-major partials with 1 KB per wave and slice.
// kGateUp: partial tiles [0, N/16) are gate rows, [N/16, N/8) up rows; out
// is h [b][N].

// Sum over the splits of element i of each slice (slice_stride apart), in
// slice order from +0; with kGateUp also of element i + up_off.  Batches of
// 8 slices: all loads of a batch issue before the in-order adds (indices
// past the last slice re-read it and are not added).
template <int MODE>
__device__ __forceinline__ void slice_sum(const f32x4_t* partials, int splits,
                                          int64_t slice_stride, int64_t i, int64_t up_off,
                                          f32x4_t& s0, f32x4_t& s1) {
  s0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  s1 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int kBatch = 8;
  for (int s = 0; s < splits; s += kBatch) {
    f32x4_t g[kBatch], u[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const f32x4_t* p = partials + (int64_t)min(s + j, splits - 1) * slice_stride + i;
      g[j] = p[0];
      if (MODE == kGateUp) u[j] = p[up_off];
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s + j < splits) {
        s0 = s0 + g[j];
        if (MODE == kGateUp) s1 = s1 + u[j];
      }
    }
  }
}

// Element i's token and first output row; false for padded tokens.
__device__ __forceinline__ bool lane_position(int64_t i, int64_t per_tile, int b, int& tok,
                                              int& r) {
  const int tile = (int)(i / per_tile);
  const int rem = (int)(i - tile * per_tile);
  const int lane = rem & (kWave - 1);
  tok = 16 * (rem / kWave) + (lane & 15);
  r = tile * 16 + 4 * (lane >> 4);
  return tok < b;
}

__device__ __forceinline__ void add_bf16x4(float (&o)[4], uint2 q2) {
  o[0] = o[0] + bf16_lo(q2.x);
  o[1] = o[1] + bf16_hi(q2.x);
  o[2] = o[2] + bf16_lo(q2.y);
  o[3] = o[3] + bf16_hi(q2.y);
}

template <int MODE>
__device__ __forceinline__ void reduce_body(int64_t i, const f32x4_t* partials, int splits, int b,
                                            int nt_blocks, int N, const uint16_t* rs,
                                            uint16_t* out) {
  const int out_tiles = N / 16;
  const int64_t per_tile = (int64_t)nt_blocks * kWave;
  if (i >= out_tiles * per_tile) return;
  int tok, r;
  if (!lane_position(i, per_tile, b, tok, r)) return;
  const int tiles_in = (MODE == kGateUp) ? 2 * out_tiles : out_tiles;
  f32x4_t s0, s1;
  slice_sum<MODE>(partials, splits, (int64_t)tiles_in * per_tile, i,
                  (int64_t)out_tiles * per_tile, s0, s1);
  if (MODE == kLinear) {
    float o[4] = {s0[0], s0[1], s0[2], s0[3]};
    if (rs) add_bf16x4(o, *reinterpret_cast<const uint2*>(rs + (int64_t)tok * N + r));
    *reinterpret_cast<uint2*>(out + (int64_t)tok * N + r) = pack4_pz(o[0], o[1], o[2], o[3]);
  } else {
    *reinterpret_cast<uint2*>(out + (int64_t)tok * N + r) =
        pack4_pz(gated(s0[0], s1[0]), gated(s0[1], s1[1]), gated(s0[2], s1[2]),
                 gated(s0[3], s1[3]));
  }
}

template <int MODE>
__global__ void __launch_bounds__(256) split_reduce_kernel(const f32x4_t* partials, int splits,
                                                          int b, int nt_blocks, int N,
                                                          const uint16_t* rs, uint16_t* out) {
  reduce_body<MODE>((int64_t)blockIdx.x * 256 + threadIdx.x, partials, splits, b,
                    nt_blocks, N, rs, out);
}

// The fused tail's middle launch: blocks [0, red_blocks) form h from the
// gate/up partials (as split_reduce_kernel<kGateUp>); each later block is
// one token's latent combine + RMSNorm (as latent_norm_kernel).  The two
// parts share no data.
__global__ void __launch_bounds__(1024) tail_mid_kernel(const f32x4_t* gu_partials, int gu_splits,
                                                        int b, int nt_blocks, int I, uint16_t* h,
                                                        int red_blocks, const uint16_t* lat,
                                                        int tp, int L, const uint16_t* gamma,
                                                        float eps, uint16_t* y) {
  __shared__ float block_ss[16];
  if ((int)blockIdx.x < red_blocks) {
    const int threads = kWave * ((L + kBlockCols - 1) / kBlockCols);  // the launch's block
    reduce_body<kGateUp>((int64_t)blockIdx.x * threads + threadIdx.x, gu_partials, gu_splits,
                         b, nt_blocks, I, nullptr, h);
    return;
  }
  latent_norm_body(lat, tp, b, L, gamma, eps, y, blockIdx.x - red_blocks, block_ss);
}

// The fused tail's last launch: rs = bf16(sum of the down partials), then
// out = bf16(sum of the up-projection partials + rs), -0 as +0 both times
// (the values moetail_shared_expert and moetail_combine_norm_upproj give).
__global__ void __launch_bounds__(256) tail_out_kernel(const f32x4_t* down_partials,
                                                      int down_splits, const f32x4_t* up_partials,
                                                      int up_splits, int b, int nt_blocks, int N,
                                                      uint16_t* rs, uint16_t* out) {
  const int64_t per_tile = (int64_t)nt_blocks * kWave;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // blocks of 256
  if (i >= (N / 16) * per_tile) return;
  int tok, r;
  if (!lane_position(i, per_tile, b, tok, r)) return;
  const int64_t slice_stride = (int64_t)(N / 16) * per_tile;
  f32x4_t d, u, unused;
  slice_sum<kLinear>(down_partials, down_splits, slice_stride, i, 0, d, unused);
  slice_sum<kLinear>(up_partials, up_splits, slice_stride, i, 0, u, unused);
  const uint2 rs2 = pack4_pz(d[0], d[1], d[2], d[3]);
  if (rs) *reinterpret_cast<uint2*>(rs + (int64_t)tok * N + r) = rs2;
  float o[4] = {u[0], u[1], u[2], u[3]};
  add_bf16x4(o, rs2);
  *reinterpret_cast<uint2*>(out + (int64_t)tok * N + r) = pack4_pz(o[0], o[1], o[2], o[3]);
}

// --------------------------------------- a projection summed in its blocks
//
// A linear projection (the up projection, the shared expert's down
// projection) for up to 64 tokens in one launch: a block holds every K split
// of its row tiles, one consumer wave per (tile, split) over the plan's K
// range of that split.  So each wave's FP32 sum is, bit for bit, the split
// partial the streamed kernel writes (the same MFMAs on the same operands in
// the same k order).  The producer wave stages each chunk of activations
// for all of the block's K ranges side by side, one sub-chunk per split.  At
// the end the waves leave their sums in LDS, and the block adds a tile's
// splits in split order from +0, adds rs and rounds once: split_reduce_kernel's
// arithmetic, with no partials in memory, no second launch, and no wait on
// any other block.
constexpr int kLocalWaves = 8;  // consumer waves a block: splits x row tiles

struct LocalArgs {
  const uint16_t* W;        // [N][K] row-major, or the tiled layout
  const uint16_t* X;        // [b][K]
  const uint16_t* rs;       // [b][N] or null
  uint16_t* out;            // [b][N]
  int N, K, b, tiled;
  int k_per_split;          // the plan's K range of a split (a multiple of 32)
};

// Columns of one split's sub-chunk: NT token blocks x kLocalCols fill the
// chunk with kS sub-chunks.  A row's pieces of 8 are swizzled by the row
// (piece ^ row) over 16 pieces, or over the 8 of a 64-column row (4 token
// blocks: the 16 rows of an operand read then meet in pairs on the LDS
// banks, which measured neutral there).
template <int NT, int kS>
constexpr int kLocalCols = kStreamCols<NT> / kS;
template <int NT, int kS>
constexpr int kLocalSwz = (kLocalCols<NT, kS> / 8 >= 16) ? 15 : (kLocalCols<NT, kS> / 8 - 1);
// Up to 2 token blocks the waves' sums have LDS of their own beside the
// ring; at 4 (32 KB of sums) they go into the ring once it is free.
template <int NT>
constexpr int kLocalLds = kRing * kStreamChunkBytes + 256 + (NT <= 2 ? kLocalWaves * NT * kWave * 16 : 0);

// Chunk x's activations for every split into its ring buffer (not waited
// for): sub-chunk q holds token rows 0 .. 16 NT - 1 of columns
// q kr + x kc .. + kc, each row's pieces swizzled by the row as in the
// streamed kernel.  Columns past the split's range or past K are valid
// pieces that no wave reads.
template <int NT, int kS>
__device__ __forceinline__ void local_issue(const LocalArgs& a, uint16_t* xs, int x) {
  constexpr int kc = kLocalCols<NT, kS>;
  constexpr int kSub = 16 * NT * kc;  // elements of a sub-chunk
  constexpr int kChunkElems = kStreamChunkBytes / 2;
  const int lane = threadIdx.x & (kWave - 1);
  uint16_t* buf = xs + (x % kRing) * kChunkElems;
#pragma unroll
  for (int j = 0; j < kStreamLoads; ++j) {
    const int e = j * 512 + lane * 8;
    const int q = e / kSub;
    const int rem = e - q * kSub;
    const int t = rem / kc;
    const int piece = ((rem - t * kc) >> 3) ^ (t & kLocalSwz<NT, kS>);
    const int col = min(q * a.k_per_split + x * kc + 8 * piece, a.K - 8);
    const uint16_t* g = a.X + (int64_t)min(t, a.b - 1) * a.K + col;
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)(buf + j * 512), 16, 0, 0);
  }
}

template <int NT, int kS, int kPF>
__global__ void __launch_bounds__(kWave * (kLocalWaves + 1)) px_local_kernel(LocalArgs a) {
  static_assert(kLocalWaves % kS == 0 && kLocalCols<NT, kS> >= 64, "sub-chunk shape");
  static_assert(kLocalWaves * NT * kWave * 16 <= kRing * kStreamChunkBytes, "sums in the ring");
  constexpr int kT = kLocalWaves / kS;     // row tiles a block
  constexpr int kc = kLocalCols<NT, kS>;
  constexpr int kSpc = kc / kKStep;        // k steps of a sub-chunk
  constexpr int kSub = 16 * NT * kc;
  constexpr int kChunkElems = kStreamChunkBytes / 2;
  extern __shared__ uint16_t xs[];
  int* flags = reinterpret_cast<int*>(xs + kRing * kChunkElems);
  f32x4_t* sums = NT <= 2 ? reinterpret_cast<f32x4_t*>(xs + kRing * kChunkElems + 128)
                          : reinterpret_cast<f32x4_t*>(xs);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lrow = lane & 15;
  const int kq = lane >> 4;
  const int pos = xcd_position(blockIdx.x, 0, gridDim.x);
  const int ntiles = a.N / 16;
  const int kr = a.k_per_split;
  const int nchunks = (kr + kc - 1) / kc;  // split 0's range is the longest
  if (threadIdx.x < 1 + kLocalWaves) flag_set(flags + threadIdx.x, 0);
  // (the producer's code and the consumers' meet only at the final barrier:
  // a consumer path through the direct loads would make the compiler wait
  // for every ring load before each chunk's flag poll)
  if (wave == kLocalWaves) {
    local_issue<NT, kS>(a, xs, 0);
    lds_barrier();
    // The producer, as the streamed kernel's (two chunks in flight): a block
    // stages the activations of all its K ranges, half as many bytes as its
    // weights at 16 tokens, as many at 32 and twice as many at 64.
    for (int x = 1; x < nchunks; ++x) {
      if (x >= kRing) producer_wait<kLocalWaves>(flags, x - kRing + 1);
      local_issue<NT, kS>(a, xs, x);
      asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
      if (lane == 0) producer_flag_set(flags, x);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) producer_flag_set(flags, nchunks);
  } else {
    lds_barrier();
    const int tau = wave / kS, split = wave - tau * kS;
    const int tile = pos * kT + tau;
    const int kb0 = split * kr;
    const int klen = (tile < ntiles && kb0 < a.K) ? min(kr, a.K - kb0) : 0;
    const int steps = klen / kKStep;
    f32x4_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (steps == 0) {
      if (lane == 0) flag_set(flags + 1 + wave, nchunks);
    } else {
      const int row0 = tile * 16;
      const uint16_t* wp = a.tiled ? a.W + (int64_t)row0 * a.K + (int64_t)kb0 * 16 + 8 * lane
                                   : a.W + (int64_t)(row0 + lrow) * a.K + kb0 + 8 * kq;
      const int sstride = a.tiled ? 512 : kKStep;
      uint4 ra[kPF];
#pragma unroll
      for (int i = 0; i < kPF; ++i) ra[i] = load16_stream(wp + (int64_t)min(i, steps - 1) * sstride);
      // operand reads: sub-chunk `split`, token row 16 nt + lrow, piece
      // (4 step + kq) ^ lrow
      const int xoff = split * kSub + lrow * kc;
      for (int q0 = 0; q0 < steps; q0 += kPF) {
#pragma unroll
        for (int i = 0; i < kPF; ++i) {
          const int st = q0 + i;
          if (st < steps) {
            const int cx = st / kSpc, ci = st - cx * kSpc;
            if (ci == 0) wait_filled(flags, cx + 1);
            const uint16_t* xp =
                xs + (cx % kRing) * kChunkElems + xoff +
                (((4 * ci + kq) ^ (lrow & kLocalSwz<NT, kS>)) << 3);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              const uint4 bq = *reinterpret_cast<const uint4*>(xp + 16 * nt * kc);
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, ra[i]), __builtin_bit_cast(bf16x8_t, bq), acc[nt],
                  0, 0, 0);
            }
            if (st == steps - 1 || ci == kSpc - 1) {
              // done with this chunk's buffer (with the range: with all of them)
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
              if (lane == 0) flag_set(flags + 1 + wave, st == steps - 1 ? nchunks : cx + 1);
            }
            ra[i] = load16_stream(wp + (int64_t)min(st + kPF, steps - 1) * sstride);
          }
        }
      }
    }
    // at 4 token blocks the sums go into the ring, free once every wave has
    // met here (the producer meets this barrier below)
    if (NT > 2) lds_barrier();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) sums[(wave * NT + nt) * kWave + lane] = acc[nt];
  }
  if (NT > 2 && wave == kLocalWaves) lds_barrier();
  lds_barrier();

  // Output tile tau's token block nt on wave tau NT + nt: the splits' sums in
  // split order from +0, + rs, one rounding (-0 as +0).  Accumulator lane
  // layout: rows 16 tile + 4 (lane / 16) + v, token 16 nt + lane % 16.
  if (wave < kT * NT) {
    const int tau = wave / NT, nt = wave - tau * NT;
    const int tile = pos * kT + tau;
    const int tok = 16 * nt + lrow;
    if (tile < ntiles && tok < a.b) {
      f32x4_t z = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < kS; ++s)
        if (s * kr < a.K) z = z + sums[((tau * kS + s) * NT + nt) * kWave + lane];
      const int r = tile * 16 + 4 * kq;
      float o[4] = {z[0], z[1], z[2], z[3]};
      if (a.rs) add_bf16x4(o, *reinterpret_cast<const uint2*>(a.rs + (int64_t)tok * a.N + r));
      *reinterpret_cast<uint2*>(a.out + (int64_t)tok * a.N + r) = pack4_pz(o[0], o[1], o[2], o[3]);
    }
  }
}

// Tiled weight layout: fragment (t, s) of a [N][K] matrix -- rows
// 16 t .. 16 t + 15, columns 32 s .. 32 s + 31 -- is 1 KB at element
// (t * K/32 + s) * 512, lane l's 8 values (row 16 t + l % 16, columns
// 32 s + 8 (l / 16) ..) at element 8 l of it: the operand order of
// v_mfma_f32_16x16x32_bf16.  One thread per 16 bytes of the result.
__global__ void __launch_bounds__(256) pack_weights_kernel(const uint16_t* w, int64_t n, int k,
                                                          uint16_t* packed) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // blocks of 256
  const int64_t pieces = n * k / 8;
  if (i >= pieces) return;
  const int64_t f = i >> 6;
  const int l = (int)(i & 63);
  const int steps = k / kKStep;
  const int64_t t = f / steps;
  const int st = (int)(f - t * steps);
  store16(packed + i * 8, load16(w + (16 * t + (l & 15)) * k + kKStep * st + 8 * (l >> 4)));
}

int token_blocks(int b) {
  const int nt = (b + 15) / 16;
  return nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : 8;
}

int round_up_i(int v, int a) { return (v + a - 1) / a * a; }


// The plan: `blocks` blocks (one per CU) split over `splits` K slices; each
// slice's activations must fit the LDS (row pitch rounded to 128 + 8
// elements keeps the LDS reads conflict-free).  Without overrides the slice
// count and waves per block are chosen to minimize the modelled bytes: the
// weight stream including idle waves of an uneven tile split and a per-tile
// overhead, the staged activations (once per block), and the FP32 partials
// (written and re-read) with the reduction launch.
// The kernel shapes built: (tiles per unit, prefetch depth, waves per block).
struct Shape {
  int mr, pf, waves;
};
constexpr Shape kShapes[] = {{1, 8, 7},  {1, 8, 8},  {1, 8, 14}, {1, 8, 16}, {2, 4, 4},
                             {2, 4, 7},  {2, 4, 8},  {2, 8, 4},  {2, 8, 7},  {2, 8, 8}};

// The multi-pass plan (two LDS slices per split): units of one tile,
// prefetch 8, 8 or 12 waves, at most 4 units a wave, every split the same
// (K a multiple of two slices).  Taken when asked for (tuning runs), or by
// the default plan when the modelled cost says so.
ProjPlan make_mp_plan(int b, int rows, int K, const ProjTuning& t) {
  const int tok = 16 * token_blocks(b);
  ProjPlan p{};
  const int kmax = ((kLdsBytes / (2 * tok)) - 8) / 128 * 128;
  const int blocks = t.target_blocks > 0 ? t.target_blocks : device_cu_count();
  const int tiles = rows / 16;
  const int passes = t.passes;
  // the fewest splits (the fewest partials) whose slice fits the LDS and
  // that give every wave of 8-wave blocks a weight stream; then the waves per
  // block with the fewest units a wave
  for (int splits = 1; splits <= 32; ++splits) {
    if (t.splits > 0 && splits != t.splits) continue;
    if (K % (passes * splits * kKStep)) continue;
    const int kps = K / (passes * splits);
    if (round_up_i(kps, 128) > kmax) continue;
    const int bps = blocks / splits;
    if (bps < 1) continue;
    if (t.splits <= 0 && (int64_t)tiles * splits < (int64_t)blocks * 8) continue;
    int best_units = 1 << 30;
    for (int w : {8, 12}) {
      if (t.waves > 0 && w != t.waves) continue;
      const int per_wave = (tiles + bps * w - 1) / (bps * w);
      // units held a wave: 4 at most; with 12 waves (168 registers a wave)
      // and 4 token blocks, one; with 8 token blocks (32 accumulator
      // registers a unit), one
      if (per_wave > 4 || (w == 12 && tok == 64 && per_wave > 1) || (tok == 128 && per_wave > 1))
        continue;
      if (per_wave < best_units) {
        best_units = per_wave;
        p.splits = splits;
        p.k_per_split = kps;
        p.pitch = round_up_i(kps, 128) + 8;
        p.lds = (size_t)tok * p.pitch * sizeof(uint16_t);
        p.waves = w;
        p.mr = 1;
        p.pf = 8;
        p.blocks_per_slice = bps;
        p.hold = per_wave;
        p.passes = passes;
      }
    }
    if (p.splits) return p;
  }
  return p;
}

// The streamed kernel's shapes: (consumer waves, prefetch depth, units held
// a wave).  One block of kW + 1 waves per CU.
struct StreamShape {
  int waves, pf, units;
};
constexpr StreamShape kStreamShapes[] = {{6, 8, 1}, {7, 8, 1}};

// The streamed plan: `splits` K ranges (multiples of the k step; the last
// may be shorter), the CUs shared evenly between them, every wave of a
// split at most one unit.  The modelled cost: the longest wave stream times
// the waves of all CUs (the time the weights take, idle waves included),
// the FP32 partials written and re-read, and the activations the blocks
// read from L2 (at a fifth of the weight cost).
ProjPlan make_stream_plan(int b, int rows, int K, const ProjTuning& t) {
  const int tok = 16 * token_blocks(b);
  const int blocks = t.target_blocks > 0 ? t.target_blocks : device_cu_count();
  const int tiles = rows / 16;
  double best = 1e300;
  ProjPlan p{};
  for (int splits = 1; splits <= 32; ++splits) {
    if (t.splits > 0 && splits != t.splits) continue;
    const int kr = round_up_i((K + splits - 1) / splits, kKStep);
    if ((K + kr - 1) / kr != splits) continue;
    const int bps = blocks / splits;
    if (bps < 1) continue;
    for (const StreamShape& sh : kStreamShapes) {
      if (t.waves > 0 && sh.waves != t.waves) continue;
      if (t.pf > 0 && sh.pf != t.pf) continue;
      const int per_wave = (tiles + bps * sh.waves - 1) / (bps * sh.waves);
      if (per_wave > sh.units) continue;
      const double cost = (double)blocks * sh.waves * per_wave * 16.0 * kr * 2.0 +
                          (double)splits * tok * rows * 8.0 + 0.2 * blocks * tok * kr * 2.0;
      if (cost < best * 0.999) {
        best = cost;
        p = ProjPlan{};
        p.splits = splits;
        p.k_per_split = kr;
        p.pitch = 0;
        p.lds = kStreamLds;
        p.waves = sh.waves;
        p.mr = 1;
        p.pf = sh.pf;
        p.blocks_per_slice = bps;
        p.hold = per_wave;
        p.passes = 1;
        p.stream = 1;
      }
    }
  }
  return p;
}

ProjPlan make_plan(int b, int rows, int K, bool always_partials, const ProjTuning& t) {
  if (t.passes == 0 && t.mr == 0) {
    // the library's choice: the streamed kernel where a shape fits
    const ProjPlan sp = make_stream_plan(b, rows, K, t);
    if (sp.splits) return sp;
  }
  if (t.passes >= 2) {
    const ProjPlan mp = make_mp_plan(b, rows, K, t);
    if (mp.splits) return mp;
  }
  if (t.passes == 0 && token_blocks(b) == 8) {
    // At 8 token blocks a slice holds at most 512 of K, so one pass a split
    // needs 13-14 splits, whose FP32 partials (6.3 MB a split for the 12288
    // gate/up rows) cost more than the weights they save streaming; with
    // one unit a wave held in registers across 2-4 LDS passes the gate/up
    // takes 4 splits and the down projection 6.  The fewest splits over the
    // pass counts that fit; the single-pass plan where none does.
    ProjPlan best{};
    for (int passes = 2; passes <= 4; ++passes) {
      ProjTuning tp = t;
      tp.passes = passes;
      const ProjPlan mp = make_mp_plan(b, rows, K, tp);
      if (mp.splits && (!best.splits || mp.splits < best.splits)) best = mp;
    }
    ProjTuning t1 = t;
    t1.passes = 1;
    const ProjPlan one = make_plan(b, rows, K, always_partials, t1);
    return (best.splits && best.splits < one.splits) ? best : one;
  }
  if (t.passes == 0 && token_blocks(b) == 4) {
    // The plan's choice: at 4 token blocks the LDS holds at most 1152 of K a
    // slice, so one pass a split needs 7 or more splits; two passes cut the
    // split partials (b=64: gate/up 8 -> 4 splits, down 8 -> 6; the up
    // projection keeps its 4).  At 1 or 2 token blocks the single-pass
    // plan's extra splits cost less than the multi-pass block's restaging
    // (measured: the shared expert at b=16 lost 2 us).
    ProjTuning t2 = t;
    t2.passes = 2;
    const ProjPlan mp = make_mp_plan(b, rows, K, t2);
    ProjTuning t1 = t;
    t1.passes = 1;
    const ProjPlan one = make_plan(b, rows, K, always_partials, t1);
    return (mp.splits && mp.splits < one.splits) ? mp : one;
  }
  const int tok = 16 * token_blocks(b);
  const int kmax = ((kLdsBytes / (2 * tok)) - 8) / 128 * 128;
  const int blocks = t.target_blocks > 0 ? t.target_blocks : device_cu_count();
  double best = 1e300;
  ProjPlan p{};
  for (int splits = 1; splits <= 64; ++splits) {
    if (t.splits > 0 && splits != t.splits) continue;
    int kps = round_up_i((K + splits - 1) / splits, kKStep);
    if (round_up_i(kps, 128) > kmax) continue;  // slice does not fit the LDS
    if (kps < kKStep * 4 && splits > 1) continue;
    const int real_splits = (K + kps - 1) / kps;
    const int bps = blocks / real_splits > 0 ? blocks / real_splits : 1;  // grid <= blocks
    for (const Shape& sh : kShapes) {
      if (t.waves > 0 && sh.waves != t.waves) continue;
      if (t.mr > 0 ? sh.mr != t.mr : sh.mr != 1) continue;
      if (t.pf > 0 && sh.pf != t.pf) continue;
      if (rows % (16 * sh.mr)) continue;
      const int w = sh.waves;
      const int units = rows / (16 * sh.mr);
      const double per_wave = (double)((units + bps * w - 1) / (bps * w));
      // a unit's epilogue and ring refill cost about 4 k steps
      const double a_bytes =
          per_wave * bps * w * 16.0 * sh.mr * (kps + 4 * kKStep) * 2.0 * real_splits;
      const double x_bytes = (double)blocks * tok * kps * 2.0;
      // partials written and re-read, plus the reduction launch (~4 us)
      const double p_bytes = (real_splits > 1 || always_partials)
                                 ? real_splits * (double)tok * rows * 4.0 * 2.0 + 16.0e6 : 0.0;
      const double cost = a_bytes + x_bytes + p_bytes;
      if (cost < best * 0.999) {
        best = cost;
        p.splits = real_splits;
        p.k_per_split = kps;
        p.pitch = round_up_i(kps, 128) + 8;
        p.lds = (size_t)tok * p.pitch * sizeof(uint16_t);
        p.waves = w;
        p.mr = sh.mr;
        p.pf = sh.pf;
        p.blocks_per_slice = bps;
        // Results held until the stream ends: up to 4 units of one tile and
        // at most 4 token blocks, at most 2 waves per SIMD (256 VGPRs a lane).
        p.hold = (sh.mr == 1 && tok <= 64 && w <= 8 && per_wave <= 4) ? 4 : 0;
      }
    }
  }
  if (best == 1e300 && (t.splits > 0 || t.waves > 0 || t.mr > 0 || t.pf > 0)) {
    // an override that cannot fit: the best plan without it
    const ProjTuning free_t{0, 0, t.target_blocks, 0, 0, t.passes == 0 ? 0 : 1};
    return make_plan(b, rows, K, always_partials, free_t);
  }
  return p;  // splits == 0: no slice of K fits the LDS
}

// A kernel may take the whole LDS: set once per device (the setting is the
// same every time; a bit per device in `done` keeps the call off later
// launches, and concurrent first calls just set it twice).
hipError_t allow_full_lds(const void* fn, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

template <int NT, int MR, int PF, int W, int H>
hipError_t px_launch(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e =
      allow_full_lds(reinterpret_cast<const void*>(px_kernel<NT, MR, PF, W, H>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((px_kernel<NT, MR, PF, W, H>), dim3(p.splits * p.blocks_per_slice),
                     dim3(kWave * W), p.lds, s, a);
  return hipGetLastError();
}

template <int MR, int PF, int W>
hipError_t px_dispatch_nt(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  switch (token_blocks(a.b)) {
    case 1: return px_launch<1, MR, PF, W, 0>(a, p, s);
    case 2: return px_launch<2, MR, PF, W, 0>(a, p, s);
    case 4: return px_launch<4, MR, PF, W, 0>(a, p, s);
    default: return px_launch<8, MR, PF, W, 0>(a, p, s);
  }
}

template <int W>
hipError_t px_dispatch_hold(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  switch (token_blocks(a.b)) {
    case 1: return px_launch<1, 1, 8, W, 4>(a, p, s);
    case 2: return px_launch<2, 1, 8, W, 4>(a, p, s);
    case 4: return px_launch<4, 1, 8, W, 4>(a, p, s);
    default: return hipErrorInvalidValue;  // not planned (more than 4 token blocks)
  }
}

template <int NT, int W, int U>
hipError_t mp_launch(const FxArgs& a0, const ProjPlan& p, hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(px_mp_kernel<NT, W, U>), lds_set);
  if (e != hipSuccess) return e;
  FxArgs a = a0;
  a.passes = p.passes;
  hipLaunchKernelGGL((px_mp_kernel<NT, W, U>), dim3(p.splits * p.blocks_per_slice),
                     dim3(kWave * W), p.lds, s, a);
  return hipGetLastError();
}

template <int W, int U>
hipError_t mp_dispatch_nt(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  switch (token_blocks(a.b)) {
    case 1: return mp_launch<1, W, U>(a, p, s);
    case 2: return mp_launch<2, W, U>(a, p, s);
    case 4: return mp_launch<4, W, U>(a, p, s);
    default:
      // 8 token blocks: one unit a wave (the planner's limit)
      if constexpr (U == 1) return mp_launch<8, W, 1>(a, p, s);
      return hipErrorInvalidValue;
  }
}

// 12 waves holding 2 or 4 units: up to 2 token blocks (4 spill registers).
template <int U>
hipError_t mp_dispatch12_nt(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  switch (token_blocks(a.b)) {
    case 1: return mp_launch<1, 12, U>(a, p, s);
    case 2: return mp_launch<2, 12, U>(a, p, s);
    default: return hipErrorInvalidValue;  // not planned
  }
}

hipError_t mp_dispatch(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  if (!a.partials) return hipErrorInvalidValue;  // the multi-pass kernel always writes partials
  const int u = p.hold <= 1 ? 1 : p.hold <= 2 ? 2 : 4;
  if (p.waves == 12 && token_blocks(a.b) == 4 && u > 1) return hipErrorInvalidValue;  // not planned
  if (token_blocks(a.b) == 8 && u > 1) return hipErrorInvalidValue;                    // not planned
  switch ((p.waves == 12 ? 3 : 0) + (u == 1 ? 0 : u == 2 ? 1 : 2)) {
    case 0: return mp_dispatch_nt<8, 1>(a, p, s);
    case 1: return mp_dispatch_nt<8, 2>(a, p, s);
    case 2: return mp_dispatch_nt<8, 4>(a, p, s);
    case 3: return mp_dispatch_nt<12, 1>(a, p, s);
    case 4: return mp_dispatch12_nt<2>(a, p, s);
    default: return mp_dispatch12_nt<4>(a, p, s);
  }
}

template <int NT, int W, int PF, int U>
hipError_t stream_launch(const FxArgs& a0, const ProjPlan& p, hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e =
      allow_full_lds(reinterpret_cast<const void*>(px_stream_kernel<NT, W, PF, U>), lds_set);
  if (e != hipSuccess) return e;
  FxArgs a = a0;
  a.passes = 1;
  hipLaunchKernelGGL((px_stream_kernel<NT, W, PF, U>), dim3(p.splits * p.blocks_per_slice),
                     dim3(kWave * (W + 1)), kStreamLds, s, a);
  return hipGetLastError();
}

template <int W, int PF, int U>
hipError_t stream_dispatch_nt(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  switch (token_blocks(a.b)) {
    case 1: return stream_launch<1, W, PF, U>(a, p, s);
    case 2: return stream_launch<2, W, PF, U>(a, p, s);
    case 4: return stream_launch<4, W, PF, U>(a, p, s);
    default: return stream_launch<8, W, PF, U>(a, p, s);
  }
}

hipError_t stream_dispatch(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  if (!a.partials || p.hold != 1 || p.pf != 8) return hipErrorInvalidValue;  // not planned
  if (p.waves == 6) return stream_dispatch_nt<6, 8, 1>(a, p, s);
  if (p.waves == 7) return stream_dispatch_nt<7, 8, 1>(a, p, s);
  return hipErrorInvalidValue;
}

hipError_t fx_dispatch(const FxArgs& a, const ProjPlan& p, hipStream_t s) {
  if (p.stream) return stream_dispatch(a, p, s);
  if (p.passes > 1) return mp_dispatch(a, p, s);
  if (p.hold && a.partials) {
    if (p.mr != 1 || p.pf != 8 || p.waves > 8 || token_blocks(a.b) > 4) return hipErrorInvalidValue;
    return p.waves == 7 ? px_dispatch_hold<7>(a, p, s) : px_dispatch_hold<8>(a, p, s);
  }
  const int key = p.mr * 1000 + p.pf * 100 + p.waves;
  switch (key) {
    case 1807: return px_dispatch_nt<1, 8, 7>(a, p, s);
    case 1808: return px_dispatch_nt<1, 8, 8>(a, p, s);
    case 1814: return px_dispatch_nt<1, 8, 14>(a, p, s);
    case 1816: return px_dispatch_nt<1, 8, 16>(a, p, s);
    case 2404: return px_dispatch_nt<2, 4, 4>(a, p, s);
    case 2407: return px_dispatch_nt<2, 4, 7>(a, p, s);
    case 2408: return px_dispatch_nt<2, 4, 8>(a, p, s);
    case 2804: return px_dispatch_nt<2, 8, 4>(a, p, s);
    case 2807: return px_dispatch_nt<2, 8, 7>(a, p, s);
    case 2808: return px_dispatch_nt<2, 8, 8>(a, p, s);
    default: return hipErrorInvalidValue;  // not a shape of kShapes
  }
}

template <int NT, int W, int H>
hipError_t group_launch(const FxArgs& a0, const FxArgs& a1, int blocks0, int blocks, size_t lds,
                        hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e =
      allow_full_lds(reinterpret_cast<const void*>(px_group_kernel<NT, W, H>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((px_group_kernel<NT, W, H>), dim3(blocks), dim3(kWave * W), lds, s, a0, a1,
                     blocks0);
  return hipGetLastError();
}

template <int NT, int W, int U>
hipError_t group_mp_launch(const FxArgs& a0, const FxArgs& a1, int blocks0, int blocks,
                           size_t lds, hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e =
      allow_full_lds(reinterpret_cast<const void*>(px_group_mp_kernel<NT, W, U>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((px_group_mp_kernel<NT, W, U>), dim3(blocks), dim3(kWave * W), lds, s, a0,
                     a1, blocks0);
  return hipGetLastError();
}

// 8 waves hold up to 4 units; 12 waves (168 registers a wave) up to 4 with
// 1 or 2 token blocks, one with 4.
hipError_t group_mp_dispatch(const FxArgs& a0, const FxArgs& a1, const GroupPlan& g, int blocks0,
                             int blocks, size_t lds, hipStream_t s) {
  const int ntb = token_blocks(a0.b);
  if (g.hold > 4 || (g.waves == 12 && ntb == 4 && g.hold > 1) || (ntb == 8 && g.hold > 1))
    return hipErrorInvalidValue;
  if (g.waves == 8) {
    switch (ntb) {
      case 1: return group_mp_launch<1, 8, 4>(a0, a1, blocks0, blocks, lds, s);
      case 2: return group_mp_launch<2, 8, 4>(a0, a1, blocks0, blocks, lds, s);
      case 4: return group_mp_launch<4, 8, 4>(a0, a1, blocks0, blocks, lds, s);
      default:
        if (g.hold > 1) return hipErrorInvalidValue;  // not planned
        return group_mp_launch<8, 8, 1>(a0, a1, blocks0, blocks, lds, s);
    }
  }
  if (g.waves == 12) {
    switch (ntb) {
      case 1: return group_mp_launch<1, 12, 4>(a0, a1, blocks0, blocks, lds, s);
      case 2: return group_mp_launch<2, 12, 4>(a0, a1, blocks0, blocks, lds, s);
      case 4: return group_mp_launch<4, 12, 1>(a0, a1, blocks0, blocks, lds, s);
      default:
        if (g.hold > 1) return hipErrorInvalidValue;  // not planned
        return group_mp_launch<8, 12, 1>(a0, a1, blocks0, blocks, lds, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int NT, int W, int PF, int U>
hipError_t pair_stream_launch(const FxArgs& a0, const FxArgs& a1, int blocks, hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_full_lds(
      reinterpret_cast<const void*>(px_pair_stream_kernel<NT, W, PF, U>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((px_pair_stream_kernel<NT, W, PF, U>), dim3(blocks), dim3(kWave * (W + 1)),
                     kStreamLds, s, a0, a1);
  return hipGetLastError();
}

// One unit of each projection a wave, 6 or 7 consumer waves.
template <int W>
hipError_t pair_stream_dispatch_nt(const FxArgs& a0, const FxArgs& a1, int blocks,
                                   hipStream_t s) {
  switch (token_blocks(a0.b)) {
    case 1: return pair_stream_launch<1, W, 8, 2>(a0, a1, blocks, s);
    case 2: return pair_stream_launch<2, W, 8, 2>(a0, a1, blocks, s);
    case 4: return pair_stream_launch<4, W, 8, 2>(a0, a1, blocks, s);
    default: return pair_stream_launch<8, W, 8, 2>(a0, a1, blocks, s);
  }
}

hipError_t pair_stream_dispatch(const FxArgs& a0, const FxArgs& a1, const GroupPlan& g,
                                int blocks, hipStream_t s) {
  if (g.hold != 2) return hipErrorInvalidValue;  // not planned
  if (g.waves == 6) return pair_stream_dispatch_nt<6>(a0, a1, blocks, s);
  if (g.waves == 7) return pair_stream_dispatch_nt<7>(a0, a1, blocks, s);
  return hipErrorInvalidValue;
}

// The fused tail's two streamed launches (h and y; rs and out formed in the
// launch): the plans' shapes, as pair_stream_dispatch and stream_dispatch.
template <int NT, int W>
hipError_t gateup_fused_launch(const FxArgs& a0, const ProjPlan& p, const FuseArgs& f,
                               hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e =
      allow_full_lds(reinterpret_cast<const void*>(px_gateup_fused_kernel<NT, W, 8>), lds_set);
  if (e != hipSuccess) return e;
  FxArgs a = a0;
  a.passes = 1;
  hipLaunchKernelGGL((px_gateup_fused_kernel<NT, W, 8>), dim3(p.splits * p.blocks_per_slice),
                     dim3(kWave * (W + 2)), kStreamLds, s, a, f);
  return hipGetLastError();
}

template <int W>
hipError_t gateup_fused_dispatch_nt(const FxArgs& a, const ProjPlan& p, const FuseArgs& f,
                                    hipStream_t s) {
  switch (token_blocks(a.b)) {
    case 1: return gateup_fused_launch<1, W>(a, p, f, s);
    case 2: return gateup_fused_launch<2, W>(a, p, f, s);
    case 4: return gateup_fused_launch<4, W>(a, p, f, s);
    default: return gateup_fused_launch<8, W>(a, p, f, s);
  }
}

// 6 consumer waves only: with 7 (9 waves a block, 168 registers a wave) the
// y wave's registers no longer fit and spill (launch_tail takes the four
// launches for such plans).
hipError_t gateup_fused_dispatch(const FxArgs& a, const ProjPlan& p, const FuseArgs& f,
                                 hipStream_t s) {
  if (!p.stream || !a.partials || p.hold != 1 || p.pf != 8 || p.waves != 6)
    return hipErrorInvalidValue;
  return gateup_fused_dispatch_nt<6>(a, p, f, s);
}

template <int NT, int W>
hipError_t pair_fused_launch(const FxArgs& a0, const FxArgs& a1, int blocks, const FuseArgs& f,
                             hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e =
      allow_full_lds(reinterpret_cast<const void*>(px_pair_fused_kernel<NT, W, 8>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((px_pair_fused_kernel<NT, W, 8>), dim3(blocks), dim3(kWave * (W + 1)),
                     kStreamLds, s, a0, a1, f);
  return hipGetLastError();
}

template <int W>
hipError_t pair_fused_dispatch_nt(const FxArgs& a0, const FxArgs& a1, int blocks,
                                  const FuseArgs& f, hipStream_t s) {
  switch (token_blocks(a0.b)) {
    case 1: return pair_fused_launch<1, W>(a0, a1, blocks, f, s);
    case 2: return pair_fused_launch<2, W>(a0, a1, blocks, f, s);
    case 4: return pair_fused_launch<4, W>(a0, a1, blocks, f, s);
    default: return pair_fused_launch<8, W>(a0, a1, blocks, f, s);
  }
}

hipError_t pair_fused_dispatch(const FxArgs& a0, const FxArgs& a1, const GroupPlan& g, int blocks,
                               const FuseArgs& f, hipStream_t s) {
  if (!g.stream || g.hold != 2) return hipErrorInvalidValue;  // not planned
  if (g.waves == 6) return pair_fused_dispatch_nt<6>(a0, a1, blocks, f, s);
  if (g.waves == 7) return pair_fused_dispatch_nt<7>(a0, a1, blocks, f, s);
  return hipErrorInvalidValue;
}

template <int W, int H>
hipError_t group_dispatch_nt(const FxArgs& a0, const FxArgs& a1, int blocks0, int blocks,
                             size_t lds, hipStream_t s) {
  switch (token_blocks(a0.b)) {
    case 1: return group_launch<1, W, H>(a0, a1, blocks0, blocks, lds, s);
    case 2: return group_launch<2, W, H>(a0, a1, blocks0, blocks, lds, s);
    case 4: return group_launch<4, W, H>(a0, a1, blocks0, blocks, lds, s);
    default:
      if (H) return hipErrorInvalidValue;  // not planned (more than 4 token blocks)
      return group_launch<8, W, 0>(a0, a1, blocks0, blocks, lds, s);
  }
}

}  // namespace

// CUs of the current device (256 on MI355X), queried once per device; 256
// when there is no device to ask (the host-side plan checks).
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];  // zero: not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const bool slot = dev >= 0 && dev < kMaxDevices;
  if (slot) {
    const int v = cus[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  if (slot) cus[dev].store(v, std::memory_order_relaxed);
  return v;
}

ProjPlan plan_projection(int b, int rows, int K, bool always_partials, const ProjTuning& t) {
  return make_plan(b, rows, K, always_partials, t);
}

size_t proj_partial_bytes(const ProjPlan& p, int b, int n_out, bool always) {
  const size_t tok = 16 * (size_t)token_blocks(b);  // padded tokens are stored too
  return (p.splits > 1 || p.passes > 1 || p.stream || always) ? sizeof(float) * (size_t)p.splits * tok * n_out
                                                   : 0;
}

// The CUs split between the two projections (each keeping its K slices),
// waves per block 7 or 8: the split that minimizes the longest wave stream
// (units per wave times k steps per unit), then the fewest idle blocks.
// With a multi-pass plan on either side, both run in the multi-pass kernel:
// 8 or 12 waves, the split with the shortest longest wave stream (units per
// wave times k steps per unit, all passes), then the most blocks.
GroupPlan plan_group_mp(int b, const ProjPlan& p0, int rows0, const ProjPlan& p1, int rows1) {
  const int cu = device_cu_count();
  const int tok = 16 * token_blocks(b);
  GroupPlan best{0, 0, 0, 0, 0, 0};
  const long long n0 = (long long)(p0.passes > 1 ? p0.passes : 1) * (p0.k_per_split / kKStep);
  const long long n1 = (long long)(p1.passes > 1 ? p1.passes : 1) * (p1.k_per_split / kKStep);
  long long best_cost = -1;
  int best_blocks = 0;
  for (int w : {8, 12}) {
    for (int bps0 = 1; bps0 * p0.splits < cu; ++bps0) {
      const int bps1 = (cu - bps0 * p0.splits) / p1.splits;
      if (bps1 < 1) break;
      const int pw0 = ((rows0 / 16) + bps0 * w - 1) / (bps0 * w);
      const int pw1 = ((rows1 / 16) + bps1 * w - 1) / (bps1 * w);
      const int pw = pw0 > pw1 ? pw0 : pw1;
      if (pw > 4 || (w == 12 && tok == 64 && pw > 1) || (tok == 128 && pw > 1))
        continue;  // registers: as the plan's
      const long long c0 = pw0 * n0, c1 = pw1 * n1;
      const long long cost = c0 > c1 ? c0 : c1;
      const int blocks = bps0 * p0.splits + bps1 * p1.splits;
      if (best_cost < 0 || cost < best_cost || (cost == best_cost && blocks > best_blocks)) {
        best_cost = cost;
        best_blocks = blocks;
        best = GroupPlan{bps0, bps1, w, pw, 1, 0};
      }
    }
  }
  return best;
}

// Both streamed with the same consumer waves: one grid in which block g
// runs split g / bps of each plan in turn, each wave one unit of each (the
// plans' own blocks per split and K ranges, so the sums of the plans' own
// launches).  The grid is the larger of the two; none when it exceeds the
// CUs.
GroupPlan plan_group_stream(const ProjPlan& p0, int rows0, const ProjPlan& p1, int rows1) {
  const int cu = device_cu_count();
  if (p0.waves != p1.waves || p0.hold != 1 || p1.hold != 1) return GroupPlan{};
  if (p0.blocks_per_slice * p0.splits > cu || p1.blocks_per_slice * p1.splits > cu)
    return GroupPlan{};
  (void)rows0;
  (void)rows1;
  return GroupPlan{p0.blocks_per_slice, p1.blocks_per_slice, p0.waves, 2, 0, 1};
}

GroupPlan plan_group(int b, const ProjPlan& p0, int rows0, const ProjPlan& p1, int rows1) {
  if (p0.stream || p1.stream)
    return (p0.stream && p1.stream) ? plan_group_stream(p0, rows0, p1, rows1) : GroupPlan{};
  if (p0.passes > 1 || p1.passes > 1) return plan_group_mp(b, p0, rows0, p1, rows1);
  const int cu = device_cu_count();
  const int tok = 16 * token_blocks(b);
  GroupPlan best{0, 0, 0, 0, 0, 0};
  long long best_cost = -1;
  int best_blocks = 0;
  for (int w = 7; w <= 8; ++w) {
    for (int bps0 = 1; bps0 * p0.splits < cu; ++bps0) {
      const int bps1 = (cu - bps0 * p0.splits) / p1.splits;
      if (bps1 < 1) break;
      const long long pw0 = ((rows0 / 16) + (long long)bps0 * w - 1) / ((long long)bps0 * w);
      const long long pw1 = ((rows1 / 16) + (long long)bps1 * w - 1) / ((long long)bps1 * w);
      const long long c0 = pw0 * (p0.k_per_split / kKStep);
      const long long c1 = pw1 * (p1.k_per_split / kKStep);
      const long long cost = c0 > c1 ? c0 : c1;
      const int blocks = bps0 * p0.splits + bps1 * p1.splits;
      if (best_cost < 0 || cost < best_cost || (cost == best_cost && blocks > best_blocks)) {
        best_cost = cost;
        best_blocks = blocks;
        best = GroupPlan{bps0, bps1, w, (tok <= 64 && pw0 <= 4 && pw1 <= 4) ? 4 : 0, 0, 0};
      }
    }
  }
  return best;  // waves == 0: the CUs cannot hold both grids
}

// The gate/up launch that forms h itself (and y beside it when lat is
// given): the fused tail's first launch and moetail_gate_up.
hipError_t gate_up_fused(const uint16_t* Wg, const uint16_t* Wu, int tiled, int I, int H,
                         const uint16_t* X, int b, uint16_t* h, const ProjPlan& plan,
                         f32x4_t* part, size_t part_bytes, unsigned* counters,
                         const uint16_t* lat, int tp, const uint16_t* gamma, float eps, int L,
                         uint16_t* y, hipStream_t s) {
  FxArgs gu{Wg, Wu, I, 2 * I, H, X, b, plan.k_per_split, plan.blocks_per_slice, plan.pitch, part,
            nullptr, nullptr, tiled};
  FuseArgs f{};
  f.counters = counters;
  f.out = h;
  f.splits0 = f.splits1 = (H + plan.k_per_split - 1) / plan.k_per_split;
  f.bytes0 = f.bytes1 = (uint32_t)part_bytes;
  f.lat = lat;
  f.gamma = gamma;
  f.y = y;
  f.tp = tp;
  f.L = L;
  f.eps = eps;
  return gateup_fused_dispatch(gu, plan, f, s);
}

bool gate_up_fusable(int b, const ProjPlan& plan, int I) {
  return plan.stream && plan.waves == 6 && proj_partial_bytes(plan, b, 2 * I, true) <= 0x7fffffff;
}

hipError_t launch_gate_up_h(const uint16_t* Wg, const uint16_t* Wu, int tiled, int I, int H,
                            const uint16_t* X, int b, uint16_t* h, const ProjPlan& plan,
                            float* partials, unsigned* counters, const uint16_t* lat, int tp,
                            const uint16_t* gamma, float eps, int L, uint16_t* y,
                            hipStream_t s) {
  if (counters && gate_up_fusable(b, plan, I))
    return gate_up_fused(Wg, Wu, tiled, I, H, X, b, h, plan,
                         reinterpret_cast<f32x4_t*>(partials),
                         proj_partial_bytes(plan, b, 2 * I, true), counters, lat, tp, gamma, eps,
                         L, y, s);
  // (plans the fused kernel does not take: the separate launches, the same bits)
  hipError_t e = launch_gate_up(Wg, Wu, tiled, I, H, X, b, h, plan, partials, s);
  if (e == hipSuccess && lat) e = launch_latent_norm(lat, tp, b, L, gamma, eps, y, s);
  return e;
}

hipError_t launch_tail(const TailArgs& a, const ProjPlan& gate_up, const ProjPlan& down,
                       const ProjPlan& up, const GroupPlan& g, hipStream_t s) {
  const int b = a.b;
  const int ntb = token_blocks(b);
  f32x4_t* part = reinterpret_cast<f32x4_t*>(a.partials);
  f32x4_t* up_part = reinterpret_cast<f32x4_t*>(reinterpret_cast<char*>(a.partials) +
                                                a.down_part_bytes);
  const size_t gu_bytes = proj_partial_bytes(gate_up, b, 2 * a.I, true);
  const size_t dn_bytes = proj_partial_bytes(down, b, a.H, true);
  const size_t up_bytes = proj_partial_bytes(up, b, a.H, true);
  if (a.counters && gate_up.stream && gate_up.waves == 6 && g.stream && gu_bytes <= 0x7fffffff &&
      dn_bytes <= 0x7fffffff && up_bytes <= 0x7fffffff) {
    // Two launches: gate/up forming h (and y beside it), then the down and
    // up projections forming rs and out -- the same sums and roundings as
    // the four launches below.
    hipError_t e = gate_up_fused(a.w_gate, a.w_upw, a.tiled, a.I, a.H, a.x, b, a.h, gate_up, part,
                                 gu_bytes, a.counters, a.lat, a.tp, a.gamma, a.eps, a.L, a.y, s);
    if (e != hipSuccess) return e;
    FxArgs dn{a.w_down, nullptr, a.H, a.H, a.I, a.h, b, down.k_per_split, g.bps0, down.pitch,
              part, nullptr, nullptr, a.tiled};
    FxArgs upa{a.w_up, nullptr, a.H, a.H, a.L, a.y, b, up.k_per_split, g.bps1, up.pitch,
               up_part, nullptr, nullptr, a.tiled};
    FuseArgs f2{};
    f2.counters = a.counters + a.I / 16;
    f2.out = a.out;
    f2.rs = a.rs;
    f2.splits0 = (a.I + down.k_per_split - 1) / down.k_per_split;
    f2.splits1 = (a.L + up.k_per_split - 1) / up.k_per_split;
    f2.bytes0 = (uint32_t)dn_bytes;
    f2.bytes1 = (uint32_t)up_bytes;
    const int g0 = g.bps0 * down.splits, g1 = g.bps1 * up.splits;
    return pair_fused_dispatch(dn, upa, g, g0 > g1 ? g0 : g1, f2, s);
  }
  // 1. gate/up partials
  FxArgs gu{a.w_gate, a.w_upw, a.I, 2 * a.I, a.H, a.x, b, gate_up.k_per_split,
            gate_up.blocks_per_slice, gate_up.pitch, part, nullptr, nullptr, a.tiled};
  hipError_t e = fx_dispatch(gu, gate_up, s);
  if (e != hipSuccess) return e;
  // 2. h from the gate/up partials, beside y from the latent partials
  const int lat_waves = (a.L + kBlockCols - 1) / kBlockCols;
  const int threads = kWave * lat_waves;
  const int64_t red_items = (int64_t)(a.I / 16) * ntb * kWave;
  const int red_blocks = (int)((red_items + threads - 1) / threads);
  hipLaunchKernelGGL(tail_mid_kernel, dim3(red_blocks + b), dim3(threads), 0, s, part,
                     gate_up.splits, b, ntb, a.I, a.h, red_blocks, a.lat, a.tp, a.L, a.gamma,
                     a.eps, a.y);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 3. down and up projections in one grid (the gate/up partials are consumed)
  FxArgs dn{a.w_down, nullptr, a.H, a.H, a.I, a.h, b, down.k_per_split, g.bps0, down.pitch,
            part, nullptr, nullptr, a.tiled};
  FxArgs upa{a.w_up, nullptr, a.H, a.H, a.L, a.y, b, up.k_per_split, g.bps1, up.pitch, up_part,
             nullptr, nullptr, a.tiled};
  const int blocks0 = g.bps0 * down.splits;
  const int blocks = blocks0 + g.bps1 * up.splits;
  const size_t lds = down.lds > up.lds ? down.lds : up.lds;
  if (g.stream) {
    const int g0 = g.bps0 * down.splits, g1 = g.bps1 * up.splits;
    e = pair_stream_dispatch(dn, upa, g, g0 > g1 ? g0 : g1, s);
  } else if (!g.waves) {
    // no grid holds both (8 token blocks, one unit a wave): two launches of
    // the same plans, so the same sums
    dn.blocks_per_slice = down.blocks_per_slice;
    upa.blocks_per_slice = up.blocks_per_slice;
    e = fx_dispatch(dn, down, s);
    if (e == hipSuccess) e = fx_dispatch(upa, up, s);
  } else if (g.mp) {
    dn.passes = down.passes > 1 ? down.passes : 1;
    upa.passes = up.passes > 1 ? up.passes : 1;
    e = group_mp_dispatch(dn, upa, g, blocks0, blocks, lds, s);
  } else if (g.waves == 7)
    e = g.hold ? group_dispatch_nt<7, 4>(dn, upa, blocks0, blocks, lds, s)
               : group_dispatch_nt<7, 0>(dn, upa, blocks0, blocks, lds, s);
  else if (g.waves == 8)
    e = g.hold ? group_dispatch_nt<8, 4>(dn, upa, blocks0, blocks, lds, s)
               : group_dispatch_nt<8, 0>(dn, upa, blocks0, blocks, lds, s);
  else
    e = hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  // 4. rs, then out = up + rs
  const int64_t out_items = (int64_t)(a.H / 16) * ntb * kWave;
  hipLaunchKernelGGL(tail_out_kernel, dim3((unsigned)((out_items + 255) / 256)), dim3(256), 0, s,
                     part, down.splits, up_part, up.splits, b, ntb, a.H, a.rs, a.out);
  return hipGetLastError();
}

hipError_t launch_pack_weights(const uint16_t* w, int64_t n, int k, uint16_t* packed,
                               hipStream_t s) {
  const int64_t pieces = n * k / 8;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s,
                     w, n, k, packed);
  return hipGetLastError();
}

template <int NT, int kS>
hipError_t local_launch(const LocalArgs& a, hipStream_t s) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e =
      allow_full_lds(reinterpret_cast<const void*>(px_local_kernel<NT, kS, 8>), lds_set);
  if (e != hipSuccess) return e;
  constexpr int kT = kLocalWaves / kS;
  const int blocks = (a.N / 16 + kT - 1) / kT;
  hipLaunchKernelGGL((px_local_kernel<NT, kS, 8>), dim3(blocks), dim3(kWave * (kLocalWaves + 1)),
                     kLocalLds<NT>, s, a);
  return hipGetLastError();
}

// The streamed plans whose K splits one block holds: 4 splits (2 row tiles
// a block: 224 blocks for 7168 rows) up to 64 tokens, or 8 at one token
// block.  Other plans keep the split-K launch and its sum launch.
bool linear_local(int b, const ProjPlan& p) {
  if (!p.stream || p.passes > 1) return false;
  const int nt = token_blocks(b);
  return (p.splits == 4 && nt <= 4) || (p.splits == 8 && nt == 1);
}

hipError_t local_dispatch(const LocalArgs& a, const ProjPlan& p, hipStream_t s) {
  switch (token_blocks(a.b) * 10 + p.splits) {
    case 14: return local_launch<1, 4>(a, s);
    case 18: return local_launch<1, 8>(a, s);
    case 24: return local_launch<2, 4>(a, s);
    case 44: return local_launch<4, 4>(a, s);
    default: return hipErrorInvalidValue;  // not a shape linear_local takes
  }
}

hipError_t launch_linear(const uint16_t* W, int tiled, int N, int K, const uint16_t* X, int b,
                         const uint16_t* rs, uint16_t* out, const ProjPlan& plan,
                         float* partials, hipStream_t s) {
  if (linear_local(b, plan)) {
    const LocalArgs la{W, X, rs, out, N, K, b, tiled, plan.k_per_split};
    return local_dispatch(la, plan, s);
  }
  const bool split = plan.splits > 1 || plan.passes > 1 || plan.stream;  // (streamed: always partials)
  f32x4_t* part = reinterpret_cast<f32x4_t*>(partials);
  FxArgs a{W, nullptr, N, N, K, X, b, plan.k_per_split, plan.blocks_per_slice, plan.pitch,
           split ? part : nullptr, rs, out, tiled};
  hipError_t e = fx_dispatch(a, plan, s);
  if (e != hipSuccess || !split) return e;
  const int ntb = token_blocks(b);
  const int64_t threads = (int64_t)(N / 16) * ntb * kWave;
  hipLaunchKernelGGL(split_reduce_kernel<kLinear>, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     0, s, part, plan.splits, b, ntb, N, rs, out);
  return hipGetLastError();
}

hipError_t launch_projection_partials(const uint16_t* W0, const uint16_t* W1, int n0, int N, int K,
                                      const uint16_t* X, int b, int tiled, const ProjPlan& plan,
                                      float* partials, hipStream_t s) {
  FxArgs a{W0, W1, n0, N, K, X, b, plan.k_per_split, plan.blocks_per_slice, plan.pitch,
           reinterpret_cast<f32x4_t*>(partials), nullptr, nullptr, tiled};
  return fx_dispatch(a, plan, s);
}

hipError_t launch_gate_up(const uint16_t* Wg, const uint16_t* Wu, int tiled, int I, int H,
                          const uint16_t* X, int b, uint16_t* h, const ProjPlan& plan,
                          float* partials, hipStream_t s) {
  // Gate rows [0, I) and up rows [I, 2I) in one grid; SiLU in the reduction.
  f32x4_t* part = reinterpret_cast<f32x4_t*>(partials);
  FxArgs a{Wg, Wu, I, 2 * I, H, X, b, plan.k_per_split, plan.blocks_per_slice, plan.pitch,
           part, nullptr, nullptr, tiled};
  hipError_t e = fx_dispatch(a, plan, s);
  if (e != hipSuccess) return e;
  const int ntb = token_blocks(b);
  const int64_t threads = (int64_t)(I / 16) * ntb * kWave;
  hipLaunchKernelGGL(split_reduce_kernel<kGateUp>, dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, s, part, plan.splits, b, ntb, I, nullptr, h);
  return hipGetLastError();
}

}  // namespace moetail
