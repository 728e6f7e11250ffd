// kernels.h -- launchers of the libmoetail kernels (internal to the library).
// The host entry points validate every argument before calling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moetail.h"

// Most (rank, route) pairs one token can have.
#define MOETAIL_KMAX_PAIRS (MOETAIL_MAX_TP * MOETAIL_MAX_ROUTES)

namespace moetail {

struct EpArgs {
  const uint16_t* rows;   // [tp][R][P]
  int64_t R;
  const int32_t* idx;     // [tp][b][K]
  const void* w;          // [b][K] FP32 or BF16
  int w_bf16;
  const uint16_t* gamma;  // [P]
  float gain_center, eps;
  int wbn;  // norm mode: 0 gain after the norm, 1 gain first, 2 no norm
  int b, K, P, tp;
  uint16_t* partials;     // [tp][b][P] or null
  uint16_t* out;          // [b][P] or null
};
hipError_t launch_ep_finalize(const EpArgs& a, hipStream_t stream);

struct TpArgs {
  const uint16_t* kpart;  // [tp][num_rows][P]
  int64_t num_rows;
  const int32_t* idx;     // [b][K]
  const void* w;
  int w_bf16;
  const uint16_t* gamma;
  float gain_center, eps;
  int wbn;
  int b, K, P, tp;
  uint16_t* out;          // [b][P]
  // tp <= kTpOnePassMaxRanks: one pass, two blocks a token exchanging through
  unsigned* gen;          // workspace [b]: each token's generation (zero at first use)
  uint64_t* slots;        // workspace [b][K][ceil(P/512)]: tagged block totals
  long long wait_ticks;   // the exchange's wait limit (100 MHz ticks; < 0: none)
  // more ranks: two passes through
  uint16_t* xr;           // workspace [b][K][P]: rank-summed route rows
  float* block_total;     // workspace [b][K][ceil(P/512)]: their sum-of-squares block totals
};
constexpr int kTpOnePassMaxRanks = 8;  // the one-pass expert-TP kernel holds 8 ranks' loads
hipError_t launch_tp_finalize(const TpArgs& a, hipStream_t stream);

// Latent combine + RMSNorm: y[b][L] = bf16((bf16(sum_d lat[d]) * inv) * gamma).
hipError_t launch_latent_norm(const uint16_t* lat, int tp, int b, int L,
                              const uint16_t* gamma, float eps, uint16_t* y,
                              hipStream_t stream);

// Skinny projections on the matrix cores.  A plan fixes the K slices (and
// so the FP32 summation order) for one (b, rows, K); forced_splits > 0
// overrides the slice count.
struct ProjPlan {
  int splits;        // K slices, partials added in slice order
  int k_per_split;   // multiple of the 32-wide k step
  int pitch;         // LDS row pitch of the staged activations (elements)
  size_t lds;        // LDS bytes per block
  int waves;         // waves per block
  int mr;            // 16-row tiles per wave unit (1 or 2)
  int pf;            // k steps in flight per wave (4 or 8)
  int blocks_per_slice;
  int hold;          // units a wave keeps in registers until its stream ends
  int passes;        // LDS slices of k_per_split per split (0 or 1: one; more: the multi-pass kernel)
  int stream;        // 1: the streamed kernel (activations through an LDS chunk ring)
};
// Plan knobs: 0 = the library's choice.
struct ProjTuning {
  int splits;         // K splits
  int waves;          // waves per block
  int target_blocks;  // blocks in the grid (default: one per CU)
  int mr;             // tiles per wave unit
  int pf;             // prefetch depth
  int passes;         // LDS slices per split: 0 the plan's choice, 1 one, n >= 2 n
};
// Compute units of the current device (queried once; 256 if the query fails).
int device_cu_count();

// rows: weight rows of the grid (2I for gate/up), K: reduction length;
// always_partials: the epilogue needs the reduction kernel even unsplit.
ProjPlan plan_projection(int b, int rows, int K, bool always_partials, const ProjTuning& t);
// FP32 partial bytes of a plan (always: also for a single slice).
size_t proj_partial_bytes(const ProjPlan& p, int b, int n_out, bool always);

// Two projections in one grid: blocks_per_slice of each (keeping each
// plan's K slices), the common waves per block and units held per wave.
struct GroupPlan {
  int bps0, bps1;
  int waves;
  int hold;
  int mp;  // both in the multi-pass kernel (either plan has passes > 1)
  int stream;  // both in the streamed kernel (both plans streamed)
};
GroupPlan plan_group(int b, const ProjPlan& p0, int rows0, const ProjPlan& p1, int rows1);

// The fused tail (moetail_tail): gate/up -> {h, y} -> {down, up} -> {rs, out}.
struct TailArgs {
  const uint16_t* x;        // [b][H]
  const uint16_t* w_gate;   // [I][H]
  const uint16_t* w_upw;    // [I][H]
  const uint16_t* w_down;   // [H][I]
  int H, I;
  const uint16_t* lat;      // [tp][b][L]
  int tp;
  const uint16_t* gamma;    // [L]
  float eps;
  const uint16_t* w_up;     // [H][L]
  int L, b;
  uint16_t* h;              // [b][I] (caller's or workspace)
  uint16_t* y;              // [b][L] (caller's or workspace)
  uint16_t* rs;             // [b][H] or null
  uint16_t* out;            // [b][H]
  float* partials;          // gate/up partials, then down and up partials
  size_t down_part_bytes;   // offset of the up partials
  int tiled;                // the four weights in the tiled layout
  unsigned* counters;       // [I/16 + H/16], zero between calls (null: the
                            // sums in launches of their own)
};
hipError_t launch_tail(const TailArgs& a, const ProjPlan& gate_up, const ProjPlan& down,
                       const ProjPlan& up, const GroupPlan& g, hipStream_t stream);

// One projection's split-K stage alone: rows [0, n0) from W0, [n0, N) from
// W1; FP32 partials in the plan's layout.
hipError_t launch_projection_partials(const uint16_t* W0, const uint16_t* W1, int n0, int N, int K,
                                      const uint16_t* X, int b, int tiled, const ProjPlan& plan,
                                      float* partials, hipStream_t stream);

// The tiled copy of a [n][k] weight matrix (n % 16 == 0, k % 32 == 0).
hipError_t launch_pack_weights(const uint16_t* w, int64_t n, int k, uint16_t* packed,
                               hipStream_t stream);

// out[b][N] = bf16(W[N][K] . X[b][K] + rs), -0 as +0; tiled: W's layout.
hipError_t launch_linear(const uint16_t* W, int tiled, int N, int K, const uint16_t* X,
                         int b, const uint16_t* rs, uint16_t* out,
                         const ProjPlan& plan, float* partials,
                         hipStream_t stream);

// The gate/up projection forming h in its own launch (counters: I/16 words,
// zero between calls), with the latent norm's y beside it when lat is set;
// other plans: the separate launches.
hipError_t launch_gate_up_h(const uint16_t* Wg, const uint16_t* Wu, int tiled, int I, int H,
                            const uint16_t* X, int b, uint16_t* h, const ProjPlan& plan,
                            float* partials, unsigned* counters, const uint16_t* lat, int tp,
                            const uint16_t* gamma, float eps, int L, uint16_t* y,
                            hipStream_t stream);
// h[b][I] = bf16(silu(bf16(Wg . x)) * bf16(Wu . x)), -0 as +0.
hipError_t launch_gate_up(const uint16_t* Wg, const uint16_t* Wu, int tiled, int I, int H,
                          const uint16_t* X, int b, uint16_t* h,
                          const ProjPlan& plan, float* partials,
                          hipStream_t stream);

}  // namespace moetail
