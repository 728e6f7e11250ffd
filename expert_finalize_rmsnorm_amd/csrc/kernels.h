// kernels.h -- launchers of the libmoetail kernels (internal to the library).
// The host entry points validate every argument before calling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moetail {

struct EpArgs {
  const uint16_t* rows;   // [tp][R][P]
  int64_t R;
  const int32_t* idx;     // [tp][b][K]
  const void* w;          // [b][K] FP32 or BF16
  int w_bf16;
  const uint16_t* gamma;  // [P]
  float gain_center, eps;
  int wbn;
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
};
hipError_t launch_tp_finalize(const TpArgs& a, hipStream_t stream);

// Latent combine + RMSNorm: y[b][L] = bf16((bf16(sum_d lat[d]) * inv) * gamma).
hipError_t launch_latent_norm(const uint16_t* lat, int tp, int b, int L,
                              const uint16_t* gamma, float eps, uint16_t* y,
                              hipStream_t stream);

// Skinny projections on the matrix cores.
struct ProjPlan {
  int splits;        // K slices reduced in a fixed order (1 = no partials)
  int k_per_split;   // multiple of the k tile
};
ProjPlan plan_upproj(int b, int N, int L);
ProjPlan plan_gate_up(int b, int I, int H);
ProjPlan plan_down(int b, int H, int I);
size_t proj_partial_bytes(const ProjPlan& p, int b, int n_out);

// out[b][N] = bf16(W[N][K] . X[b][K] + rs), -0 as +0.
hipError_t launch_linear(const uint16_t* W, int N, int K, const uint16_t* X,
                         int b, const uint16_t* rs, uint16_t* out,
                         const ProjPlan& plan, float* partials,
                         hipStream_t stream);

// h[b][I] = bf16(silu(bf16(Wg . x)) * bf16(Wu . x)), -0 as +0.
hipError_t launch_gate_up(const uint16_t* Wg, const uint16_t* Wu, int I, int H,
                          const uint16_t* X, int b, uint16_t* h,
                          const ProjPlan& plan, float* partials,
                          hipStream_t stream);

}  // namespace moetail
