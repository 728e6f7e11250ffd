/*
 * oracle.h -- plain CPU oracle of the MoE decode tail (TEST INFRASTRUCTURE).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The product path (libmoetail) never links, loads or
 * calls it, and the two share no code.
 *
 * Sources (web pages, cited by title and section):
 *   [tail]         vllm.models.muse_spark.nvidia.specialized_decode.cutedsl.moe.tail
 *                  (module docstring formulas; _TailReduceKernel; _TpTailKernel and
 *                  its helpers gains / warp_sum_of_squares / normalized;
 *                  _check_tail_args; tail_weight)
 *   [tail_runtime] vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.tail_runtime
 *                  (module docstring: finalize, latent all-reduce, RMSNorm, up projection)
 *   [shared]       vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.shared
 *                  (module docstring; SharedUmma.owned_h; SharedBase.push)
 *
 * BF16 values are passed as uint16_t bit patterns.  Every array is dense
 * row-major host memory owned by the caller.  nthreads <= 0 means "use the
 * OpenMP default"; results never depend on it (threads split independent
 * tokens or output rows only).
 */
#ifndef MOETAIL_ORACLE_H
#define MOETAIL_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_W_F32 0
#define ORACLE_W_BF16 1

/* Sum-of-squares orders (oracle_set_ss_order). */
#define ORACLE_SS_W64 0 /* the wave64 tree (default) */
#define ORACLE_SS_SEQ 1 /* plain sequential sum in column order */

/* IEEE round-to-nearest-even of n floats to BF16 bit patterns. */
void oracle_bf16_round(const float* x, uint16_t* y, int64_t n);

/* The sum of squares of v[0..P), P % 8 == 0, in the order last set by
 * oracle_set_ss_order (the wave64 tree unless set). */
float oracle_sum_of_squares(const float* v, int P);
void oracle_set_ss_order(int order);

/* One route's normalization step by step, exposed for pinning:
 * 1 / sqrt(ss * fp32(1/P) + eps), correctly rounded to FP32; and a BF16
 * row x[P]'s weighted normalized FP32 products p[P] (gains
 * fp32(gamma) + gain_center, the gain before or after the norm). */
float oracle_inv_rms(float ss, int P, float eps);
void oracle_route_products(const uint16_t* x, const uint16_t* gamma, float gain_center,
                           float w, float eps, int weight_before_norm, int P, float* p);

/* EP finalize: partials[tp][b][P] from rows[tp][R][P], idx[tp][b][K],
 * w[b][K] (FP32 or BF16), gamma[P]; out[b][P] (rank combine) if non-NULL. */
void oracle_finalize(const uint16_t* rows, int64_t R, const int32_t* idx,
                     const void* w, int w_dtype, const uint16_t* gamma,
                     float gain_center, float eps, int weight_before_norm,
                     int b, int K, int P, int tp,
                     uint16_t* partials, uint16_t* out, int nthreads);

/* The finalize without a per-route norm (Kimi): route-weighted sum. */
void oracle_finalize_plain(const uint16_t* rows, int64_t R, const int32_t* idx,
                           const void* w, int w_dtype, int b, int K, int P, int tp,
                           uint16_t* partials, uint16_t* out, int nthreads);

/* Rank-order combine: out[b][P] = bf16(sum over d of partials[d][b][P]). */
void oracle_rank_combine(const uint16_t* partials, int tp, int b, int P,
                         uint16_t* out);

/* Expert-TP finalize: kpart[tp][num_rows][P], idx[b][K] -> out[b][P]. */
void oracle_tp_finalize(const uint16_t* kpart, int64_t num_rows,
                        const int32_t* idx, const void* w, int w_dtype,
                        const uint16_t* gamma, float gain_center, float eps,
                        int weight_before_norm, int b, int K, int P, int tp,
                        uint16_t* out, int nthreads);

/* Latent combine + RMSNorm + up projection:
 * lat[tp][b][L], gamma[L], w_up[N][L], rs[b][N] or NULL ->
 * normed[b][L] (or NULL), out[b][N]. */
void oracle_combine_norm_upproj(const uint16_t* lat, int tp,
                                const uint16_t* gamma, float eps,
                                const uint16_t* w_up, int N,
                                const uint16_t* rs, int b, int L,
                                uint16_t* normed, uint16_t* out, int nthreads);

/* Shared expert: x[b][H], w_gate/w_up[I][H], w_down[H][I] ->
 * h[b][I] (or NULL), rs[b][H]. */
void oracle_shared_expert(const uint16_t* x, int b, int H,
                          const uint16_t* w_gate, const uint16_t* w_upw, int I,
                          const uint16_t* w_down, uint16_t* h, uint16_t* rs,
                          int nthreads);

#ifdef __cplusplus
}
#endif
#endif
