/*
 * moetail.h -- C ABI of libmoetail, the MoE decode tail on one MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [tail]         vllm.models.muse_spark.nvidia.specialized_decode.cutedsl.moe.tail
 *   [tail_runtime] vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.tail_runtime
 *   [shared]       vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.shared
 *
 * Conventions for every entry point:
 *   - BF16 arrays are uint16_t bit patterns.  Every array pointer is a DEVICE
 *     pointer to dense row-major memory owned by the caller; the library
 *     keeps no pointer after the call returns and allocates nothing (as
 *     the [tail] BoundTail run call is capturable and allocation-free).
 *     Scratch, where an entry point needs any, is the caller's workspace,
 *     sized by moetail_workspace_bytes.
 *   - BF16/FP32 array pointers must be 16-byte aligned (the kernels move
 *     8 BF16 columns per 16-byte access); index and route-weight arrays
 *     4-byte (FP32) or 2-byte (BF16) aligned; the workspace 256-byte aligned.
 *   - Every call validates all of its arguments before it enqueues anything
 *     ([tail] _check_tail_args: a refused call launches nothing).  A refused
 *     call returns a negative status and leaves every buffer untouched.
 *   - b == 0 returns MOETAIL_OK at once, before any other check, and
 *     enqueues nothing ([tail] BoundTail.run returns for zero rows first).
 *   - Work is enqueued asynchronously on `stream` (NULL = the default
 *     stream); nothing synchronizes with the host, so the calls can be
 *     captured into a HIP graph.  Results are deterministic: the same inputs
 *     give the same bits on every call.
 *   - Every BF16 word the library writes is rounded to nearest even from
 *     FP32, and a -0 result is written as +0 (the rule of the [tail]
 *     _TpTailKernel epilogue and of the [shared] SharedBase.push stores).
 */
#ifndef MOETAIL_H
#define MOETAIL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOETAIL_OK 0
#define MOETAIL_EINVAL (-1)       /* null pointer, bad shape, dtype or alignment */
#define MOETAIL_EUNSUPPORTED (-2) /* outside the library's limits below */
#define MOETAIL_EWORKSPACE (-3)   /* workspace missing or too small */
#define MOETAIL_EHIP (-4)         /* a HIP launch failed */

/* Route-weight dtypes ([tail] _check_tail_args: BF16 or FP32). */
#define MOETAIL_F32 0
#define MOETAIL_BF16 1

/* Norm modes of moetail_finalize (its weight_before_norm argument). */
#define MOETAIL_NORM_GAIN_AFTER 0 /* n = (x * inv) * g */
#define MOETAIL_NORM_GAIN_FIRST 1 /* weight_before_norm: s = x * g, n = s * inv */
#define MOETAIL_NO_NORM 2         /* [tail_runtime] Kimi finalize: n = x */

/* Weight layouts of the projections (their w_layout argument). */
#define MOETAIL_W_ROWS 0  /* dense row-major [N][K]: row n makes output column n */
#define MOETAIL_W_TILED 1 /* the tiled copy moetail_pack_weights makes */

/* Operation ids for moetail_workspace_bytes. */
#define MOETAIL_OP_FINALIZE 0
#define MOETAIL_OP_TP_FINALIZE 1
#define MOETAIL_OP_COMBINE_NORM_UPPROJ 2
#define MOETAIL_OP_SHARED_EXPERT 3
#define MOETAIL_OP_TAIL 4
#define MOETAIL_OP_PROJECTION 5
#define MOETAIL_OP_GATE_UP 6

/* Projection kinds of moetail_set_projection_tuning. */
#define MOETAIL_PROJ_UPPROJ 0 /* the up projection (moetail_combine_norm_upproj, the tail's) */
#define MOETAIL_PROJ_GATEUP 1 /* the shared expert's gate/up projection */
#define MOETAIL_PROJ_DOWN 2   /* the shared expert's down projection */

/* Limits.  P (and L) % 8 == 0 ([tail] 8-column fragments). */
#define MOETAIL_MAX_WIDTH 8192  /* P, L: rows held in registers, 512 columns per wave */
#define MOETAIL_MAX_TP 32       /* [tail] _TailReduceKernel: tp between 1 and 32 */
#define MOETAIL_MAX_ROUTES 32   /* K */
#define MOETAIL_MAX_TOKENS 65535
#define MOETAIL_MAX_GEMM_TOKENS 128 /* b of the two projections */
#define MOETAIL_MAX_GEMM_K 32768    /* H and I of the shared expert */

/*
 * EP finalize ([tail] module docstring, the expert-parallel case):
 * for every simulated rank d and token t, over the routes k local to d in
 * ascending order, with x the route's row and w its weight,
 *     g       = fp32(gamma) + gain_center
 *     s       = x * g  (weight_before_norm)   or   x
 *     inv     = 1 / sqrt(sum_of_squares(s) * fp32(1/P) + eps)
 *     n       = s * inv  (weight_before_norm) or   (x * inv) * g
 *     partial = bf16(sum_k n * w)              FP32 from +0.0
 * and, when `out` is given, the rank combine ([tail] _TailReduceKernel)
 *     out[t]  = bf16(sum_{d=0}^{tp-1} fp32(partial[d][t]))   FP32 from +0.0.
 * weight_before_norm is the norm mode: MOETAIL_NORM_GAIN_AFTER (0, false),
 * MOETAIL_NORM_GAIN_FIRST (1, true), or MOETAIL_NO_NORM (2: the finalize of
 * the [tail_runtime] module docstring, with no per-route norm,
 *     partial = bf16(sum_k fp32(x) * w)        FP32 from +0.0,
 * where gamma, gain_center and eps are not used and gamma may be NULL).
 *
 *   rows          [tp][rows_per_rank][P] BF16: rank d's GEMM2 output rows.
 *   permuted_idx  [tp][b][K] int32: row of route k of token t in rank d's
 *                 rows; a value outside [0, rows_per_rank) means the route
 *                 is not local to rank d (it contributes nothing there).
 *   route_w       [b][K] FP32 or BF16 (route_w_dtype): full top-K weights.
 *   gamma         [P] BF16 norm weight (ones when the norm has none); NULL
 *                 allowed with MOETAIL_NO_NORM.
 *   partials      [tp][b][P] BF16 written (the resident rank-partial
 *                 buffer), or NULL when only `out` is wanted.
 *   out           [b][P] BF16 written, or NULL for partials only.
 *   At least one of partials / out must be given.  With out alone the
 *   combine happens in the launch that forms the partials (they are never
 *   written); with both, out is the rank-order sum of the written partials.
 *   The results are the same bits either way.
 *   eps >= 0 and finite; gain_center finite.
 *   Limits: 1 <= K <= 32, 1 <= tp <= 32, 8 <= P <= 8192, P % 8 == 0,
 *   b <= 65535, rows_per_rank >= 1.
 */
int moetail_finalize(const uint16_t* rows, int64_t rows_per_rank,
                     const int32_t* permuted_idx, const void* route_w,
                     int route_w_dtype, const uint16_t* gamma,
                     float gain_center, float eps, int weight_before_norm,
                     int b, int K, int P, int tp, uint16_t* partials,
                     uint16_t* out, hipStream_t stream);

/*
 * Expert-TP finalize ([tail] module docstring, the expert-TP case, and
 * _TpTailKernel): every rank holds a K-partial of every route row.
 *     x_r    = bf16(sum_{d=0}^{tp-1} fp32(kpartials[d][idx[t][k]]))  FP32 from +0.0
 *     out[t] = bf16(sum_k fp32(n(x_r) * w[t][k]))   routes in order, from +0.0
 * with n() the normalization of moetail_finalize (same gain, eps, switch).
 *
 *   kpartials     [tp][num_rows][P] BF16.
 *   permuted_idx  [b][K] int32 (the same on every rank); a value outside
 *                 [0, num_rows) marks an absent route (contributes nothing).
 *   route_w       [b][K] FP32 or BF16.   gamma [P] BF16.   out [b][P] BF16.
 *   workspace     at least moetail_workspace_bytes(MOETAIL_OP_TP_FINALIZE,
 *                 b, K, P, tp) bytes, 256-byte aligned, and ZERO BEFORE ITS
 *                 FIRST USE (every call leaves it so).  With tp <= 8 the
 *                 finalize is one pass: two blocks a token (the row's two
 *                 halves) keep x_r on chip and meet once through the
 *                 workspace's first words ([b][2] flags, then each half's
 *                 sum-of-squares block totals [b][2][K][8] FP32); a wait
 *                 for the other half is bounded (moetail_set_tp_wait_limit)
 *                 and past it a block forms the other half's totals itself,
 *                 so results never depend on the two running at once.  With
 *                 more ranks (or tp = 0 in the size query) the workspace
 *                 also holds the two-pass path's x_r rows [b][K][P] BF16
 *                 and their 512-column block totals [b][K][ceil(P/512)] FP32.
 *                 Calls that overlap must not share a workspace.
 *   Limits: 1 <= K <= 32, 1 <= tp <= 32, 8 <= P <= 8192, P % 8 == 0.
 */
int moetail_tp_finalize(const uint16_t* kpartials, int64_t num_rows,
                        const int32_t* permuted_idx, const void* route_w,
                        int route_w_dtype, const uint16_t* gamma,
                        float gain_center, float eps, int weight_before_norm,
                        int b, int K, int P, int tp, uint16_t* out,
                        void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * Latent combine + RMSNorm + up projection ([tail_runtime] module docstring:
 * the latent partials are all-reduced and RMS-normalized, then the K-split
 * up projection; MoeTailWeights: shard [7168/TP, 3584] and RMS weight):
 *     l[t]      = bf16(sum_{d=0}^{tp-1} fp32(latent_partials[d][t]))  FP32 from +0.0
 *     y[t]      = bf16((l * inv) * fp32(gamma)),  inv = 1/sqrt(ss(l)*fp32(1/L) + eps)
 *     out[t][n] = bf16(sum_k fp32(w_up[n][k]) * fp32(y[t][k]) + fp32(rs[t][n]))
 * (FP32 accumulation on the matrix cores; the rs add is skipped when rs is NULL).
 *
 *   latent_partials [tp][b][L] BF16.   gamma [L] BF16.
 *   w_up            [N][L] BF16 (row n makes output column n).
 *   rs              [b][N] BF16 shared-expert reduce-scatter partial, or NULL.
 *   normed          [b][L] BF16 written (y), or NULL.
 *   out             [b][N] BF16 written.
 *   w_layout        MOETAIL_W_ROWS or MOETAIL_W_TILED: the layout of w_up.
 *   workspace       at least moetail_workspace_bytes(MOETAIL_OP_COMBINE_NORM_UPPROJ,
 *                   b, L, N, tp) bytes of device memory, 256-byte aligned.
 *   Limits: b <= 128, 1 <= tp <= 32, 32 <= L <= 8192, L % 32 == 0,
 *   N % 64 == 0.
 */
int moetail_combine_norm_upproj(const uint16_t* latent_partials, int tp,
                                const uint16_t* gamma, float eps,
                                const uint16_t* w_up, int N,
                                const uint16_t* rs, int b, int L,
                                uint16_t* normed, uint16_t* out, int w_layout,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Shared expert ([shared] module docstring and SharedUmma.owned_h / push):
 *     gs = bf16(w_gate . x),  us = bf16(w_upw . x)        FP32 accumulation
 *     h  = bf16(silu(fp32 gs) * fp32 us),  silu(z) = z / (1 + e^-z)
 *     rs = bf16(w_down . h)                               FP32 accumulation
 * (the pages name the activation but never define it; this library takes
 * SiLU).
 *
 *   x       [b][H] BF16.   w_gate, w_upw [I][H] BF16 each (a stacked [2I][H]
 *           tensor passes p and p + I*H).   w_down [H][I] BF16.
 *   h       [b][I] BF16 written, or NULL.
 *   rs      [b][H] BF16 written (the input of moetail_combine_norm_upproj).
 *   w_layout MOETAIL_W_ROWS or MOETAIL_W_TILED: the layout of the three weights.
 *   workspace at least moetail_workspace_bytes(MOETAIL_OP_SHARED_EXPERT,
 *           b, H, I, 0) bytes, 256-byte aligned.
 *   Limits: b <= 128, H % 64 == 0, I % 64 == 0, 64 <= H, I <= MOETAIL_MAX_GEMM_K.
 */
int moetail_shared_expert(const uint16_t* x, int b, int H,
                          const uint16_t* w_gate, const uint16_t* w_upw, int I,
                          const uint16_t* w_down, uint16_t* h, uint16_t* rs,
                          int w_layout, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * One skinny projection's split-K stage alone ([tail_runtime] module
 * docstring: "the K-split up projection"; [shared] SharedUmma: the gate/up
 * and down products), the stage that dominates moetail_shared_expert and
 * moetail_tail, for a caller that forms its own epilogue from the FP32
 * partial sums (an expert GEMM epilogue, say) and for timing the stage:
 *     partial[s][t][r] = sum over k in K range s, in k order, of
 *                        fp32 W[r][k] * fp32 x[t][k]        (FP32 accumulation)
 * with the plan of that stage in those calls (the same K ranges), so the
 * same partial sums.  Adding them in split order from +0 gives the sums
 * those calls round.
 *
 *   kind     MOETAIL_PROJ_GATEUP: w0 = w_gate, w1 = w_upw, each [N/2][K] BF16
 *            (rows [0, N/2) of the output are gate rows, [N/2, N) up rows);
 *            MOETAIL_PROJ_DOWN or MOETAIL_PROJ_UPPROJ: w0 [N][K], w1 NULL.
 *   x        [b][K] BF16.   w_layout MOETAIL_W_ROWS or MOETAIL_W_TILED.
 *   partials FP32, at least moetail_workspace_bytes(MOETAIL_OP_PROJECTION, b,
 *            N, K, kind) bytes, 256-byte aligned; the splits S are that size
 *            over N * T * 4, T = b rounded up to 16, 32, 64 or 128 tokens.
 *            Split s, row r, token t sits at float index
 *              4 * (((s * (N / 16) + r / 16) * (T / 16) + t / 16) * 64
 *                   + 16 * ((r % 16) / 4) + t % 16) + r % 4
 *            (the matrix cores' accumulator order); tokens t >= b hold token
 *            b - 1's sums.
 *   Limits: b <= 128, N % 16 == 0 (N % 32 with MOETAIL_PROJ_GATEUP),
 *           K % 32 == 0, K <= MOETAIL_MAX_GEMM_K.
 */
int moetail_projection_partials(int kind, const uint16_t* w0, const uint16_t* w1, int N,
                                int K, const uint16_t* x, int b, int w_layout, float* partials,
                                size_t partial_bytes, hipStream_t stream);

/*
 * The shared expert's gate/up projection and its activation in one launch
 * ([shared] module docstring: h = bf16(SiLU(x W_g^T) * (x W_u^T))), with,
 * when latent_partials is given, the latent combine + RMSNorm y of
 * moetail_combine_norm_upproj formed by the same launch beside it: the first
 * launch of moetail_tail, as a call of its own.  The K-split sums are formed
 * in the launch (per-tile counters in the workspace; the wave completing a
 * tile adds its splits in split order, the bits of the separate sum).
 *
 *   x [b][H], w_gate, w_upw [I][H], w_layout: as in moetail_shared_expert.
 *   h               [b][I] BF16 written: the bits moetail_shared_expert
 *                   writes to its h.
 *   latent_partials [tp][b][L], gamma [L], eps: as in
 *                   moetail_combine_norm_upproj; normed [b][L] BF16 written
 *                   (its normed bits).  latent_partials NULL: no y (tp,
 *                   gamma, eps, L and normed are not read).
 *   workspace       at least moetail_workspace_bytes(MOETAIL_OP_GATE_UP, b,
 *                   H, I) bytes, 256-byte aligned, ZERO BEFORE ITS FIRST USE
 *                   (it starts with the h tiles' counters; every call leaves
 *                   them at zero).
 *   Limits: those of moetail_shared_expert, and with y those of
 *   moetail_combine_norm_upproj (tp <= 32, L % 32 == 0, L <= 8192).  With
 *   plan overrides that select other kernels the work is the separate
 *   launches (the same bits).
 */
int moetail_gate_up(const uint16_t* x, int b, int H, const uint16_t* w_gate,
                    const uint16_t* w_upw, int I, uint16_t* h,
                    const uint16_t* latent_partials, int tp, const uint16_t* gamma,
                    float eps, int L, uint16_t* normed, int w_layout, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * The decode tail after the finalize in one call ([tail_runtime] module
 * docstring: the latent combine, RMSNorm and K-split up projection with the
 * shared expert's reduce-scatter partial added; [shared] for that partial):
 *     rs  = moetail_shared_expert(x)                       (as that call)
 *     out = moetail_combine_norm_upproj(latent_partials, rs) (as that call)
 * with the hidden width H as the up projection's output width N.  The
 * results are the same bits as those two calls in that order.  With the
 * library's own (streamed) plans the work is two launches (the two calls
 * take five to seven): gate/up forming h in the launch, beside y; then the down and up
 * projections as one grid forming rs and out in the launch.  (With plan
 * overrides that select other kernels: four launches, gate/up; {h, y};
 * {down, up}; {rs, out}.)
 *
 *   latent_partials [tp][b][L], gamma [L], w_up [H][L]: as in
 *                   moetail_combine_norm_upproj (N = H).
 *   x [b][H], w_gate, w_upw [I][H], w_down [H][I]: as in
 *                   moetail_shared_expert.
 *   out             [b][H] BF16 written.
 *   rs, normed, h   [b][H], [b][L], [b][I] BF16 written, or NULL (then kept
 *                   in the workspace or not kept).
 *   w_layout        MOETAIL_W_ROWS or MOETAIL_W_TILED: the layout of all four
 *                   weights.
 *   workspace       at least moetail_workspace_bytes(MOETAIL_OP_TAIL, b, L,
 *                   H, I) bytes, 256-byte aligned, ZERO BEFORE ITS FIRST USE:
 *                   it starts with the output-tile counters of the launches
 *                   that form their own split sums, which every call leaves
 *                   at zero.  A workspace used by another operation in
 *                   between must be zeroed again.
 *   Limits: those of the two calls: b <= 128, 1 <= tp <= 32, L % 32 == 0,
 *   L <= 8192, H % 64 == 0, I % 64 == 0, H, I <= MOETAIL_MAX_GEMM_K.
 */
int moetail_tail(const uint16_t* latent_partials, int tp, const uint16_t* gamma,
                 float eps, const uint16_t* w_up, int L, const uint16_t* x,
                 const uint16_t* w_gate, const uint16_t* w_upw,
                 const uint16_t* w_down, int H, int I, int b, uint16_t* out,
                 uint16_t* rs, uint16_t* normed, uint16_t* h, int w_layout,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The whole decode tail in one call, from the routed experts' GEMM2 rows to
 * the output row ([tail] module docstring for the finalize; [tail_runtime]
 * and [shared] for the rest, as in moetail_tail):
 *     latent_partials = moetail_finalize(rows, ..., partials only)
 *     out             = moetail_tail(latent_partials, ...)
 * with the finalize's width P equal to the latent width L.  The results are
 * the same bits as those two calls in that order (latent_partials is
 * written, the resident rank-partial buffer): three launches with the
 * library's own plans, every argument of both checked before the first.
 *
 *   rows .. K        as in moetail_finalize (fin_gamma, fin_eps: its gamma
 *                    [L] and eps; weight_before_norm: its norm mode).
 *   latent_partials  [tp][b][L] BF16 written.
 *   gamma .. h       as in moetail_tail (gamma [L] and eps: the latent norm's).
 *   w_layout, workspace: as in moetail_tail (workspace bytes of MOETAIL_OP_TAIL).
 *   Limits: those of moetail_finalize and moetail_tail.
 */
int moetail_decode_tail(const uint16_t* rows, int64_t rows_per_rank,
                        const int32_t* permuted_idx, const void* route_w,
                        int route_w_dtype, const uint16_t* fin_gamma,
                        float gain_center, float fin_eps, int weight_before_norm,
                        int K, uint16_t* latent_partials, int tp,
                        const uint16_t* gamma, float eps, const uint16_t* w_up,
                        int L, const uint16_t* x, const uint16_t* w_gate,
                        const uint16_t* w_upw, const uint16_t* w_down, int H,
                        int I, int b, uint16_t* out, uint16_t* rs,
                        uint16_t* normed, uint16_t* h, int w_layout,
                        void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * moetail_decode_tail without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same arguments but the workspace, the same
 * kernels and the same bits.  Its scratch (the split partials, and h and y
 * when not given) is a static device array of the library, one per GPU,
 * MOETAIL_NOALLOC_SCRATCH_BYTES long, held until the process ends; the call
 * allocates nothing.  A call whose sizes need more scratch than that (the
 * workspace moetail_decode_tail would take, moetail_workspace_bytes(
 * MOETAIL_OP_TAIL, b, L, H, I), beyond the maximum) returns
 * MOETAIL_EWORKSPACE and enqueues nothing; at L = 3584, H = 7168,
 * I = 6144 every b <= 64 fits (18.7 MiB at b = 64).  Every call on a GPU
 * shares that GPU's scratch: calls that overlap on one GPU (other streams,
 * other host threads) race and must not be issued.  The scratch starts
 * with the tail's output-tile counters, which must be zero when a call
 * starts: a static array is zero when the library loads, and every call
 * leaves them at zero.  The first call on a device looks the scratch's
 * address up (make it before any graph capture).
 */
#define MOETAIL_NOALLOC_SCRATCH_BYTES ((size_t)24 << 20)
int moetail_decode_tail_noalloc(const uint16_t* rows, int64_t rows_per_rank,
                                const int32_t* permuted_idx, const void* route_w,
                                int route_w_dtype, const uint16_t* fin_gamma,
                                float gain_center, float fin_eps, int weight_before_norm,
                                int K, uint16_t* latent_partials, int tp,
                                const uint16_t* gamma, float eps, const uint16_t* w_up,
                                int L, const uint16_t* x, const uint16_t* w_gate,
                                const uint16_t* w_upw, const uint16_t* w_down, int H,
                                int I, int b, uint16_t* out, uint16_t* rs,
                                uint16_t* normed, uint16_t* h, int w_layout,
                                hipStream_t stream);

/*
 * The tiled copy of a weight matrix, made once when the weights are loaded
 * (weights are static at decode time).  The projections read either layout
 * (their w_layout argument) and give the same bits from both; the tiled one
 * lets every wave-wide weight load read 1 KB of contiguous memory instead
 * of 64 bytes of each of 16 rows (measured on MI355X: 5.9 against 4.4 TB/s
 * for a weight stream).  Not on the pages: their kernels read row-major
 * weights through TMA into swizzled shared memory.
 *     packed[((t * k/32) + s) * 512 + 8 l + e]
 *         = w[(16 t + l % 16) * k + 32 s + 8 (l / 16) + e]
 * for every 16-row tile t, 32-column step s, lane l < 64 and e < 8: each
 * 16 x 32 block is 1 KB in the operand order of the MFMA that reads it.  A
 * stacked [2I][H] gate/up matrix packs as one [2I][H] matrix (the up half
 * starts I*H elements in, as in the row-major layout).
 *
 *   w       [n][k] BF16 row-major.   packed [n][k] elements BF16, written;
 *           it may not overlap w.
 *   Limits: n % 16 == 0, k % 32 == 0 (EUNSUPPORTED otherwise); n == 0 is OK.
 */
int moetail_pack_weights(const uint16_t* w, int64_t n, int k, uint16_t* packed,
                         hipStream_t stream);

/*
 * Workspace bytes an operation needs (0 when none):
 *   MOETAIL_OP_FINALIZE:            0
 *   MOETAIL_OP_TP_FINALIZE:         dim0 = K, dim1 = P, dim2 = tp (0: any tp)
 *   MOETAIL_OP_COMBINE_NORM_UPPROJ: dim0 = L, dim1 = N, dim2 = tp
 *   MOETAIL_OP_SHARED_EXPERT:       dim0 = H, dim1 = I
 *   MOETAIL_OP_TAIL:                dim0 = L, dim1 = H, dim2 = I
 *   MOETAIL_OP_PROJECTION:          dim0 = N, dim1 = K, dim2 = kind
 *   MOETAIL_OP_GATE_UP:             dim0 = H, dim1 = I
 * Returns 0 for an unknown op or out-of-range sizes.
 */
size_t moetail_workspace_bytes(int op, int b, int dim0, int dim1, int dim2);

/*
 * Plan overrides for one projection kind, for measurement runs and tests
 * only: every later call of this process (every device and stream) plans
 * that projection with them.  Each knob 0 leaves the library's choice:
 *   splits          K slices (their FP32 partials are added in slice order)
 *   waves           waves per block (7, 8, 14, 16; 8 or 12 multi-pass)
 *   blocks          blocks in the grid (default: one per CU)
 *   tiles_per_unit  16-row tiles a wave streams together (1 or 2)
 *   prefetch        k steps in flight per wave (4 or 8)
 *   passes          LDS slices per split (1: one; 2 or more: multi-pass)
 * All zeros restores the library's plan.  An override that names no built
 * kernel shape, or whose slice does not fit the LDS, falls back to the
 * library's plan.  The K slices fix the FP32 summation order, so an
 * override changes the projection outputs' bits (within the same error
 * bound); production callers never set one.  Setting is thread-safe; calls
 * running meanwhile use either the old or the new plan.
 * Returns MOETAIL_EINVAL for an unknown kind or a negative knob.
 */
int moetail_set_projection_tuning(int kind, int splits, int waves, int blocks,
                                  int tiles_per_unit, int prefetch, int passes);

/*
 * The one-pass expert-TP finalize's wait limit for the meeting of a token's
 * two blocks, in ticks of the GPU's 100 MHz clock (default 2,000,000: 20 ms).
 * A negative value skips the wait: every block forms its partner's totals
 * itself (slower, the same bits).  For tests of that path; process-wide.
 */
void moetail_set_tp_wait_limit(int64_t ticks);

/*
 * Plan searches and plan-cache hits so far in this process.  The projection
 * plans of a shape are searched once (per CU count and set of overrides) and
 * looked up by every later call; diagnostics only.  Either pointer may be
 * NULL.
 */
void moetail_plan_cache_stats(uint64_t* searches, uint64_t* hits);

/* A static, human-readable text for a status code. */
const char* moetail_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
