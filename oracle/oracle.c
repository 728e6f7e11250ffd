/*
 * oracle.c -- plain, slow, obviously correct CPU oracle of the MoE decode
 * tail.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it; the product library never does.
 *
 * Every method on the pages reaches an exactly defined result once the
 * order of the FP32 operations is fixed, so the oracle is that definition
 * written out in scalar loops, in the order the pages give:
 *
 *   * FP32 arithmetic, each operation rounded on its own (built with
 *     -ffp-contract=off: no fused multiply-add anywhere);
 *   * BF16 round-to-nearest-even exactly where the pages round;
 *   * a BF16 word that would be -0 is written as +0 where a result leaves
 *     a kernel (the rule stated in the [tail] _TpTailKernel docstring and
 *     at the [shared] SharedBase.push stores).
 *
 * Readings taken where the pages leave a step open are stated next to the
 * code that takes them.  Page keys ([tail], [tail_runtime], [shared]) are
 * defined in oracle.h.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- BF16 -- */

/* FP32 value of a BF16 bit pattern: BF16 is the upper half of an FP32. */
static float f32_of(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Nearest BF16 to f, ties to even (IEEE 754 roundTiesToEven).  The 16
 * discarded bits are compared with one half unit of the kept 16 bits; a
 * carry out of the mantissa moves the exponent up, which also turns the
 * largest finite values into infinity as the standard requires.  NaN stays
 * NaN (quiet bit set). */
static uint16_t bf16_of(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (kept & 1u)))
        kept += 1;
    return (uint16_t)kept;
}

/* -0 leaves as +0 (the only change). */
static uint16_t plus_zero(uint16_t h) { return h == 0x8000u ? 0 : h; }

void oracle_bf16_round(const float* x, uint16_t* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = bf16_of(x[i]);
}

/* Route weight (t, k) widened to FP32 ([tail] _TpTailKernel: the weight is
 * read as Float32 whatever its dtype; _check_tail_args: BF16 or FP32). */
static float route_weight(const void* w, int w_dtype, int64_t i) {
    if (w_dtype == ORACLE_W_BF16) return f32_of(((const uint16_t*)w)[i]);
    return ((const float*)w)[i];
}

/* ------------------------------------------------------ sum of squares -- */

/* The sum-of-squares order, chosen by oracle_set_ss_order (W64 unless set):
 * the tree below, or the plain sequential sum (SEQ), which shows that the
 * acceptance bar (within 1 BF16 step, at least 99.9% bit-exact) does not
 * depend on the tree.  Tests set it between calls, never during one. */
static int ss_order = ORACLE_SS_W64;

void oracle_set_ss_order(int order) {
    ss_order = order == ORACLE_SS_SEQ ? ORACLE_SS_SEQ : ORACLE_SS_W64;
}

/* The sum-of-squares tree.  [tail] _TpTailKernel.warp_sum_of_squares: each
 * thread owns 8 consecutive columns and adds their squares one by one from
 * 0.0; an xor butterfly over the warp's lanes makes the warp total; warps
 * then fold in column order.  Reading for a 64-lane wavefront: the row is
 * cut into blocks of 512 columns (64 lanes x 8 columns); lane l of block j
 * adds the squares of columns 512 j + 8 l .. + 7 in order from 0.0;
 * butterfly partners l ^ 1, l ^ 2, ..., l ^ 32 are added (s + s') so every
 * lane holds the block total; the block totals are added in ascending
 * block order from 0.0 (one band: the band split of the pages is a
 * property of an NVIDIA SM count).  Columns at or past P add nothing. */
static float sum_of_squares_w64(const float* v, int P) {
    float total = 0.0f;
    for (int block = 0; block * 512 < P; ++block) {
        float lane[64], next[64];
        for (int l = 0; l < 64; ++l) {
            float s = 0.0f;
            for (int c = 0; c < 8; ++c) {
                int col = block * 512 + 8 * l + c;
                if (col < P) {
                    float sq = v[col] * v[col];
                    s = s + sq;
                }
            }
            lane[l] = s;
        }
        for (int offset = 1; offset < 64; offset <<= 1) {
            for (int l = 0; l < 64; ++l) next[l] = lane[l] + lane[l ^ offset];
            memcpy(lane, next, sizeof lane);
        }
        total = total + lane[0];
    }
    return total;
}

/* The plain order: squares added one by one in column order from 0.0. */
static float sum_of_squares_seq(const float* v, int P) {
    float total = 0.0f;
    for (int c = 0; c < P; ++c) {
        float sq = v[c] * v[c];
        total = total + sq;
    }
    return total;
}

float oracle_sum_of_squares(const float* v, int P) {
    return ss_order == ORACLE_SS_SEQ ? sum_of_squares_seq(v, P) : sum_of_squares_w64(v, P);
}

/* 1 / sqrt(mean + eps).  [tail] _TpTailKernel: total * (1.0 / POOLED) + eps
 * then rsqrt.  Readings: 1/P is the FP32 nearest to the double 1.0/P; the
 * multiply and the add are two FP32 roundings; rsqrt is taken correctly
 * rounded through double: (float)(1.0 / sqrt((double)m)). */
static float inv_rms(float ss, int P, float eps) {
    float scale = (float)(1.0 / (double)P);
    float m = ss * scale;
    m = m + eps;
    return (float)(1.0 / sqrt((double)m));
}

float oracle_inv_rms(float ss, int P, float eps) { return inv_rms(ss, P, eps); }

/* One route row x[P] (BF16) -> its weighted, normalized FP32 products p[P].
 * [tail] module docstring: s_r = x_r * (gamma + gain_center) with
 * weight_before_norm, then s_r * rsqrt(mean(s_r^2) + eps) times w_r;
 * without it the gain multiplies after the norm.  Order per element from
 * the helpers gains / normalized and the route weight multiplied last on
 * its own (every product rounds separately):
 *   wbn:  v = x * g,  n = v * inv,           p = n * w
 *   else: v = x,      n = (x * inv) * g,     p = n * w
 * with g = fp32(gamma) + gain_center in FP32. */
static void route_products(const uint16_t* x, const float* gain, float w,
                           float eps, int wbn, int P, float* v, float* p) {
    for (int c = 0; c < P; ++c) {
        float xc = f32_of(x[c]);
        v[c] = wbn ? xc * gain[c] : xc;
    }
    float inv = inv_rms(oracle_sum_of_squares(v, P), P, eps);
    for (int c = 0; c < P; ++c) {
        float n;
        if (wbn) {
            n = v[c] * inv;
        } else {
            float xc = f32_of(x[c]);
            float t = xc * inv;
            n = t * gain[c];
        }
        p[c] = n * w;
    }
}

/* [tail] gains: the norm weight's columns plus the gain center, FP32 add. */
static void make_gains(const uint16_t* gamma, float gain_center, int P,
                       float* gain) {
    for (int c = 0; c < P; ++c) gain[c] = f32_of(gamma[c]) + gain_center;
}

void oracle_route_products(const uint16_t* x, const uint16_t* gamma, float gain_center,
                           float w, float eps, int weight_before_norm, int P, float* p) {
    float* gain = (float*)malloc(sizeof(float) * (size_t)P);
    float* v = (float*)malloc(sizeof(float) * (size_t)P);
    make_gains(gamma, gain_center, P, gain);
    route_products(x, gain, w, eps, weight_before_norm, P, v, p);
    free(gain);
    free(v);
}

/* ------------------------------------------------------- EP finalize ---- */

void oracle_rank_combine(const uint16_t* partials, int tp, int b, int P,
                         uint16_t* out) {
    /* [tail] module docstring: out = bf16(sum over ranks, in rank order, of
     * partial), FP32 sum; _TailReduceKernel: from 0.0 in rank order. */
    for (int t = 0; t < b; ++t)
        for (int c = 0; c < P; ++c) {
            float acc = 0.0f;
            for (int d = 0; d < tp; ++d)
                acc = acc + f32_of(partials[((int64_t)d * b + t) * P + c]);
            out[(int64_t)t * P + c] = plus_zero(bf16_of(acc));
        }
}

void oracle_finalize(const uint16_t* rows, int64_t R, const int32_t* idx,
                     const void* w, int w_dtype, const uint16_t* gamma,
                     float gain_center, float eps, int weight_before_norm,
                     int b, int K, int P, int tp,
                     uint16_t* partials, uint16_t* out, int nthreads) {
    float* gain = (float*)malloc(sizeof(float) * (size_t)P);
    make_gains(gamma, gain_center, P, gain);
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
    for (int dt = 0; dt < tp * b; ++dt) {
        int d = dt / b, t = dt % b;
        float* v = (float*)malloc(sizeof(float) * (size_t)P);
        float* p = (float*)malloc(sizeof(float) * (size_t)P);
        float* acc = (float*)malloc(sizeof(float) * (size_t)P);
        for (int c = 0; c < P; ++c) acc[c] = 0.0f;
        /* [tail] module docstring: per token, over the routes local to the
         * rank.  Reading: a route is local to rank d when its index into
         * rank d's rows lies in [0, R) (the kernels' predicated loads);
         * local routes are added in ascending route order from +0.0. */
        for (int k = 0; k < K; ++k) {
            int32_t r = idx[((int64_t)d * b + t) * K + k];
            if (r < 0 || (int64_t)r >= R) continue;
            const uint16_t* x = rows + ((int64_t)d * R + r) * P;
            route_products(x, gain, route_weight(w, w_dtype, (int64_t)t * K + k),
                           eps, weight_before_norm, P, v, p);
            for (int c = 0; c < P; ++c) acc[c] = acc[c] + p[c];
        }
        uint16_t* dst = partials + ((int64_t)d * b + t) * P;
        for (int c = 0; c < P; ++c) dst[c] = plus_zero(bf16_of(acc[c]));
        free(v);
        free(p);
        free(acc);
    }
    free(gain);
    if (out) oracle_rank_combine(partials, tp, b, P, out);
}

/* [tail_runtime] module docstring, the Kimi finalize: no per-route norm, the
 * partial is the route-weighted sum of the token's local rows,
 *   partial[d][t] = bf16(sum over local k, ascending, from +0.0, of
 *                        fp32(x_k) * w_k)      (-0 written as +0)
 * each product rounded on its own, then the same rank combine. */
void oracle_finalize_plain(const uint16_t* rows, int64_t R, const int32_t* idx,
                           const void* w, int w_dtype, int b, int K, int P, int tp,
                           uint16_t* partials, uint16_t* out, int nthreads) {
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
    for (int dt = 0; dt < tp * b; ++dt) {
        int d = dt / b, t = dt % b;
        float* acc = (float*)malloc(sizeof(float) * (size_t)P);
        for (int c = 0; c < P; ++c) acc[c] = 0.0f;
        for (int k = 0; k < K; ++k) {
            int32_t r = idx[((int64_t)d * b + t) * K + k];
            if (r < 0 || (int64_t)r >= R) continue;
            const uint16_t* x = rows + ((int64_t)d * R + r) * P;
            float wk = route_weight(w, w_dtype, (int64_t)t * K + k);
            for (int c = 0; c < P; ++c) {
                float prod = f32_of(x[c]) * wk;
                acc[c] = acc[c] + prod;
            }
        }
        uint16_t* dst = partials + ((int64_t)d * b + t) * P;
        for (int c = 0; c < P; ++c) dst[c] = plus_zero(bf16_of(acc[c]));
        free(acc);
    }
    if (out) oracle_rank_combine(partials, tp, b, P, out);
}

/* --------------------------------------------------- expert-TP finalize -- */

void oracle_tp_finalize(const uint16_t* kpart, int64_t num_rows,
                        const int32_t* idx, const void* w, int w_dtype,
                        const uint16_t* gamma, float gain_center, float eps,
                        int weight_before_norm, int b, int K, int P, int tp,
                        uint16_t* out, int nthreads) {
    float* gain = (float*)malloc(sizeof(float) * (size_t)P);
    make_gains(gamma, gain_center, P, gain);
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
    for (int t = 0; t < b; ++t) {
        uint16_t* xr = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)P);
        float* v = (float*)malloc(sizeof(float) * (size_t)P);
        float* p = (float*)malloc(sizeof(float) * (size_t)P);
        float* acc = (float*)malloc(sizeof(float) * (size_t)P);
        for (int c = 0; c < P; ++c) acc[c] = 0.0f;
        /* [tail] module docstring and _TpTailKernel: routes in order from
         * 0.0; a route whose row index is outside [0, num_rows) loads
         * nothing (predicated), which contributes nothing. */
        for (int k = 0; k < K; ++k) {
            int32_t r = idx[(int64_t)t * K + k];
            if (r < 0 || (int64_t)r >= num_rows) continue;
            /* x_r = bf16(sum over ranks, in rank order, of the K-partials),
             * FP32 from 0.0, rounded to BF16 before the norm. */
            for (int c = 0; c < P; ++c) {
                float s = 0.0f;
                for (int d = 0; d < tp; ++d)
                    s = s + f32_of(kpart[((int64_t)d * num_rows + r) * P + c]);
                xr[c] = bf16_of(s);
            }
            route_products(xr, gain, route_weight(w, w_dtype, (int64_t)t * K + k),
                           eps, weight_before_norm, P, v, p);
            for (int c = 0; c < P; ++c) acc[c] = acc[c] + p[c];
        }
        for (int c = 0; c < P; ++c)
            out[(int64_t)t * P + c] = plus_zero(bf16_of(acc[c]));
        free(xr);
        free(v);
        free(p);
        free(acc);
    }
    free(gain);
}

/* ------------------------------------- latent combine + norm + up proj -- */

void oracle_combine_norm_upproj(const uint16_t* lat, int tp,
                                const uint16_t* gamma, float eps,
                                const uint16_t* w_up, int N,
                                const uint16_t* rs, int b, int L,
                                uint16_t* normed, uint16_t* out, int nthreads) {
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
    for (int t = 0; t < b; ++t) {
        float* l = (float*)malloc(sizeof(float) * (size_t)L);
        float* y = (float*)malloc(sizeof(float) * (size_t)L);
        /* [tail_runtime] module docstring: the latent partials are
         * all-reduced, then RMS-normalized.  Reading: the sum is the rank
         * combine (FP32 in rank order from 0.0, rounded to BF16), the
         * statistic spans the whole latent row, and the normalized row is
         * rounded to BF16 as the projection's operand:
         *   y = bf16((l * inv) * fp32(gamma)). */
        for (int c = 0; c < L; ++c) {
            float s = 0.0f;
            for (int d = 0; d < tp; ++d)
                s = s + f32_of(lat[((int64_t)d * b + t) * L + c]);
            l[c] = f32_of(bf16_of(s));
        }
        float inv = inv_rms(oracle_sum_of_squares(l, L), L, eps);
        for (int c = 0; c < L; ++c) {
            float n = l[c] * inv;
            float g = n * f32_of(gamma[c]);
            uint16_t yb = plus_zero(bf16_of(g));
            y[c] = f32_of(yb);
            if (normed) normed[(int64_t)t * L + c] = yb;
        }
        /* Up projection: out[t][n] = bf16(sum_k W[n][k] * y[k] + rs[t][n]).
         * FP32 accumulation from 0.0 in ascending k; the shared expert's
         * reduce-scatter partial is added once after the full sum (reading). */
        for (int n = 0; n < N; ++n) {
            const uint16_t* wrow = w_up + (int64_t)n * L;
            float a = 0.0f;
            for (int k = 0; k < L; ++k) {
                float prod = f32_of(wrow[k]) * y[k];
                a = a + prod;
            }
            if (rs) a = a + f32_of(rs[(int64_t)t * N + n]);
            out[(int64_t)t * N + n] = plus_zero(bf16_of(a));
        }
        free(l);
        free(y);
    }
}

/* --------------------------------------------------------- shared expert -- */

/* SiLU in FP32: z / (1 + e^-z).  [shared] names its activation "SiTU" and
 * never defines it; the workload on these pages takes SiLU. */
static float silu(float z) {
    float e = expf(-z);
    float den = 1.0f + e;
    return z / den;
}

void oracle_shared_expert(const uint16_t* x, int b, int H,
                          const uint16_t* w_gate, const uint16_t* w_upw, int I,
                          const uint16_t* w_down, uint16_t* h, uint16_t* rs,
                          int nthreads) {
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
    for (int t = 0; t < b; ++t) {
        const uint16_t* xt = x + (int64_t)t * H;
        float* ht = (float*)malloc(sizeof(float) * (size_t)I);
        /* [shared] SharedUmma.owned_h: gate and up summed in FP32, each
         * rounded to BF16, then the activation, rounded to BF16 as h. */
        for (int i = 0; i < I; ++i) {
            const uint16_t* g_row = w_gate + (int64_t)i * H;
            const uint16_t* u_row = w_upw + (int64_t)i * H;
            float G = 0.0f, U = 0.0f;
            for (int j = 0; j < H; ++j) {
                float xj = f32_of(xt[j]);
                float pg = f32_of(g_row[j]) * xj;
                float pu = f32_of(u_row[j]) * xj;
                G = G + pg;
                U = U + pu;
            }
            float gs = f32_of(bf16_of(G));
            float us = f32_of(bf16_of(U));
            float a = silu(gs);
            float hv = a * us;
            uint16_t hb = plus_zero(bf16_of(hv));
            ht[i] = f32_of(hb);
            if (h) h[(int64_t)t * I + i] = hb;
        }
        /* [shared] module docstring / SharedBase.push: the down rows in FP32,
         * BF16 with -0 made +0, into the reduce-scatter partial. */
        for (int n = 0; n < H; ++n) {
            const uint16_t* d_row = w_down + (int64_t)n * I;
            float a = 0.0f;
            for (int i = 0; i < I; ++i) {
                float prod = f32_of(d_row[i]) * ht[i];
                a = a + prod;
            }
            rs[(int64_t)t * H + n] = plus_zero(bf16_of(a));
        }
        free(ht);
    }
}
