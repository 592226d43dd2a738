/*
 * lto.c -- CPU fp64 oracle for the latent-MoE output tail.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * HIP library is checked against.  Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the library itself never
 * links, calls or includes anything from this directory, and this file
 * includes nothing from the library.
 *
 * Sources (the three web pages this project follows):
 *   [PR51253]  prhub report of vLLM PR #51253, "[ROCm][Perf] Kimi-K3 Shard
 *              Latent MoE up-projection for ROCm path".
 *   [PR50383]  prhub report of vLLM PR #50383 (column-parallel up-projection
 *              tier of the K3 latent-MoE runner, `_shard_up_proj_tail`).
 *   [PR50593]  prhub report of vLLM PR #50593, "[Kimi-K3][AMD] Fuse AttnRes
 *              state updates and norms".
 *
 * What is computed (one GPU's share of the tail, TP all-reduce replaced by a
 * local sum over n_partials, final all-reduce left to the caller):
 *
 *   s[t,k]   = sum_p partials[p,t,k]                      (fp64, p ascending)
 *   s'[t,k]  = bf16(s[t,k])                               (R1: the reduced
 *              latent is a bf16 tensor on the pages' path)
 *   if norm_w:  r_t = 1 / sqrt( (1/L) sum_k s'[t,k]^2 + eps )
 *               y[t,k] = bf16( s'[t,k] * r_t * w[k] )     (R2: one rounding)
 *   else        y[t,k] = s'[t,k]
 *   out[t, c0+j] = bf16( out[t, c0+j] + sum_k y[t,k] * W[c0+j, k] )  (R3)
 *
 * for t < T, 0 <= j < n; every other element of out is left untouched.
 *
 * Everything between the three bf16 rounding points is fp64.  bf16 rounding
 * is round-to-nearest, ties-to-even, written here from its definition (the
 * nearest multiple of the bf16 spacing at the value's binade).
 *
 * Pins: every function here is checked in tests/test_oracle_pins.py against
 * closed forms, invariants, library routines and exact-arithmetic brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 bit pattern -> double (exact: bf16 is the top half of an IEEE float). */
double lto_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * double -> bf16, round to nearest, ties to even, straight from the
 * definition: bf16 keeps 8 significant bits, so in the binade [2^e, 2^(e+1))
 * the representable values are the multiples of 2^(e-7); below the smallest
 * normal (2^-126) they are the multiples of 2^-133.  nearbyint() in the
 * default rounding mode picks the nearest integer with ties to even.
 * Values that round to 2^128 or beyond become infinity.  NaN stays NaN
 * (quiet, sign kept).  The pages use PyTorch's bf16 casts, which round this way.
 */
uint16_t lto_f64_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
    double ax = fabs(x);
    if (ax == 0.0) return sign;

    int e2;
    frexp(ax, &e2);             /* ax in [2^(e2-1), 2^e2) */
    int quantum_exp = (e2 - 1) - 7;
    if (quantum_exp < -133) quantum_exp = -133;
    double q = ldexp(nearbyint(ldexp(ax, -quantum_exp)), quantum_exp);
    if (q >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    if (q == 0.0) return sign;

    float f = (float)q;         /* exact: q has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* Round-trip helper: the double value of bf16(x). */
static double rne(double x) { return lto_bf16_to_f64(lto_f64_to_bf16(x)); }

int lto_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Latent of the tail: partial sum, storage round trip, RMSNorm.
 *
 * [PR51253 Key source snippets, `_check_matches_replicated`]: the expected
 * value applies `F.rms_norm` over the latent width, with the norm weight and
 * eps, to the all-reduced routed output -- the reduction comes first and the
 * norm second.  [PR50383 Key source snippets, `_shard_up_proj_tail`]: the
 * norm is optional; without it the all-reduced latent goes straight to the
 * projection.  [PR50593 Implementation, item 1]: accumulate in high
 * precision, round to bf16 storage precision, then use that value as the
 * source; the norm's variance is not computed in bf16.
 *
 * partials: [P][T][L] bf16 bits, packed.  norm_w: [L] bf16 bits or NULL.
 * y: [T][L] bf16 bits, written.  Returns 0, or -1 on bad arguments or when
 * a row's scratch cannot be allocated.
 */
int lto_latent(const uint16_t *partials, int P, int64_t T, int64_t L,
               const uint16_t *norm_w, double eps, uint16_t *y)
{
    if (P < 1 || T < 0 || L < 1 || (T > 0 && (!partials || !y))) return -1;

    int nomem = 0;
#pragma omp parallel for schedule(static) reduction(| : nomem)
    for (int64_t t = 0; t < T; ++t) {
        double *sr = (double *)malloc((size_t)L * sizeof(double));
        if (!sr) {
            nomem = 1;
            continue;
        }
        /* step 1 + R1: sum of the partials in fp64, then bf16 storage */
        for (int64_t k = 0; k < L; ++k) {
            double s = 0.0;
            for (int p = 0; p < P; ++p)
                s += lto_bf16_to_f64(partials[((int64_t)p * T + t) * L + k]);
            sr[k] = rne(s);
        }
        if (norm_w) {
            /* step 2 + R2: RMSNorm, eps inside the square root */
            double ss = 0.0;
            for (int64_t k = 0; k < L; ++k) ss += sr[k] * sr[k];
            double ms = ss / (double)L;
            double r = 1.0 / sqrt(ms + eps);
            for (int64_t k = 0; k < L; ++k)
                y[t * L + k] = lto_f64_to_bf16(sr[k] * r * lto_bf16_to_f64(norm_w[k]));
        } else {
            for (int64_t k = 0; k < L; ++k) y[t * L + k] = lto_f64_to_bf16(sr[k]);
        }
        free(sr);
    }
    return nomem ? -1 : 0;
}

/*
 * The whole tail for one GPU's column window.
 *
 * [PR50383 Key source snippets, `_shard_up_proj_tail`]: rows
 * [c0, c0+n) of the replicated up-projection weight W[H][L] are narrowed out,
 * the same columns of the shared-expert output are narrowed out, and the
 * projection is added in place (`addmm_`, beta = alpha = 1: one rounding of
 * C + A*B^T).  [PR51253 Key source snippets, `_check_writes_only_its_own_shard`]:
 * before the final collective only the window has changed; columns outside
 * it are bit-identical.  [PR51253 Implementation, item 2]: the routed scaling
 * factor is 1, so there is no alpha.
 *
 * out: [T][ld_out] bf16 bits, updated in place on columns [c0, c0+n) only.
 * nthreads <= 0 keeps the OpenMP default.  Returns 0, or -1 on bad arguments.
 */
int lto_latent_tail(const uint16_t *partials, int P, int64_t T, int64_t L,
                    const uint16_t *norm_w, double eps,
                    const uint16_t *W, int64_t H, int64_t c0, int64_t n,
                    uint16_t *out, int64_t ld_out, int nthreads)
{
    if (P < 1 || T < 0 || L < 1 || H < 0 || c0 < 0 || n < 0 || c0 + n > H ||
        ld_out < H)
        return -1;
    if (T == 0 || n == 0) return 0;
    if (!partials || !W || !out) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

    uint16_t *y = (uint16_t *)malloc((size_t)T * (size_t)L * sizeof(uint16_t));
    if (!y) return -1;
    if (lto_latent(partials, P, T, L, norm_w, eps, y) != 0) {
        free(y);
        return -1;
    }

    /* step 3 + R3: projection onto the window, beta-add of the shared output */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < n; ++j) {
            const uint16_t *wrow = W + (c0 + j) * L;
            const uint16_t *yrow = y + t * L;
            double acc = 0.0;
            for (int64_t k = 0; k < L; ++k)
                acc += lto_bf16_to_f64(yrow[k]) * lto_bf16_to_f64(wrow[k]);
            uint16_t *o = out + t * ld_out + c0 + j;
            *o = lto_f64_to_bf16(lto_bf16_to_f64(*o) + acc);
        }
    }
    free(y);
    return 0;
}

/*
 * The tail followed by the decoder layer's residual update, on the window.
 *
 * [PR50593 Key source snippets, `forward_attn_residual`]: after the MLP the
 * layer adds the MLP output to the running prefix sum, `prefix_sum +
 * hidden_states`, as a bf16 add (one rounding of the exact sum).  Here the
 * MLP output is the tail's result, so after lto_latent_tail
 *
 *   resid[t, c0+j] = bf16( prefix[t, c0+j] + out[t, c0+j] )       (R4)
 *
 * for t < T, 0 <= j < n, with out already updated by R3.  Columns outside the
 * window of resid are left untouched.  resid may be the prefix buffer itself
 * (same pointer and row stride): every element is read before it is written.
 *
 * prefix: [T][ld_prefix], resid: [T][ld_resid] bf16 bits, ld >= c0 + n.
 * Returns 0, or -1 on bad arguments.
 */
int lto_latent_tail_residual(const uint16_t *partials, int P, int64_t T, int64_t L,
                             const uint16_t *norm_w, double eps,
                             const uint16_t *W, int64_t H, int64_t c0, int64_t n,
                             uint16_t *out, int64_t ld_out,
                             const uint16_t *prefix, int64_t ld_prefix,
                             uint16_t *resid, int64_t ld_resid, int nthreads)
{
    if (ld_prefix < c0 + n || ld_resid < c0 + n) return -1;
    if (T > 0 && n > 0 && (!prefix || !resid)) return -1;
    int rc = lto_latent_tail(partials, P, T, L, norm_w, eps, W, H, c0, n, out, ld_out, nthreads);
    if (rc != 0) return rc;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = c0; j < c0 + n; ++j) {
            const double a = lto_bf16_to_f64(prefix[t * ld_prefix + j]);
            const double b = lto_bf16_to_f64(out[t * ld_out + j]);
            resid[t * ld_resid + j] = lto_f64_to_bf16(a + b);
        }
    }
    return 0;
}

/*
 * AttnRes state update and output norm, zero-block path.
 *
 * [PR50593 Implementation, item 1]: the fused AttnRes kernel loads the prefix
 * sum and the delta, adds them in high precision, rounds the sum to bf16
 * storage precision and uses that value from then on as the residual source
 * (the prefix is updated in place); with a block-write index the same value
 * lands in that slot of the block residual; the output RMSNorm keeps its
 * variance out of bf16.  With no valid blocks the softmax over sources has
 * the prefix as its only source, so the aggregated value is the prefix
 * itself.  [PR50593 Key source snippets, `forward_attn_residual`]: the delta
 * stands for the unfused `prefix_sum + hidden_states` (a bf16 add).
 *
 *   p'[t,h] = bf16(prefix[t,h] + delta[t,h])       (delta != NULL; else prefix)
 *   prefix[t,h] <- p'[t,h]                          (delta != NULL)
 *   block[t, idx, h] <- p'[t,h]                     (idx >= 0)
 *   out[t,h] = bf16(p'[t,h] * r_t * w[h]),  r_t = 1/sqrt((1/H) sum_h p'^2 + eps)
 *                                                   (norm_w != NULL; else p')
 *
 * prefix, delta, out: [T][H]; block: [T][num_slots][H]; norm_w: [H]; all
 * bf16 bits, packed.  Every other element is left untouched.
 * Returns 0, or -1 on bad arguments or when a row's scratch cannot be
 * allocated.
 */
int lto_attn_res_zero_block(uint16_t *prefix, const uint16_t *delta, int64_t T, int64_t H,
                            uint16_t *block, int64_t num_slots, int64_t block_idx,
                            const uint16_t *norm_w, double eps, uint16_t *out)
{
    if (T < 0 || H < 1 || num_slots < 0 || block_idx >= num_slots) return -1;
    if (T == 0) return 0;
    if (!prefix || !out || (block_idx >= 0 && !block)) return -1;

    int nomem = 0;
#pragma omp parallel for schedule(static) reduction(| : nomem)
    for (int64_t t = 0; t < T; ++t) {
        double *p = (double *)malloc((size_t)H * sizeof(double));
        if (!p) {
            nomem = 1;
            continue;
        }
        /* the updated prefix: one rounding of the exact sum */
        for (int64_t h = 0; h < H; ++h) {
            double v = lto_bf16_to_f64(prefix[t * H + h]);
            if (delta) v += lto_bf16_to_f64(delta[t * H + h]);
            p[h] = rne(v);
        }
        if (delta)
            for (int64_t h = 0; h < H; ++h) prefix[t * H + h] = lto_f64_to_bf16(p[h]);
        if (block_idx >= 0)
            for (int64_t h = 0; h < H; ++h)
                block[(t * num_slots + block_idx) * H + h] = lto_f64_to_bf16(p[h]);
        if (norm_w) {
            double ss = 0.0;
            for (int64_t h = 0; h < H; ++h) ss += p[h] * p[h];
            double r = 1.0 / sqrt(ss / (double)H + eps);
            for (int64_t h = 0; h < H; ++h)
                out[t * H + h] = lto_f64_to_bf16(p[h] * r * lto_bf16_to_f64(norm_w[h]));
        } else {
            for (int64_t h = 0; h < H; ++h) out[t * H + h] = lto_f64_to_bf16(p[h]);
        }
        free(p);
    }
    return nomem ? -1 : 0;
}
