/*
 * Host-side driver that exercises every entry point of the CPU oracle
 * (oracle/lto.c) on small ragged shapes, for a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py builds and
 * runs it).  Every buffer is allocated at its exact size, so any read or
 * write outside a tensor is reported; the driver also checks that nothing
 * outside the column window (or outside the written AttnRes rows) changes,
 * that argument errors return -1 without touching memory, and that the
 * residual form works in place.  Exit status 0 means every check passed.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int lto_latent(const uint16_t *partials, int P, int64_t T, int64_t L,
               const uint16_t *norm_w, double eps, uint16_t *y);
int lto_latent_tail(const uint16_t *partials, int P, int64_t T, int64_t L,
                    const uint16_t *norm_w, double eps,
                    const uint16_t *W, int64_t H, int64_t c0, int64_t n,
                    uint16_t *out, int64_t ld_out, int nthreads);
int lto_latent_tail_residual(const uint16_t *partials, int P, int64_t T, int64_t L,
                             const uint16_t *norm_w, double eps,
                             const uint16_t *W, int64_t H, int64_t c0, int64_t n,
                             uint16_t *out, int64_t ld_out,
                             const uint16_t *prefix, int64_t ld_prefix,
                             uint16_t *resid, int64_t ld_resid, int nthreads);
int lto_attn_res_zero_block(uint16_t *prefix, const uint16_t *delta, int64_t T, int64_t H,
                            uint16_t *block, int64_t num_slots, int64_t block_idx,
                            const uint16_t *norm_w, double eps, uint16_t *out);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* splitmix64 */
static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* a finite bf16 pattern with a modest exponent (|x| in about [2^-8, 2^3)) */
static uint16_t rand_bf16(void)
{
    const uint64_t r = next_u64();
    const uint16_t sign = (uint16_t)((r & 1u) << 15);
    const uint16_t exp = (uint16_t)(119 + (r >> 1) % 11);
    const uint16_t man = (uint16_t)((r >> 8) & 0x7F);
    return (uint16_t)(sign | (exp << 7) | man);
}

static uint16_t *alloc_fill(size_t count)
{
    uint16_t *p = (uint16_t *)malloc((count ? count : 1) * sizeof(uint16_t));
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    for (size_t i = 0; i < count; ++i) p[i] = rand_bf16();
    return p;
}

static uint16_t *dup(const uint16_t *p, size_t count)
{
    uint16_t *q = (uint16_t *)malloc((count ? count : 1) * sizeof(uint16_t));
    if (!q) exit(2);
    memcpy(q, p, count * sizeof(uint16_t));
    return q;
}

static int failures = 0;

static void check(int cond, const char *what)
{
    if (!cond) {
        fprintf(stderr, "FAIL: %s\n", what);
        ++failures;
    }
}

/* every element of out outside columns [c0, c0+n) equals before */
static int outside_unchanged(const uint16_t *out, const uint16_t *before, int64_t T,
                             int64_t ld, int64_t c0, int64_t n)
{
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < ld; ++j)
            if ((j < c0 || j >= c0 + n) && out[t * ld + j] != before[t * ld + j]) return 0;
    return 1;
}

static void tail_case(int P, int64_t T, int64_t L, int64_t H, int64_t c0, int64_t n,
                      int64_t ld, int with_norm)
{
    uint16_t *partials = alloc_fill((size_t)(P * T * L));
    uint16_t *norm_w = with_norm ? alloc_fill((size_t)L) : NULL;
    uint16_t *W = alloc_fill((size_t)(H * L));
    uint16_t *out = alloc_fill((size_t)(T * ld));
    uint16_t *before = dup(out, (size_t)(T * ld));
    check(lto_latent_tail(partials, P, T, L, norm_w, 1e-6, W, H, c0, n, out, ld, 2) == 0,
          "lto_latent_tail returns 0");
    check(outside_unchanged(out, before, T, ld, c0, n), "lto_latent_tail leaves the rest of out");

    /* the same call through the residual form, resid in place on prefix */
    uint16_t *out2 = dup(before, (size_t)(T * ld));
    uint16_t *prefix = alloc_fill((size_t)(T * ld));
    uint16_t *pbefore = dup(prefix, (size_t)(T * ld));
    check(lto_latent_tail_residual(partials, P, T, L, norm_w, 1e-6, W, H, c0, n, out2, ld,
                                   prefix, ld, prefix, ld, 1) == 0,
          "lto_latent_tail_residual returns 0");
    check(memcmp(out, out2, (size_t)(T * ld) * sizeof(uint16_t)) == 0,
          "residual form gives the same out");
    check(outside_unchanged(prefix, pbefore, T, ld, c0, n),
          "residual form leaves the rest of resid");

    /* the latent alone, and argument errors that must not touch memory */
    uint16_t *y = alloc_fill((size_t)(T * L));
    check(lto_latent(partials, P, T, L, norm_w, 1e-6, y) == 0, "lto_latent returns 0");
    uint16_t *after = dup(out, (size_t)(T * ld));
    check(lto_latent_tail(partials, 0, T, L, norm_w, 1e-6, W, H, c0, n, out, ld, 1) == -1,
          "P = 0 refused");
    check(lto_latent_tail(partials, P, T, L, norm_w, 1e-6, W, H, c0, n + 1 + H, out, ld, 1) == -1,
          "window past H refused");
    check(lto_latent_tail(partials, P, T, L, norm_w, 1e-6, W, H, c0, n, out, H - 1, 1) == -1,
          "ld_out below H refused");
    check(lto_latent_tail(partials, P, 0, L, norm_w, 1e-6, W, H, c0, n, out, ld, 1) == 0,
          "T = 0 is a no-op");
    check(lto_latent_tail(partials, P, T, L, norm_w, 1e-6, W, H, c0, 0, out, ld, 1) == 0,
          "n = 0 is a no-op");
    check(memcmp(out, after, (size_t)(T * ld) * sizeof(uint16_t)) == 0,
          "refused and empty calls leave out unchanged");

    free(partials);
    free(norm_w);
    free(W);
    free(out);
    free(before);
    free(out2);
    free(prefix);
    free(pbefore);
    free(y);
    free(after);
}

static void attn_res_case(int64_t T, int64_t H, int64_t slots, int64_t idx, int with_delta,
                          int with_norm)
{
    uint16_t *prefix = alloc_fill((size_t)(T * H));
    uint16_t *delta = with_delta ? alloc_fill((size_t)(T * H)) : NULL;
    uint16_t *block = slots > 0 ? alloc_fill((size_t)(T * slots * H)) : NULL;
    uint16_t *bbefore = slots > 0 ? dup(block, (size_t)(T * slots * H)) : NULL;
    uint16_t *norm_w = with_norm ? alloc_fill((size_t)H) : NULL;
    uint16_t *out = alloc_fill((size_t)(T * H));
    uint16_t *pbefore = dup(prefix, (size_t)(T * H));
    check(lto_attn_res_zero_block(prefix, delta, T, H, block, slots, idx, norm_w, 1e-6, out) == 0,
          "lto_attn_res_zero_block returns 0");
    if (!with_delta)
        check(memcmp(prefix, pbefore, (size_t)(T * H) * sizeof(uint16_t)) == 0,
              "no delta: prefix unchanged");
    if (slots > 0) {
        int ok = 1;
        for (int64_t t = 0; t < T; ++t)
            for (int64_t s = 0; s < slots; ++s)
                for (int64_t h = 0; h < H; ++h) {
                    const int64_t i = (t * slots + s) * H + h;
                    if (s == idx) {
                        if (block[i] != prefix[t * H + h]) ok = 0;
                    } else if (block[i] != bbefore[i]) {
                        ok = 0;
                    }
                }
        check(ok, "block write lands in its slot only");
    }
    check(lto_attn_res_zero_block(prefix, delta, T, H, block, slots, slots, norm_w, 1e-6, out) == -1,
          "block index past the slots refused");
    free(prefix);
    free(delta);
    free(block);
    free(bbefore);
    free(norm_w);
    free(out);
    free(pbefore);
}

int main(void)
{
    tail_case(1, 5, 24, 40, 3, 30, 45, 1);
    tail_case(3, 7, 64, 33, 0, 33, 33, 1);
    tail_case(2, 1, 8, 9, 8, 1, 12, 0);
    tail_case(4, 17, 40, 70, 11, 50, 77, 0);
    attn_res_case(3, 128, 4, 2, 1, 1);
    attn_res_case(7, 72, 0, -1, 0, 1);
    attn_res_case(1, 16, 2, 0, 1, 0);
    attn_res_case(5, 40, 3, -1, 1, 0);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
