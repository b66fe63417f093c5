/*
 * Runs the CPU oracle's functions on small seeded cases under
 * AddressSanitizer and UndefinedBehaviorSanitizer (built by
 * tests/test_sanitizers.py).  It checks no values (the oracle's pins do that);
 * every array is allocated at exactly the size the oracle's contract states,
 * so an access past it is reported.  Prints "ok" on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_start_loc(const int32_t *counts, int n_active, int max_loras, int32_t *start_loc);
int oracle_prepare(const int32_t *mapping, int num_tokens, int max_loras, int32_t *mapping_copy, int32_t *sorted,
                   int32_t *active_ids, int32_t *counts, int32_t *start_loc, int32_t *no_lora_flag);
int oracle_shrink(const uint16_t *x, int64_t ldx, int num_tokens, int hidden, const uint16_t *const *lora_a,
                  int num_slices, int rank, int max_loras, float *buf, const int32_t *mapping, double scale,
                  const int32_t *tokens, int ntok, double *bound, int nthreads);
int oracle_expand(const float *buf, int num_tokens, int rank, const uint16_t *const *lora_b,
                  const uint16_t *const *bias, const int32_t *widths, int num_slices, uint16_t *y, int64_t ldy,
                  int offset_start, int add_inputs, const int32_t *mapping, int max_loras, const int32_t *tokens,
                  int ntok, double *mag, int nthreads);
uint16_t oracle_double_to_bf16(double v);
double oracle_bf16_to_double(uint16_t h);

static uint32_t rng_state = 12345u;
static uint32_t rnd(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return rng_state >> 8;
}

static uint16_t rnd_bf16(void) { return oracle_double_to_bf16(((double)(rnd() % 2001) - 1000.0) / 700.0); }

static void *xmalloc(size_t n) { return malloc(n ? n : 1); }

static void one_case(int n, int hidden, int rank, int max_loras, int num_slices, const int *widths_in,
                     int with_bias, int add_inputs, int nthreads, int neg_every, int bad_every)
{
    int32_t *mapping = xmalloc(sizeof(int32_t) * n);
    for (int t = 0; t < n; ++t) {
        mapping[t] = (int32_t)(rnd() % (uint32_t)max_loras);
        if (neg_every && t % neg_every == 0) mapping[t] = -1;
        if (bad_every && t % bad_every == 1) mapping[t] = (t & 2) ? max_loras + 3 : -7;
    }
    int32_t *copy = xmalloc(sizeof(int32_t) * n), *sorted = xmalloc(sizeof(int32_t) * n);
    int32_t *ids = xmalloc(sizeof(int32_t) * (max_loras + 1)), *counts = xmalloc(sizeof(int32_t) * (max_loras + 1));
    int32_t *start = xmalloc(sizeof(int32_t) * (max_loras + 2)), flag = 0;
    oracle_prepare(mapping, n, max_loras, copy, sorted, ids, counts, start, &flag);

    int64_t ldx = hidden + 8;
    uint16_t *x = xmalloc(sizeof(uint16_t) * (size_t)(n * ldx));
    for (int64_t k = 0; k < n * ldx; ++k) x[k] = rnd_bf16();
    const uint16_t *a[8], *b[8], *bias[8];
    int32_t widths[8];
    int total = 0;
    for (int i = 0; i < num_slices; ++i) {
        widths[i] = widths_in[i];
        total += widths[i];
        uint16_t *ai = xmalloc(sizeof(uint16_t) * (size_t)max_loras * rank * hidden);
        for (int64_t k = 0; k < (int64_t)max_loras * rank * hidden; ++k) ai[k] = rnd_bf16();
        uint16_t *bi = xmalloc(sizeof(uint16_t) * (size_t)max_loras * widths[i] * rank);
        for (int64_t k = 0; k < (int64_t)max_loras * widths[i] * rank; ++k) bi[k] = rnd_bf16();
        uint16_t *ci = xmalloc(sizeof(uint16_t) * (size_t)max_loras * widths[i]);
        for (int64_t k = 0; k < (int64_t)max_loras * widths[i]; ++k) ci[k] = rnd_bf16();
        a[i] = ai;
        b[i] = bi;
        bias[i] = (with_bias && i % 2 == 0) ? ci : NULL;
        if (!bias[i]) free(ci);
    }
    float *buf = xmalloc(sizeof(float) * (size_t)num_slices * n * rank);
    for (int64_t k = 0; k < (int64_t)num_slices * n * rank; ++k) buf[k] = 0.f;
    /* every token, then a token subset with bounds */
    oracle_shrink(x, ldx, n, hidden, a, num_slices, rank, max_loras, buf, mapping, 0.5, NULL, 0, NULL, nthreads);
    int ntok = n / 3 + 1;
    int32_t *tokens = xmalloc(sizeof(int32_t) * ntok);
    for (int p = 0; p < ntok; ++p) tokens[p] = (int32_t)((p * 3) % n);
    double *bound = xmalloc(sizeof(double) * (size_t)num_slices * ntok * rank);
    oracle_shrink(x, ldx, n, hidden, a, num_slices, rank, max_loras, buf, mapping, -0.25, tokens, ntok, bound,
                  nthreads);

    int offset = 8;
    int64_t ldy = offset + total + 8;
    uint16_t *y = xmalloc(sizeof(uint16_t) * (size_t)(n * ldy));
    for (int64_t k = 0; k < n * ldy; ++k) y[k] = rnd_bf16();
    double *mag = xmalloc(sizeof(double) * (size_t)ntok * total);
    oracle_expand(buf, n, rank, b, with_bias ? bias : NULL, widths, num_slices, y, ldy, offset, add_inputs,
                  mapping, max_loras, NULL, 0, NULL, nthreads);
    oracle_expand(buf, n, rank, b, with_bias ? bias : NULL, widths, num_slices, y, ldy, offset, !add_inputs,
                  mapping, max_loras, tokens, ntok, mag, nthreads);

    for (int i = 0; i < num_slices; ++i) {
        free((void *)a[i]);
        free((void *)b[i]);
        if (bias[i]) free((void *)bias[i]);
    }
    free(mapping); free(copy); free(sorted); free(ids); free(counts); free(start);
    free(x); free(buf); free(tokens); free(bound); free(y); free(mag);
}

int main(void)
{
    /* the scan alone, with the printed worked-example counts */
    int32_t counts[4] = {3, 10, 5, 2}, start[5];
    oracle_start_loc(counts, 4, 3, start);

    /* prepare: empty, all -1, single token */
    int32_t one = -1, c1, s1, ids[2], cn[2], st[3], flag;
    oracle_prepare(&one, 0, 1, &c1, &s1, ids, cn, st, &flag);
    oracle_prepare(&one, 1, 1, &c1, &s1, ids, cn, st, &flag);

    /* rounding edge cases */
    volatile double sink = 0.0;
    const double vals[] = {0.0, -0.0, 1.0, 3.0e38, 3.4e38, 1e-40, -1e-45, 1.0 / 3.0};
    for (unsigned k = 0; k < sizeof vals / sizeof vals[0]; ++k)
        sink += oracle_bf16_to_double(oracle_double_to_bf16(vals[k]));

    const int w1[] = {16}, w3[] = {24, 8, 40}, w8[] = {8, 8, 8, 8, 8, 8, 8, 8};
    one_case(64, 32, 8, 3, 1, w1, 0, 1, 1, 4, 0);
    one_case(37, 72, 16, 5, 3, w3, 1, 0, 2, 3, 7);
    one_case(20, 16, 8, 1, 8, w8, 1, 1, 4, 0, 0);
    one_case(5, 8, 128, 2, 1, w1, 0, 1, 3, 2, 0);
    printf("ok\n");
    return sink == 12345.0;
}
