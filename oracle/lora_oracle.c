/*
 * lora_oracle.c -- plain CPU oracle for the segmented-gather multi-LoRA path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library calls, links or includes
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load it.  It shares no code, header or table with the HIP path.
 *
 * Every function is the plain definition of what the pages compute, written
 * as per-token loops with double accumulation; no blocking, fusion or
 * reordering.  Sources (vLLM API documentation pages):
 *   - "lora_kernel_metadata" page, class LoRAKernelMeta: make (buffer sizes,
 *     padding and the worked example in its comments), _reset (padding values)
 *     and prepare_tensors (all(-1) check, mapping copy, stable sort,
 *     unique with counts, cumsum into lora_token_start_loc).
 *   - "punica_gpu" page, PunicaWrapperGPU: add_shrink docstring (per slice,
 *     y[i] += (x @ lora_a[i]) * scale), add_expand docstring (per slice,
 *     y[:, offset:offset+slice] += x[i] @ lora_b[i] + bias[i]),
 *     add_lora_linear (fp32 shrink buffer).
 *   - "punica_tpu" page, PunicaWrapperTPU: add_expand (running column offset
 *     per slice) and _apply_bias (bias gathered per token, zero for id -1).
 *
 * Readings where the pages are silent (listed with reasons in the design
 * notes): tokens with id -1 are left untouched by shrink and expand; an id
 * outside [-1, max_loras) is reported and treated as -1; add_inputs = 0 means
 * the slice columns of an active token are overwritten; bias is added inside
 * expand with a single rounding to bfloat16; the shrink update is "+=".
 *
 * Numerics: bfloat16 -> double is exact; every sum is a double sum in index
 * order; the shrink result is stored to float with C's round-to-nearest-even
 * conversion; y is rounded to bfloat16 with round-to-nearest-even written out
 * from the definition of the format (8 significant bits, exponent range of
 * float, subnormal quantum 2^-133).
 *
 * Parity pins for every function live in the CPU test-suite: printed values
 * from the pages' worked example, torch CPU sort/unique/cumsum on the same
 * mappings, a numpy dense masked brute force, closed forms and invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ID 1

static double bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 value, ties to even, straight from
 * the format's definition: 8 significant bits for normal numbers, the float
 * exponent range, a fixed quantum of 2^-133 below 2^-126, overflow to inf. */
uint16_t oracle_double_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    double r;
    if (a == 0.0) {
        r = 0.0;
    } else {
        int e;
        (void)frexp(a, &e);            /* a in [2^(e-1), 2^e) */
        int qexp = e - 8;              /* quantum for 8 significant bits */
        if (qexp < -133)
            qexp = -133;
        r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);   /* ties to even */
        if (r >= ldexp(1.0, 128))
            r = INFINITY;
    }
    float f = (float)(neg ? -r : r);   /* exact: r is a bfloat16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

double oracle_bf16_to_double(uint16_t h) { return bf16_to_double(h); }

static int clean_id(int32_t id, int max_loras, int *bad)
{
    if (id < -1 || id >= max_loras) {
        *bad = 1;
        return -1;
    }
    return id;
}

/* Segment starts: start_loc[0] = 0, start_loc[k+1] = counts[0] + ... +
 * counts[k] for k < n_active, every later entry 0 (the reset value).
 * (make's comment: the first index is always 0; prepare_tensors writes the
 * cumsum into positions 1 .. n.) */
void oracle_start_loc(const int32_t *counts, int n_active, int max_loras, int32_t *start_loc)
{
    for (int k = 0; k < max_loras + 2; ++k)
        start_loc[k] = 0;
    int64_t run = 0;
    for (int k = 0; k < n_active; ++k) {
        run += counts[k];
        start_loc[k + 1] = (int32_t)run;
    }
}

/* LoRAKernelMeta.prepare_tensors.  Output arrays have the sizes make()
 * gives them: mapping_copy and sorted [max_num_tokens >= num_tokens],
 * active_ids and counts [max_loras+1], start_loc [max_loras+2].
 * Returns ORACLE_BAD_ID if some id was outside [-1, max_loras). */
int oracle_prepare(const int32_t *mapping, int num_tokens, int max_loras,
                   int32_t *mapping_copy, int32_t *sorted, int32_t *active_ids,
                   int32_t *counts, int32_t *start_loc, int32_t *no_lora_flag)
{
    int bad = 0;
    /* _reset */
    for (int k = 0; k < max_loras + 1; ++k) {
        active_ids[k] = -1;
        counts[k] = 0;
    }
    for (int k = 0; k < max_loras + 2; ++k)
        start_loc[k] = 0;

    /* all(mapping == -1); true for an empty mapping */
    int all_neg = 1;
    for (int t = 0; t < num_tokens; ++t)
        if (clean_id(mapping[t], max_loras, &bad) != -1)
            all_neg = 0;
    *no_lora_flag = all_neg;
    if (all_neg)
        return bad ? ORACLE_BAD_ID : ORACLE_OK;   /* early exit */

    /* mapping copy */
    for (int t = 0; t < num_tokens; ++t)
        mapping_copy[t] = clean_id(mapping[t], max_loras, &bad);

    /* unique ids in ascending order, with counts; -1 included when present */
    int n_active = 0;
    for (int id = -1; id < max_loras; ++id) {
        int c = 0;
        for (int t = 0; t < num_tokens; ++t)
            if (mapping_copy[t] == id)
                ++c;
        if (c > 0) {
            active_ids[n_active] = id;
            counts[n_active] = c;
            ++n_active;
        }
    }

    /* stable sort of token indices by id: ids ascending, ties in token order */
    int pos = 0;
    for (int k = 0; k < n_active; ++k)
        for (int t = 0; t < num_tokens; ++t)
            if (mapping_copy[t] == active_ids[k])
                sorted[pos++] = t;

    oracle_start_loc(counts, n_active, max_loras, start_loc);
    return bad ? ORACLE_BAD_ID : ORACLE_OK;
}

/* lora_shrink: for every listed token t whose id m is not -1, every slice i
 * and every j < rank,
 *     buf[i][t][j] += scale * sum_k x[t][k] * A_i[m][j][k]
 * in double, stored to float.  `tokens` (ntok entries) lists the tokens to
 * compute (NULL = all num_tokens tokens).  If `bound` is not NULL it receives
 * |scale| * sum_k |x[t][k] * A_i[m][j][k]| at [i][p][j], p being the token's
 * position in the list.  `buf` is [num_slices][num_tokens][rank]. */
int oracle_shrink(const uint16_t *x, int64_t ldx, int num_tokens, int hidden,
                  const uint16_t *const *lora_a, int num_slices, int rank, int max_loras,
                  float *buf, const int32_t *mapping, double scale,
                  const int32_t *tokens, int ntok, double *bound, int nthreads)
{
    int bad = 0;
    int count = tokens ? ntok : num_tokens;
    (void)nthreads;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : bad)
#endif
    for (int p = 0; p < count; ++p) {
        int t = tokens ? tokens[p] : p;
        int b = 0;
        int m = clean_id(mapping[t], max_loras, &b);
        bad |= b;
        for (int i = 0; i < num_slices; ++i) {
            for (int j = 0; j < rank; ++j) {
                if (bound)
                    bound[((int64_t)i * count + p) * rank + j] = 0.0;
                if (m == -1)
                    continue;
                const uint16_t *arow = lora_a[i] + ((int64_t)m * rank + j) * hidden;
                const uint16_t *xrow = x + (int64_t)t * ldx;
                double s = 0.0, sa = 0.0;
                for (int k = 0; k < hidden; ++k) {
                    double prod = bf16_to_double(xrow[k]) * bf16_to_double(arow[k]);
                    s += prod;
                    sa += fabs(prod);
                }
                float *dst = buf + ((int64_t)i * num_tokens + t) * rank + j;
                *dst = (float)((double)*dst + scale * s);
                if (bound)
                    bound[((int64_t)i * count + p) * rank + j] = fabs(scale) * sa;
            }
        }
    }
    return bad ? ORACLE_BAD_ID : ORACLE_OK;
}

/* lora_expand with the bias folded in: for every listed token t whose id m
 * is not -1, every slice i (columns start at offset_start and follow slice
 * after slice) and every c < widths[i],
 *     v = sum_j buf[i][t][j] * B_i[m][c][j]  (+ bias_i[m][c] if bias_i given)
 *     y[t][off_i + c] = bf16_rne((add_inputs ? y[t][off_i + c] : 0) + v)
 * `bias` may be NULL, or hold NULL entries.  If `mag` is not NULL it receives
 * add_inputs*|y0| + |bias| + sum_j |buf * B| at [p][col - offset_start].
 * Rows of tokens with id -1 are not touched. */
int oracle_expand(const float *buf, int num_tokens, int rank,
                  const uint16_t *const *lora_b, const uint16_t *const *bias,
                  const int32_t *widths, int num_slices, uint16_t *y, int64_t ldy,
                  int offset_start, int add_inputs, const int32_t *mapping, int max_loras,
                  const int32_t *tokens, int ntok, double *mag, int nthreads)
{
    int bad = 0;
    int count = tokens ? ntok : num_tokens;
    int64_t total_w = 0;
    for (int i = 0; i < num_slices; ++i)
        total_w += widths[i];
    (void)nthreads;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : bad)
#endif
    for (int p = 0; p < count; ++p) {
        int t = tokens ? tokens[p] : p;
        int b = 0;
        int m = clean_id(mapping[t], max_loras, &b);
        bad |= b;
        int64_t off = offset_start;
        for (int i = 0; i < num_slices; ++i) {
            for (int c = 0; c < widths[i]; ++c) {
                int64_t col = off + c;
                if (mag)
                    mag[(int64_t)p * total_w + (col - offset_start)] = 0.0;
                if (m == -1)
                    continue;
                const float *brow = buf + ((int64_t)i * num_tokens + t) * rank;
                const uint16_t *wrow = lora_b[i] + ((int64_t)m * widths[i] + c) * rank;
                double v = 0.0, mv = 0.0;
                for (int j = 0; j < rank; ++j) {
                    double prod = (double)brow[j] * bf16_to_double(wrow[j]);
                    v += prod;
                    mv += fabs(prod);
                }
                if (bias && bias[i]) {
                    double bv = bf16_to_double(bias[i][(int64_t)m * widths[i] + c]);
                    v += bv;
                    mv += fabs(bv);
                }
                uint16_t *dst = y + (int64_t)t * ldy + col;
                double y0 = add_inputs ? bf16_to_double(*dst) : 0.0;
                mv += fabs(y0);
                *dst = oracle_double_to_bf16(y0 + v);
                if (mag)
                    mag[(int64_t)p * total_w + (col - offset_start)] = mv;
            }
            off += widths[i];
        }
    }
    return bad ? ORACLE_BAD_ID : ORACLE_OK;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
