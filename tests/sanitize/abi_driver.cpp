// Calls every entry point of include/lora_mi355x.h with arguments that the
// host-side checks reject, plus the host-only calls (lora_meta_bytes,
// lora_meta_bind on host memory, the launch-count query, lora_status_string),
// in a build whose host code has AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  No call reaches a
// kernel launch, so no GPU is needed.  Prints "ok" on success.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lora_mi355x.h"

static int failures = 0;
#define EXPECT(expr, want)                                                          \
    do {                                                                            \
        const int got_ = (expr);                                                    \
        if (got_ != (want)) {                                                       \
            fprintf(stderr, "%s:%d: %s = %d, want %d\n", __FILE__, __LINE__, #expr, \
                    got_, (int)(want));                                            \
            ++failures;                                                             \
        }                                                                           \
    } while (0)

int main() {
    // statuses
    for (int s = -12; s <= 1; ++s)
        if (!lora_status_string(s) || !*lora_status_string(s)) ++failures;

    // sizes and binding on host memory (nothing is written through the views)
    EXPECT((int)(lora_meta_bytes(0, 10) == 0), 1);
    EXPECT((int)(lora_meta_bytes(1024, 10) == 0), 1);
    EXPECT((int)(lora_meta_bytes(3, LORA_MAX_TOKENS + 1) == 0), 1);
    const int ml = 7, maxn = 300;
    const size_t nb = lora_meta_bytes(ml, maxn);
    void *raw = nullptr;
    if (posix_memalign(&raw, 256, nb) != 0) return 2;
    lora_meta_t m;
    EXPECT(lora_meta_bind(raw, nb, ml, maxn, &m), LORA_OK);
    EXPECT(lora_meta_bind(static_cast<char *>(raw) + 16, nb, ml, maxn, &m), LORA_ERR_BUFFER);
    EXPECT(lora_meta_bind(raw, nb - 1, ml, maxn, &m), LORA_ERR_BUFFER);
    EXPECT(lora_meta_bind(nullptr, nb, ml, maxn, &m), LORA_ERR_NULL);
    EXPECT(lora_meta_bind(raw, nb, 0, maxn, &m), LORA_ERR_MAX_LORAS);
    EXPECT(lora_meta_bind(raw, nb, ml, maxn, &m), LORA_OK);
    char *end = static_cast<char *>(raw) + nb;
    EXPECT((int)(reinterpret_cast<char *>(m.sync) < end), 1);

    // prepare: rejected before any launch
    int32_t ids[4] = {0, 1, -1, 2};
    EXPECT(lora_prepare_meta(ids, maxn + 1, &m, nullptr), LORA_ERR_NUM_TOKENS);
    EXPECT(lora_prepare_meta(ids, -1, &m, nullptr), LORA_ERR_NUM_TOKENS);
    EXPECT(lora_prepare_meta(nullptr, 4, &m, nullptr), LORA_ERR_NULL);
    EXPECT(lora_prepare_meta(ids, 4, nullptr, nullptr), LORA_ERR_NULL);

    // shrink / expand / fused: rejected by the argument checks
    alignas(16) static uint16_t x[64 * 72], a0[7 * 16 * 64], b0[7 * 64 * 16], y[64 * 96];
    alignas(16) static float buf[2 * 64 * 16];
    const void *a[2] = {a0, a0}, *b[2] = {b0, b0};
    const int widths[2] = {64, 32};
    m.num_tokens = 64;
    EXPECT(lora_shrink(x, 72, 63, 64, a, 2, 16, buf, &m, 1.f, nullptr), LORA_ERR_NUM_TOKENS);
    EXPECT(lora_shrink(x, 72, 64, 64, a, 0, 16, buf, &m, 1.f, nullptr), LORA_ERR_SLICES);
    EXPECT(lora_shrink(x, 72, 64, 60, a, 2, 16, buf, &m, 1.f, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_shrink(x, 72, 64, 64, a, 2, 12, buf, &m, 1.f, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_shrink(x + 1, 72, 64, 64, a, 2, 16, buf, &m, 1.f, nullptr), LORA_ERR_ALIGN);
    EXPECT(lora_expand(buf, 64, 16, b, nullptr, widths, 2, y, 88, 0, 1, &m, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_expand(buf, 64, 16, b, nullptr, widths, 9, y, 96, 0, 1, &m, nullptr), LORA_ERR_SLICES);
    EXPECT(lora_expand(buf, 64, 16, b, nullptr, widths, 2, y, 96, 4, 1, &m, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_shrink_expand(x, 72, 64, 64, a, b, nullptr, widths, 2, 16, buf, y, 88, 0, 1, &m, 1.f, nullptr),
           LORA_ERR_SHAPE);
    EXPECT(lora_prepare_shrink_expand(ids, maxn + 1, x, 72, 64, a, b, nullptr, widths, 2, 16, buf, y, 96, 0, 1, &m,
                                      1.f, nullptr),
           LORA_ERR_NUM_TOKENS);
    // empty batches return before any launch
    m.num_tokens = 0;
    EXPECT(lora_shrink(x, 72, 0, 64, a, 2, 16, buf, &m, 1.f, nullptr), LORA_OK);
    EXPECT(lora_expand(buf, 0, 16, b, nullptr, widths, 2, y, 96, 0, 1, &m, nullptr), LORA_OK);

    // launch-count query (host only) over a spread of shapes
    int seen = 0;
    for (int n = 1; n <= 40000; n = n * 3 + 1)
        for (int loras = 1; loras <= 1023; loras = loras * 4 + 3)
            for (int r = 8; r <= 128; r *= 2)
                for (int s = 1; s <= 8; s *= 2)
                    for (int prep = 0; prep < 2; ++prep) {
                        const int k = lora_shrink_expand_launches(n, loras, 4096, s, r, prep);
                        if (k < 1 || k > 4) ++failures;
                        ++seen;
                    }
    EXPECT(lora_shrink_expand_launches(0, 32, 4096, 3, 16, 1), LORA_ERR_NUM_TOKENS);
    EXPECT(lora_shrink_expand_launches(256, 32, 12, 3, 16, 1), LORA_ERR_SHAPE);

    // measurement aids: argument checks
    EXPECT(lora_probe_read(nullptr, 1024, 4, buf, nullptr), LORA_ERR_NULL);
    EXPECT(lora_probe_read(x, 1000, 4, buf, nullptr), LORA_ERR_SHAPE);
    EXPECT(lora_probe_read(x + 1, 1024, 4, buf, nullptr), LORA_ERR_ALIGN);
    EXPECT(lora_probe_empty(0, nullptr), LORA_ERR_SHAPE);

    free(raw);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok %d\n", seen);
    return 0;
}
