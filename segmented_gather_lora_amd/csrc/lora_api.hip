// lora_api.hip -- the C ABI of liblora_mi355x.so: argument checks on the host
// (before any HIP call, so a rejected call launches nothing), metadata region
// layout, and launch of the gfx950 kernels.  Declarations and the full
// contract are in include/lora_mi355x.h.
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "lora_internal.h"

using namespace lora;

// Workgroups of `fn` (256 threads, `lds` bytes of dynamic LDS) that the
// device can hold at once: the register/wave limit per CU from the runtime's
// occupancy query (cached per kernel and device), the LDS limit from the
// kernel's static LDS plus `lds`, times the CU count.  Persistent grids are
// capped at this so that no workgroup waits for another to exit.
int lora::resident_grid(const void *fn, int threads, size_t lds) {
    struct Entry {
        const void *fn;
        int dev, per_cu, cus;
        size_t static_lds, lds_per_cu;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1 << 30;
    Entry e{};
    bool found = false;
    {
        std::lock_guard<std::mutex> g(mu);
        for (const Entry &c : cache)
            if (c.fn == fn && c.dev == dev) {
                e = c;
                found = true;
                break;
            }
    }
    if (!found) {
        e.fn = fn;
        e.dev = dev;
        hipFuncAttributes attr;
        int v = 0;
        e.per_cu = (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, fn, threads, 0) == hipSuccess && v > 0) ? v : 1;
        e.cus = (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ? v : 1;
        e.lds_per_cu = (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess && v > 0)
                           ? (size_t)v : (size_t)65536;
        e.static_lds = hipFuncGetAttributes(&attr, fn) == hipSuccess ? attr.sharedSizeBytes : 0;
        std::lock_guard<std::mutex> g(mu);
        cache.push_back(e);
    }
    const size_t per_block = e.static_lds + lds;
    int per_cu = e.per_cu;
    if (per_block > 0) {
        const size_t by_lds = e.lds_per_cu / per_block;
        if ((size_t)per_cu > by_lds) per_cu = (int)(by_lds > 0 ? by_lds : 1);
    }
    return per_cu * e.cus;
}

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int env_int(const char *name) {
    const char *e = getenv(name);
    return e ? atoi(e) : 0;
}

MetaView view_of(const lora_meta_t *m) {
    MetaView v;
    v.sorted = m->token_indices_sorted;
    v.active_ids = m->active_lora_ids;
    v.counts = m->num_tokens_per_lora;
    v.start_loc = m->lora_token_start_loc;
    v.no_lora = m->no_lora_flag;
    v.nslots = m->max_loras + 1;
    v.lds_tokens = 0;
    return v;
}

int check_meta(const lora_meta_t *m) {
    if (!m) return LORA_ERR_NULL;
    if (!m->token_lora_mapping || !m->token_indices_sorted || !m->active_lora_ids ||
        !m->num_tokens_per_lora || !m->lora_token_start_loc || !m->no_lora_flag || !m->status || !m->sync)
        return LORA_ERR_NULL;
    if (m->max_loras < 1 || m->max_loras > LORA_MAX_LORAS) return LORA_ERR_MAX_LORAS;
    if (m->max_num_tokens < 0 || m->max_num_tokens > LORA_MAX_TOKENS) return LORA_ERR_NUM_TOKENS;
    return LORA_OK;
}

}  // namespace

extern "C" {

size_t lora_meta_bytes(int max_loras, int max_num_tokens) {
    if (max_loras < 1 || max_loras > LORA_MAX_LORAS || max_num_tokens < 0 || max_num_tokens > LORA_MAX_TOKENS)
        return 0;
    const size_t tok = round_up(sizeof(int32_t) * (size_t)(max_num_tokens > 0 ? max_num_tokens : 1));
    return 2 * tok + 2 * round_up(sizeof(int32_t) * (max_loras + 1)) +
           round_up(sizeof(int32_t) * (max_loras + 2)) + 2 * kAlign +
           round_up(sizeof(int32_t) * (size_t)meta_region_words(max_num_tokens, max_loras + 1));
}

int lora_meta_bind(void *dev, size_t bytes, int max_loras, int max_num_tokens, lora_meta_t *out) {
    if (!dev || !out) return LORA_ERR_NULL;
    if (max_loras < 1 || max_loras > LORA_MAX_LORAS) return LORA_ERR_MAX_LORAS;
    if (max_num_tokens < 0 || max_num_tokens > LORA_MAX_TOKENS) return LORA_ERR_NUM_TOKENS;
    if ((reinterpret_cast<uintptr_t>(dev) & (kAlign - 1)) != 0) return LORA_ERR_BUFFER;
    const size_t need = lora_meta_bytes(max_loras, max_num_tokens);
    if (bytes < need) return LORA_ERR_BUFFER;
    char *p = static_cast<char *>(dev);
    const size_t tok = round_up(sizeof(int32_t) * (size_t)(max_num_tokens > 0 ? max_num_tokens : 1));
    const size_t ids = round_up(sizeof(int32_t) * (max_loras + 1));
    out->token_lora_mapping = reinterpret_cast<int32_t *>(p);
    p += tok;
    out->token_indices_sorted = reinterpret_cast<int32_t *>(p);
    p += tok;
    out->active_lora_ids = reinterpret_cast<int32_t *>(p);
    p += ids;
    out->num_tokens_per_lora = reinterpret_cast<int32_t *>(p);
    p += ids;
    out->lora_token_start_loc = reinterpret_cast<int32_t *>(p);
    p += round_up(sizeof(int32_t) * (max_loras + 2));
    out->no_lora_flag = reinterpret_cast<int32_t *>(p);
    p += kAlign;
    out->status = reinterpret_cast<int32_t *>(p);
    p += kAlign;
    out->sync = reinterpret_cast<int32_t *>(p);
    out->host_no_lora = nullptr;
    out->max_loras = max_loras;
    out->max_num_tokens = max_num_tokens;
    out->num_tokens = -1;
    return LORA_OK;
}

}  // extern "C"

namespace {

// The fused calls' accumulation area: after the counters, at an offset fixed
// by the sizes the region was bound for.
float *fused_acc(const lora_meta_t *meta) {
    return reinterpret_cast<float *>(meta->sync + fused_acc_offset(meta->max_num_tokens, meta->max_loras + 1));
}

// The LoRA-major kernel's part slots, after the accumulation area.
float *fused_slots(const lora_meta_t *meta) {
    return reinterpret_cast<float *>(meta->sync + fused_sync_words(meta->max_num_tokens, meta->max_loras + 1));
}

// The stream-K shrink's counters and slots, after the part slots (nullptr
// when the region was bound for fewer than kSkMinTokens tokens).
int32_t *sk_counters(const lora_meta_t *meta) {
    if (sk_region_words(meta->max_num_tokens) == 0) return nullptr;
    return meta->sync + fused_region_words(meta->max_num_tokens, meta->max_loras + 1);
}
float *sk_slots(const lora_meta_t *meta) {
    int32_t *c = sk_counters(meta);
    return c ? reinterpret_cast<float *>(c + kSkCounterWords) : nullptr;
}

PrepareArgs prepare_args(const int32_t *mapping, int num_tokens, const lora_meta_t *meta) {
    PrepareArgs a;
    a.mapping = mapping;
    a.mapping_copy = meta->token_lora_mapping;
    a.sorted = meta->token_indices_sorted;
    a.active_ids = meta->active_lora_ids;
    a.counts = meta->num_tokens_per_lora;
    a.start_loc = meta->lora_token_start_loc;
    a.no_lora = meta->no_lora_flag;
    a.status = meta->status;
    a.sync = meta->sync;
    const bool fused = fused_batch(num_tokens, meta->max_loras + 1);
    a.sync_tiles = fused ? (int32_t)fused_tiles(num_tokens, meta->max_loras + 1) : 0;
    a.acc = fused_acc(meta);
    a.acc_floats = fused ? (int32_t)fused_acc_floats(num_tokens) : 0;
    a.num_tokens = num_tokens;
    a.max_loras = meta->max_loras;
    return a;
}

// The optional host copy of the no-LoRA flag, after a prepare on `stream`.
int mirror_flag(const lora_meta_t *meta, hipStream_t stream) {
    if (meta->host_no_lora &&
        hipMemcpyAsync(meta->host_no_lora, meta->no_lora_flag, sizeof(int32_t), hipMemcpyDeviceToHost, stream) !=
            hipSuccess)
        return LORA_ERR_LAUNCH;
    return LORA_OK;
}

}  // namespace

extern "C" {

int lora_prepare_meta(const int32_t *mapping, int num_tokens, lora_meta_t *meta, hipStream_t stream) {
    int st = check_meta(meta);
    if (st) return st;
    if (num_tokens < 0 || num_tokens > meta->max_num_tokens) return LORA_ERR_NUM_TOKENS;
    if (num_tokens > 0 && !mapping) return LORA_ERR_NULL;
    // the stream-K shrink's counters start every batch that may use it at zero
    int32_t *skc = sk_counters(meta);
    const int sk_words = skc && num_tokens >= kSkMinTokens ? kSkCounterWords : 0;
    if (launch_prepare(prepare_args(mapping, num_tokens, meta), skc, sk_words, stream) != hipSuccess)
        return LORA_ERR_LAUNCH;
    if ((st = mirror_flag(meta, stream))) return st;
    meta->num_tokens = num_tokens;
    return LORA_OK;
}

}  // extern "C"

namespace {

// Checks and kernel arguments of lora_shrink; `skip` is set when there is no
// work (num_tokens == 0).
int shrink_args(const void *x, int64_t ldx, int num_tokens, int hidden, const void *const *lora_a,
                int num_slices, int rank, float *buf, const lora_meta_t *meta, float scale, ShrinkArgs &a,
                bool &skip) {
    int st = check_meta(meta);
    if (st) return st;
    if (meta->num_tokens < 0 || num_tokens != meta->num_tokens) return LORA_ERR_NUM_TOKENS;
    if (num_slices < 1 || num_slices > LORA_MAX_SLICES) return LORA_ERR_SLICES;
    if (!lora_a) return LORA_ERR_NULL;
    if (hidden < 8 || hidden % 8 || ldx < hidden || ldx % 8) return LORA_ERR_SHAPE;
    if (rank < 8 || rank > LORA_MAX_RANK || rank % 8) return LORA_ERR_SHAPE;
    if (num_tokens > 0 && (!x || !buf)) return LORA_ERR_NULL;
    for (int i = 0; i < num_slices; ++i) {
        if (!lora_a[i]) return LORA_ERR_NULL;
        if (!aligned16(lora_a[i])) return LORA_ERR_ALIGN;
    }
    skip = num_tokens == 0;
    if (skip) return LORA_OK;
    if (!aligned16(x) || !aligned16(buf)) return LORA_ERR_ALIGN;

    memset(&a, 0, sizeof a);
    a.meta = view_of(meta);
    a.x = static_cast<const uint16_t *>(x);
    a.ldx = ldx;
    for (int i = 0; i < num_slices; ++i) a.a[i] = static_cast<const uint16_t *>(lora_a[i]);
    a.buf = buf;
    a.num_tokens = num_tokens;
    a.hidden = hidden;
    a.rank = rank;
    a.rows = num_slices * rank;
    a.scale = scale;
    return LORA_OK;
}

SkArgs sk_args(const lora_meta_t *meta) {
    SkArgs k;
    k.slots = sk_slots(meta);
    k.counters = sk_counters(meta);
    k.status = meta->status;
    return k;
}

ShrinkTuning shrink_tuning() {
    ShrinkTuning cfg;
    cfg.tile_tokens = env_int("LORA_SHRINK_TILE_TOKENS");
    cfg.waves_k = env_int("LORA_SHRINK_WAVES_K");
    cfg.mtiles_per_wave = env_int("LORA_SHRINK_MTILES");
    cfg.k_splits = env_int("LORA_SHRINK_KSPLIT");
    cfg.grid_cap = env_int("LORA_SHRINK_GRID");
    cfg.variant = env_int("LORA_SHRINK_VARIANT");
    cfg.staged_cfg = env_int("LORA_SHRINK_STAGED");
    cfg.stream_k = env_int("LORA_SHRINK_SK");
    return cfg;
}

// Checks and kernel arguments of lora_expand.
int expand_args(const float *buf, int num_tokens, int rank, const void *const *lora_b, const void *const *bias,
                const int *slice_widths, int num_slices, void *y, int64_t ldy, int offset_start, int add_inputs,
                const lora_meta_t *meta, ExpandArgs &a, bool &skip) {
    int st = check_meta(meta);
    if (st) return st;
    if (meta->num_tokens < 0 || num_tokens != meta->num_tokens) return LORA_ERR_NUM_TOKENS;
    if (num_slices < 1 || num_slices > LORA_MAX_SLICES) return LORA_ERR_SLICES;
    if (!lora_b || !slice_widths) return LORA_ERR_NULL;
    if (rank < 8 || rank > LORA_MAX_RANK || rank % 8) return LORA_ERR_SHAPE;
    if (ldy < 8 || ldy % 8 || offset_start < 0 || offset_start % 8) return LORA_ERR_SHAPE;
    int64_t total = offset_start;
    for (int i = 0; i < num_slices; ++i) {
        if (slice_widths[i] <= 0 || slice_widths[i] % 8) return LORA_ERR_SHAPE;
        total += slice_widths[i];
        if (!lora_b[i]) return LORA_ERR_NULL;
        if (!aligned16(lora_b[i])) return LORA_ERR_ALIGN;
        if (bias && bias[i] && !aligned16(bias[i])) return LORA_ERR_ALIGN;
    }
    if (total > ldy) return LORA_ERR_SHAPE;
    if (num_tokens > 0 && (!buf || !y)) return LORA_ERR_NULL;
    skip = num_tokens == 0;
    if (skip) return LORA_OK;
    if (!aligned16(buf) || !aligned16(y)) return LORA_ERR_ALIGN;

    memset(&a, 0, sizeof a);
    a.meta = view_of(meta);
    a.buf = buf;
    int off = offset_start;
    for (int i = 0; i < num_slices; ++i) {
        a.b[i] = static_cast<const uint16_t *>(lora_b[i]);
        a.bias[i] = bias ? static_cast<const uint16_t *>(bias[i]) : nullptr;
        a.width[i] = slice_widths[i];
        a.col_off[i] = off;
        off += slice_widths[i];
    }
    a.y = static_cast<uint16_t *>(y);
    a.ldy = ldy;
    a.num_slices = num_slices;
    a.num_tokens = num_tokens;
    a.rank = rank;
    a.add_inputs = add_inputs ? 1 : 0;
    return LORA_OK;
}

ExpandTuning expand_tuning() {
    ExpandTuning cfg;
    cfg.tile_tokens = env_int("LORA_EXPAND_TILE_TOKENS");
    if (cfg.tile_tokens % 16) cfg.tile_tokens = 0;
    cfg.grid_cap = env_int("LORA_EXPAND_GRID");
    cfg.run_blocks = env_int("LORA_EXPAND_RUN");
    cfg.share = env_int("LORA_EXPAND_SHARE");
    return cfg;
}

}  // namespace

extern "C" {

int lora_shrink(const void *x, int64_t ldx, int num_tokens, int hidden, const void *const *lora_a,
                int num_slices, int rank, float *buf, const lora_meta_t *meta, float scale,
                hipStream_t stream) {
    ShrinkArgs a;
    bool skip = false;
    const int st = shrink_args(x, ldx, num_tokens, hidden, lora_a, num_slices, rank, buf, meta, scale, a, skip);
    if (st || skip) return st;
    if (launch_shrink(a, sk_args(meta), shrink_tuning(), stream) != hipSuccess) return LORA_ERR_LAUNCH;
    return LORA_OK;
}

int lora_expand(const float *buf, int num_tokens, int rank, const void *const *lora_b, const void *const *bias,
                const int *slice_widths, int num_slices, void *y, int64_t ldy, int offset_start, int add_inputs,
                const lora_meta_t *meta, hipStream_t stream) {
    ExpandArgs a;
    bool skip = false;
    const int st = expand_args(buf, num_tokens, rank, lora_b, bias, slice_widths, num_slices, y, ldy, offset_start,
                               add_inputs, meta, a, skip);
    if (st || skip) return st;
    if (launch_expand(a, expand_tuning(), stream) != hipSuccess) return LORA_ERR_LAUNCH;
    return LORA_OK;
}

int lora_shrink_expand(const void *x, int64_t ldx, int num_tokens, int hidden, const void *const *lora_a,
                       const void *const *lora_b, const void *const *bias, const int *slice_widths,
                       int num_slices, int rank, float *buf, void *y, int64_t ldy, int offset_start,
                       int add_inputs, const lora_meta_t *meta, float scale, hipStream_t stream) {
    ShrinkArgs sa;
    ExpandArgs ea;
    bool skip = false;
    int st = shrink_args(x, ldx, num_tokens, hidden, lora_a, num_slices, rank, buf, meta, scale, sa, skip);
    if (st) return st;
    st = expand_args(buf, num_tokens, rank, lora_b, bias, slice_widths, num_slices, y, ldy, offset_start,
                     add_inputs, meta, ea, skip);
    if (st || skip) return st;
    sa.overwrite = 1;   // add_lora_linear's buffer is a fresh one: buf = shrink
    const bool fused_allowed = env_int("LORA_FUSED") >= 0;   // LORA_FUSED=-1: always two launches
    if (fused_allowed) {
        // test knobs: polls before a waiter helps (default 128), owners leaving
        // their parts to the waiters (forces the helping path)
        const int help = getenv("LORA_FUSED_HELP_AFTER") ? env_int("LORA_FUSED_HELP_AFTER") : 128;
        const hipError_t e = launch_fused(sa, ea, meta->token_lora_mapping, meta->max_loras, meta->sync, fused_acc(meta),
                                          fused_slots(meta), meta->status,
                                          help, env_int("LORA_FUSED_OWNERS_SKIP"), stream);
        if (e == hipSuccess) return LORA_OK;
        if (e != hipErrorNotSupported) return LORA_ERR_LAUNCH;
    }
    if (launch_shrink(sa, sk_args(meta), shrink_tuning(), stream) != hipSuccess) return LORA_ERR_LAUNCH;
    if (launch_expand(ea, expand_tuning(), stream) != hipSuccess) return LORA_ERR_LAUNCH;
    return LORA_OK;
}

int lora_shrink_expand_launches(int num_tokens, int max_loras, int hidden, int num_slices, int rank,
                                int with_prepare) {
    if (num_tokens < 1 || num_tokens > LORA_MAX_TOKENS) return LORA_ERR_NUM_TOKENS;
    if (max_loras < 1 || max_loras > LORA_MAX_LORAS) return LORA_ERR_MAX_LORAS;
    if (num_slices < 1 || num_slices > LORA_MAX_SLICES) return LORA_ERR_SLICES;
    if (rank < 8 || rank > LORA_MAX_RANK || rank % 8) return LORA_ERR_SHAPE;
    if (hidden < 8 || hidden % 8) return LORA_ERR_SHAPE;
    if (env_int("LORA_FUSED") >= 0 &&
        one_launch_range(num_tokens, (long)max_loras + 1, num_slices * rank, rank, with_prepare != 0))
        return 1;
    return (with_prepare ? prepare_launches(num_tokens, max_loras) : 0) +
           shrink_launches(num_tokens, max_loras + 1, num_slices * rank, hidden, true, shrink_tuning()) + 1;
}

int lora_prepare_meta_launches(int num_tokens, int max_loras) {
    if (num_tokens < 0 || num_tokens > LORA_MAX_TOKENS) return LORA_ERR_NUM_TOKENS;
    if (max_loras < 1 || max_loras > LORA_MAX_LORAS) return LORA_ERR_MAX_LORAS;
    return prepare_launches(num_tokens, max_loras);
}

int lora_prepare_shrink_expand(const int32_t *mapping, int num_tokens, const void *x, int64_t ldx, int hidden,
                               const void *const *lora_a, const void *const *lora_b, const void *const *bias,
                               const int *slice_widths, int num_slices, int rank, float *buf, void *y,
                               int64_t ldy, int offset_start, int add_inputs, lora_meta_t *meta, float scale,
                               hipStream_t stream) {
    int st = check_meta(meta);
    if (st) return st;
    if (num_tokens < 0 || num_tokens > meta->max_num_tokens) return LORA_ERR_NUM_TOKENS;
    if (num_tokens > 0 && !mapping) return LORA_ERR_NULL;
    // the layer's arguments are checked against the batch about to be prepared
    lora_meta_t m = *meta;
    m.num_tokens = num_tokens;
    ShrinkArgs sa;
    ExpandArgs ea;
    bool skip = false;
    if ((st = shrink_args(x, ldx, num_tokens, hidden, lora_a, num_slices, rank, buf, &m, scale, sa, skip))) return st;
    if ((st = expand_args(buf, num_tokens, rank, lora_b, bias, slice_widths, num_slices, y, ldy, offset_start,
                          add_inputs, &m, ea, skip)))
        return st;
    if (!skip && env_int("LORA_FUSED") >= 0) {
        const int help = getenv("LORA_FUSED_HELP_AFTER") ? env_int("LORA_FUSED_HELP_AFTER") : 128;
        const hipError_t e = launch_prepare_fused(prepare_args(mapping, num_tokens, meta), sa, ea, meta->sync,
                                                  fused_acc(meta), fused_slots(meta), meta->status, help, env_int("LORA_FUSED_OWNERS_SKIP"), stream);
        if (e == hipSuccess) {
            if ((st = mirror_flag(meta, stream))) return st;
            meta->num_tokens = num_tokens;
            return LORA_OK;
        }
        if (e != hipErrorNotSupported) return LORA_ERR_LAUNCH;
    }
    if ((st = lora_prepare_meta(mapping, num_tokens, meta, stream))) return st;
    return lora_shrink_expand(x, ldx, num_tokens, hidden, lora_a, lora_b, bias, slice_widths, num_slices, rank, buf,
                              y, ldy, offset_start, add_inputs, meta, scale, stream);
}

const char *lora_status_string(int status) {
    switch (status) {
        case LORA_OK: return "ok";
        case LORA_ERR_NULL: return "a required pointer is NULL";
        case LORA_ERR_NUM_TOKENS: return "num_tokens out of range or different from the prepared batch";
        case LORA_ERR_SHAPE: return "hidden, rank, slice width or leading dimension out of range";
        case LORA_ERR_MAX_LORAS: return "max_loras out of range";
        case LORA_ERR_BUFFER: return "metadata region too small or not 256-byte aligned";
        case LORA_ERR_ALIGN: return "operand not 16-byte aligned";
        case LORA_ERR_SLICES: return "num_slices out of range";
        case LORA_ERR_LAUNCH: return "HIP launch failed";
        case LORA_ERR_ID_RANGE: return "a LoRA id was outside [-1, max_loras) and was treated as -1";
        case LORA_ERR_SYNC: return "a shrink's wait on the device timed out";
        case LORA_ERR_SCRATCH: return "the shrink buffer would exceed the library's static device array";
        default: return "unknown status";
    }
}

}  // extern "C"
