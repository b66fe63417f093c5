// lora_internal.h -- device helpers and kernel argument blocks shared by the
// gfx950 kernels of liblora_mi355x.so (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_mi355x.h"

namespace lora {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Wave index within the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (uint64_t(1) << lane_id()) - 1;
}

// Mask of the lanes whose `key` equals this lane's, among lanes with `valid`
// set: one ballot per key bit (keys are < 2^nbits).
__device__ __forceinline__ uint64_t match_key(int key, bool valid, int nbits) {
    uint64_t m = ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        bool bit = (key >> b) & 1;
        uint64_t bb = ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// Inclusive prefix sum over the 64 lanes of a wave, with DPP lane moves:
// shifts by 1, 2, 4, 8 inside each row of 16 lanes, then the last lane of a
// row is broadcast into the next row (row_bcast:15) and the last lane of row 1
// into rows 2 and 3 (row_bcast:31).  Lanes without a source add 0.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
    return v;
}

// Touch every 64-byte line of a kernel's argument block at entry with scalar
// loads issued together and waited for once, so that the scattered scalar
// loads of the arguments later in the kernel hit the scalar cache instead of
// each paying a memory round trip at its first use.  Only lines that lie
// inside the block are touched.
#define LORA_KA_LOAD(i, off) "s_load_dword %" #i ", %11, " #off "\n\t"
#define LORA_KA_L1 LORA_KA_LOAD(0, 0x0)
#define LORA_KA_L2 LORA_KA_L1 LORA_KA_LOAD(1, 0x40)
#define LORA_KA_L3 LORA_KA_L2 LORA_KA_LOAD(2, 0x80)
#define LORA_KA_L4 LORA_KA_L3 LORA_KA_LOAD(3, 0xc0)
#define LORA_KA_L5 LORA_KA_L4 LORA_KA_LOAD(4, 0x100)
#define LORA_KA_L6 LORA_KA_L5 LORA_KA_LOAD(5, 0x140)
#define LORA_KA_L7 LORA_KA_L6 LORA_KA_LOAD(6, 0x180)
#define LORA_KA_L8 LORA_KA_L7 LORA_KA_LOAD(7, 0x1c0)
#define LORA_KA_L9 LORA_KA_L8 LORA_KA_LOAD(8, 0x200)
#define LORA_KA_L10 LORA_KA_L9 LORA_KA_LOAD(9, 0x240)
#define LORA_KA_L11 LORA_KA_L10 LORA_KA_LOAD(10, 0x280)
#define LORA_KA_ASM(loads)                                                              \
    asm volatile(loads "s_waitcnt lgkmcnt(0)"                                           \
                 : "=&s"(d[0]), "=&s"(d[1]), "=&s"(d[2]), "=&s"(d[3]), "=&s"(d[4]),     \
                   "=&s"(d[5]), "=&s"(d[6]), "=&s"(d[7]), "=&s"(d[8]), "=&s"(d[9]),     \
                   "=&s"(d[10])                                                         \
                 : "s"(k)                                                               \
                 : "memory")

template <typename Args>
__device__ __forceinline__ void prefetch_kernargs() {
    constexpr int lines = (int)((sizeof(Args) + 63) / 64);
    static_assert(lines >= 1 && lines <= 11, "argument block larger than the prefetch covers");
    auto k = __builtin_amdgcn_kernarg_segment_ptr();
    int d[11];
    if constexpr (lines == 1) LORA_KA_ASM(LORA_KA_L1);
    else if constexpr (lines == 2) LORA_KA_ASM(LORA_KA_L2);
    else if constexpr (lines == 3) LORA_KA_ASM(LORA_KA_L3);
    else if constexpr (lines == 4) LORA_KA_ASM(LORA_KA_L4);
    else if constexpr (lines == 5) LORA_KA_ASM(LORA_KA_L5);
    else if constexpr (lines == 6) LORA_KA_ASM(LORA_KA_L6);
    else if constexpr (lines == 7) LORA_KA_ASM(LORA_KA_L7);
    else if constexpr (lines == 8) LORA_KA_ASM(LORA_KA_L8);
    else if constexpr (lines == 9) LORA_KA_ASM(LORA_KA_L9);
    else if constexpr (lines == 10) LORA_KA_ASM(LORA_KA_L10);
    else LORA_KA_ASM(LORA_KA_L11);
}

// Entry i of a per-slice table in the argument block; i is uniform or nearly
// so, and each entry is compared rather than indexed.
template <typename T, int N>
__device__ __forceinline__ T select_slice(const T (&p)[N], int i) {
    T r = p[0];
#pragma unroll
    for (int s = 1; s < N; ++s)
        if (i == s) r = p[s];
    return r;
}

// Pointer i of a kernel-argument pointer table, where i differs between
// lanes.  Every entry is taken through readfirstlane, so the table is read
// with scalar loads and the pick is a per-lane select; a plain p[i] would
// become a per-lane gather from the argument block on the vector memory path,
// whose wait also holds up every load issued before it.  The entries are
// rebuilt as global-memory pointers: rebuilt as plain (generic) pointers they
// would make flat loads, which count on the LDS counter as well, so that
// every LDS wait after them (the next barrier) would wait for them too.
template <typename T, int N>
__device__ __forceinline__ T *lane_slice_ptr(T *const (&p)[N], int i) {
    typedef __attribute__((address_space(1))) T GT;
    GT *r = nullptr;
#pragma unroll
    for (int s = 0; s < N; ++s) {
        const uint64_t v = reinterpret_cast<uint64_t>(p[s]);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
        GT *ps = (GT *)(((uint64_t)hi << 32) | lo);
        r = (s == 0 || i == s) ? ps : r;
    }
    return (T *)r;
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
    return __uint_as_float(h << 16);
}

// float -> bfloat16 bit pattern, round to nearest, ties to even (inputs are
// finite or inf; NaN maps to a quiet NaN).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const floatx4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) {
    return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------- metadata view

struct MetaView {
    const int32_t *sorted;       // token_indices_sorted
    const int32_t *active_ids;   // [max_loras + 1]
    const int32_t *counts;       // [max_loras + 1]
    const int32_t *start_loc;    // [max_loras + 2]
    const int32_t *no_lora;      // [1]
    int32_t nslots;              // max_loras + 1
    int32_t lds_tokens;          // > 0: the first lds_tokens sorted indices are copied to LDS
};

constexpr int kLdsTokensMax = 2048;   // batches up to this size keep sorted indices in LDS
constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, workgroups dispatched round-robin

// Per-workgroup table of work tiles, built in LDS from the metadata: every
// slot whose id is not -1 owns ceil(count / tile_tokens) tiles, in slot order
// (so no order of the segments is assumed).  Layout in `smem` (ints):
//   pre[nslots + 1]  exclusive prefix of tiles per slot (pre[nslots] = total)
//   sid[nslots], sstart[nslots], scnt[nslots]
// followed, for batches of at most kLdsTokensMax tokens, by the sorted token
// indices.  Every metadata read (the no-LoRA flag, ids, counts, segment
// starts, sorted indices) is issued before any is used: the table costs one
// memory round trip.  A batch flagged no-LoRA has no tiles (its reset
// metadata has none either).  All NTHREADS threads of the block must call it;
// returns the total number of tiles.
__device__ __forceinline__ int tile_table_ints(int nslots) { return 4 * nslots + 1; }

// Sorted token index `idx`: from the LDS copy made by build_tile_table when
// the batch is small (one memory round trip less per work unit), else HBM.
__device__ __forceinline__ int sorted_at(const MetaView &m, const int *smem, int idx) {
    return m.lds_tokens > 0 ? smem[4 * m.nslots + 1 + idx] : m.sorted[idx];
}

template <int NTHREADS>
__device__ __forceinline__ int build_tile_table(const MetaView &m, int tile_tokens, int *smem, int *s_wsum) {
    constexpr int kPerMax = (LORA_MAX_LORAS + 1 + NTHREADS - 1) / NTHREADS;   // slots per thread
    constexpr int kTokPer = (kLdsTokensMax + NTHREADS - 1) / NTHREADS;        // sorted indices per thread
    constexpr int kWavesT = NTHREADS / kWave;
    const int nslots = m.nslots;
    int *pre = smem, *sid = smem + nslots + 1, *sst = sid + nslots, *scn = sst + nslots;
    const int tid = threadIdx.x;
    const int per = (nslots + NTHREADS - 1) / NTHREADS;
    const int beg = tid * per;

    // ---- all loads first (clamped addresses, no branches)
    const int flag = *m.no_lora;
    int ids[kPerMax], cnt[kPerMax], st[kPerMax];
#pragma unroll
    for (int i = 0; i < kPerMax; ++i) {
        int k = beg + i;
        k = k < nslots ? k : nslots - 1;
        ids[i] = m.active_ids[k];
        cnt[i] = m.counts[k];
        st[i] = m.start_loc[k];
    }
    int tok[kTokPer];
    const int ntok = m.lds_tokens;
    if (ntok > 0) {
#pragma unroll
        for (int i = 0; i < kTokPer; ++i) {
            int k = tid + i * NTHREADS;
            k = k < ntok ? k : ntok - 1;
            tok[i] = m.sorted[k];
        }
    }

    // ---- LDS copies and the per-thread tile counts
    if (ntok > 0) {
#pragma unroll
        for (int i = 0; i < kTokPer; ++i) {
            const int k = tid + i * NTHREADS;
            if (k < ntok) smem[4 * nslots + 1 + k] = tok[i];
        }
    }
    int nt[kPerMax];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kPerMax; ++i) {
        const int k = beg + i;
        nt[i] = 0;
        if (i < per && k < nslots) {
            nt[i] = (flag == 0 && ids[i] >= 0) ? (cnt[i] + tile_tokens - 1) / tile_tokens : 0;
            sid[k] = ids[i];
            scn[k] = cnt[i];
            sst[k] = nt[i] ? st[i] : 0;
            sum += nt[i];
        }
    }
    const int lane = lane_id(), wave = tid / kWave;
    const int incl = wave_inclusive_scan(sum);
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWavesT; ++w) {
        const int v = s_wsum[w];
        base += w < wave ? v : 0;
        total += v;
    }
    int run = base + incl - sum;
#pragma unroll
    for (int i = 0; i < kPerMax; ++i) {
        const int k = beg + i;
        if (i < per && k < nslots) {
            pre[k] = run;
            run += nt[i];
        }
    }
    if (tid == 0) pre[nslots] = total;
    __syncthreads();
    return total;
}

struct TileRef {
    int lora_id, seg_start, seg_count, tile;
};

// Slot of tile `t` (< total): the last k with pre[k] <= t (binary search; the
// argument is uniform across the wave, so every read is an LDS broadcast).
__device__ __forceinline__ TileRef lookup_tile(const int *smem, int nslots, int t) {
    const int *pre = smem, *sid = smem + nslots + 1, *sst = sid + nslots, *scn = sst + nslots;
    int lo = 0, hi = nslots - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    TileRef r;
    r.lora_id = sid[lo];
    r.seg_start = sst[lo];
    r.seg_count = scn[lo];
    r.tile = t - pre[lo];
    return r;
}

// Units are numbered in a canonical order (tile-major) and cut into kNumXcd
// contiguous chunks; workgroup b walks chunk b % 8.  Workgroups are dealt to
// the XCDs round-robin, so all workgroups with the same b % 8 run on one XCD and
// neighbouring units -- the tiles of one segment, or the row/column blocks of
// one tile -- run on the same XCD and share its L2.
struct UnitWalker {
    int chunk, first, stride, limit, xcd;
    __device__ __forceinline__ UnitWalker(int units) {
        chunk = (units + kNumXcd - 1) / kNumXcd;
        xcd = blockIdx.x % kNumXcd;
        first = blockIdx.x / kNumXcd;
        stride = gridDim.x / kNumXcd;
        limit = units;
    }
    // unit index for the i-th step of this workgroup, or -1 when done
    __device__ __forceinline__ int unit(int j) const {
        if (j >= chunk) return -1;
        const int u = xcd * chunk + j;
        return u < limit ? u : -1;
    }
};

// ---------------------------------------------------------------- kernel args

struct PrepareArgs {
    const int32_t *mapping;
    int32_t *mapping_copy;
    int32_t *sorted;
    int32_t *active_ids;
    int32_t *counts;
    int32_t *start_loc;
    int32_t *no_lora;
    int32_t *status;
    int32_t *sync;        // work counters of the fused call, zeroed here
    float *acc;           // the fused call's accumulation area, zeroed here
    int32_t sync_tiles;   // tiles whose counters the batch can use (0: none)
    int32_t acc_floats;   // floats of the accumulation area the batch can use (0: none)
    int32_t num_tokens;
    int32_t max_loras;
};

struct ShrinkArgs {
    MetaView meta;
    const uint16_t *x;
    int64_t ldx;
    const uint16_t *a[LORA_MAX_SLICES];
    float *buf;
    int32_t num_tokens;
    int32_t hidden;
    int32_t rank;
    int32_t rows;         // num_slices * rank
    int32_t row_blocks;   // row blocks per tile
    int32_t k_splits;     // K chunks per tile
    int32_t k_chunk;      // elements of K per chunk (multiple of 64)
    int32_t num_units;    // tiles upper bound * row_blocks * k_splits
    int32_t overwrite;    // 1: buf = result (a fresh buffer), 0: buf += result
    float scale;
};

// The stream-K shrink's extra arguments: part slots and counters in the
// library-owned area (nullptr when the area has none), and the status word
// for a wait that times out.
struct SkArgs {
    float *slots;
    int32_t *counters;
    int32_t *status;
};

struct ExpandArgs {
    MetaView meta;
    const float *buf;
    const uint16_t *b[LORA_MAX_SLICES];
    const uint16_t *bias[LORA_MAX_SLICES];
    uint16_t *y;
    int64_t ldy;
    int32_t width[LORA_MAX_SLICES];
    int32_t col_off[LORA_MAX_SLICES];      // first y column of each slice
    int32_t run_begin[LORA_MAX_SLICES + 1];    // prefix of column-block runs per slice
    int32_t num_slices;
    int32_t num_tokens;
    int32_t rank;
    int32_t run_blocks;   // column blocks per run (the last run of a slice may be shorter)
    int32_t runs;         // total runs
    int32_t tile_tokens;  // tokens per work unit (multiple of 16)
    int32_t num_units;
    int32_t add_inputs;
    int32_t share;        // 1: workgroups take equal shares of the (tile, column block) list
};

// Launch-geometry overrides (0 = automatic), read from the environment by the
// API layer for tuning sweeps; they change tiling only, never the result.
struct ShrinkTuning {
    int tile_tokens;       // 16, 32, 64 or 128
    int waves_k;           // 1, 2 or 4
    int mtiles_per_wave;   // 1..4
    int k_splits;
    int grid_cap;
    int variant;           // 2 = direct-load kernel, 3 = LDS-staged kernel
    int staged_cfg;        // 1-based index into the LDS-staged configurations
    int stream_k;          // 0 automatic, 1 never, 2 whenever the batch allows it
};
struct ExpandTuning {
    int tile_tokens;       // 16, 32 or 64
    int grid_cap;
    int run_blocks;        // column blocks per unit
    int share;             // 0 automatic, 1 shares of the block list, 2 units of run_blocks
};

// Workgroups of kernel `fn` the device holds at once (host side, cached).
int resident_grid(const void *fn, int threads, size_t lds);
// Persistent grid: at most `units` workgroups and at most what is resident at
// once, a multiple of the XCD count (at least one workgroup per XCD).
inline long persistent_grid(long units, long cap, const void *fn, int threads, size_t lds) {
    long g = units < cap ? units : cap;
    const long res = resident_grid(fn, threads, lds);
    if (g > res) g = res;
    g = g / kNumXcd * kNumXcd;
    return g < kNumXcd ? kNumXcd : g;
}

// Host-side launchers (defined next to their kernels).
// Also zeroes the stream-K shrink's counters (sk_words words at sk_counters;
// none when sk_words is 0).
hipError_t launch_prepare(const PrepareArgs &a, int32_t *sk_counters, int sk_words, hipStream_t s);
// Kernel launches launch_prepare makes for a batch of n tokens (host only):
// 2 for batches sorted by several workgroups, else 1.
int prepare_launches(int n, int max_loras);
hipError_t launch_shrink(const ShrinkArgs &a, const SkArgs &sk, const ShrinkTuning &cfg, hipStream_t s);
// Kernel launches launch_shrink makes for these sizes (host only): 2 when a
// fresh buffer (overwrite) is combined from K chunks and its rows are zeroed
// first, else 1 (0 for an empty batch).
int shrink_launches(int n, int nslots, int rows, int hidden, bool overwrite, const ShrinkTuning &cfg);
hipError_t launch_expand(const ExpandArgs &a, const ExpandTuning &cfg, hipStream_t s);
// Fused shrink -> expand for short segments.  Returns hipErrorNotSupported
// (launching nothing) when the shape is outside the fused kernel's range; the
// caller then launches shrink and expand.  `mapping_copy` is the prepared
// batch's id copy (ids outside [-1, max_loras) already -1), read by the
// LoRA-major layout.
hipError_t launch_fused(const ShrinkArgs &s, const ExpandArgs &e, const int32_t *mapping_copy, int max_loras,
                        int32_t *sync, float *acc, float *slots, int32_t *status, int help_after, int owners_skip,
                        hipStream_t stream);
// The same with the batch's prepare done inside the launch (at most 2048
// tokens); hipErrorNotSupported likewise.
hipError_t launch_prepare_fused(const PrepareArgs &p, const ShrinkArgs &s, const ExpandArgs &e, int32_t *sync,
                                float *acc, float *slots, int32_t *status, int help_after, int owners_skip,
                                hipStream_t stream);

// The fused call serves batches of short segments only: fewer than 24
// tokens per LoRA on average, so at most kFusedMaxTokens tokens.
constexpr long kFusedMaxTokens = 24L * (LORA_MAX_LORAS + 1);
// Words of the fused call's counter area for batches of up to n tokens and
// nslots slots: 128 words (512 bytes) per 16-token tile: the exit counter,
// the polled done counter on a 128-byte line of its own, and one taken flag
// per shrink part (at most kFusedMaxParts).
constexpr int kFusedTileWords = 128;
constexpr int kFusedPastWait = 0, kFusedPartsDone = 32, kFusedFlags = 64;   // word offsets
constexpr int kFusedMaxParts = 64;
inline long fused_tiles(long n, long nslots) {
    if (n > kFusedMaxTokens) n = kFusedMaxTokens;
    return (n + 15) / 16 + (nslots < n ? nslots : n) + 1;
}
// After the counters, the fp32 accumulation area of the fused calls: the
// shrink parts add into it (it is laid out like buf, [S][N][r] with S*r <=
// kFusedAccPerToken), the expand reads it, and the last reader of each tile
// (or LoRA id) clears its rows again, so it is all zero between calls.
constexpr int kFusedAccPerToken = 64;
inline long fused_acc_floats(long n) { return kFusedAccPerToken * (n < kFusedMaxTokens ? n : kFusedMaxTokens); }
inline long fused_sync_words(long n, long nslots) {
    return kFusedTileWords * fused_tiles(n, nslots) + fused_acc_floats(n);
}
// Word offset of the accumulation area in a region bound for max_num_tokens.
inline long fused_acc_offset(long max_num_tokens, long nslots) {
    return kFusedTileWords * fused_tiles(max_num_tokens, nslots);
}
// After the accumulation area, the LoRA-major kernel's part slots: each
// shrink part stores its partial sums in a slot of its own ([part][S][N][r],
// S*r <= kFusedAccPerToken), and the expand adds the slots up, so that area
// needs no clearing.  Batches of at most kLmMaxTokens tokens, at most
// kLmMaxParts parts.
constexpr int kLmMaxParts = 16;
constexpr long kLmMaxTokens = 2048;
inline long lm_slot_floats(long n) { return (long)kLmMaxParts * kFusedAccPerToken * (n < kLmMaxTokens ? n : kLmMaxTokens); }
inline long fused_region_words(long max_num_tokens, long nslots) {
    return fused_sync_words(max_num_tokens, nslots) + lm_slot_floats(max_num_tokens);
}
// After the part slots, for regions bound for at least kSkMinTokens tokens,
// the stream-K shrink's area: kSkCounterWords counters (one per share
// boundary and row block, zeroed by prepare and left zero by every launch),
// then kSkSlotArea floats of part slots (one per workgroup, for the partial
// sums of the tile it starts in the middle of).  Up to kSkMaxGroups
// workgroups.
constexpr long kSkMinTokens = 1024;
constexpr int kSkMaxGroups = 512;
constexpr int kSkCounterWords = 1024;
constexpr long kSkSlotArea = 8L << 20;
inline long sk_region_words(long max_num_tokens) {
    return max_num_tokens >= kSkMinTokens ? kSkCounterWords + kSkSlotArea : 0;
}
inline long meta_region_words(long max_num_tokens, long nslots) {
    return fused_region_words(max_num_tokens, nslots) + sk_region_words(max_num_tokens);
}
// Batches a fused call can take (by size alone): fewer than 24 tokens per
// segment on average and at most kFusedMaxTokens tokens.  Only their
// counters need zeroing by prepare.
inline bool fused_batch(long n, long nslots) {
    if (n < 1 || n > kFusedMaxTokens) return false;
    const long segs = nslots < n ? nslots : n;
    return (n + segs - 1) / segs < 24;
}

// Batches that a one-launch call prepares itself: at most this many tokens.
constexpr long kPrepMaxTokensHost = 2048;

// Whether lora_shrink_expand (with_prepare: lora_prepare_shrink_expand) runs
// a layer of S * rank = rows weight rows in one launch: a decode-like batch
// (fused_batch), rows <= 64 and rank <= 64, and with the prepare at most
// kPrepMaxTokensHost tokens.  Host-only; the launcher and the launch-count
// query both use it.
inline bool one_launch_range(long n, long nslots, int rows, int rank, bool with_prepare) {
    if (!fused_batch(n, nslots) || rows > 64 || rank > 64) return false;
    return !with_prepare || n <= kPrepMaxTokensHost;
}

}  // namespace lora
