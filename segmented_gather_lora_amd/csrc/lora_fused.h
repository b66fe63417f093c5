// lora_fused.h -- the argument block, constants and device helpers shared by
// the two one-launch shrink->expand kernels: the tile-major kernel (work
// follows the sorted segments) and the LoRA-major kernel (work follows the
// LoRA ids, so weights are read before the batch is sorted).
#pragma once

#include "lora_internal.h"

namespace lora {

struct FusedArgs {
    ShrinkArgs s;
    ExpandArgs e;
    PrepareArgs p;          // the batch's mapping and metadata outputs (PREP kernels)
    int32_t *sync;
    int32_t *status;
    int32_t blocks;         // expand column blocks per tile (all slices)
    int32_t block_begin[LORA_MAX_SLICES + 1];   // prefix of column blocks per slice
    int32_t help_after;     // polls without progress before a waiter takes free parts
    int32_t owners_skip;    // test only: owners leave their parts to the waiters
};

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 16;            // tokens per tile
constexpr int kBlockCols = 256;      // expand columns per unit
constexpr int kWaveCols = 64;
constexpr int kSpinLimit = 1 << 18;  // polls about 0.5 us apart: ~0.1 s
// s_waitcnt vmcnt(0) with the other counters left at their maximum
constexpr int kVmcntZero = (7 << 4) | (15 << 8);

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return lo16 | (hi16 << 16); }
__device__ __forceinline__ int clamp_group(int c, int width) { return c < width ? c : width - 4; }

template <typename T, int N>
__device__ __forceinline__ T select_slice(const T (&p)[N], int i) {
    T r = p[0];
#pragma unroll
    for (int s = 1; s < N; ++s)
        if (i == s) r = p[s];
    return r;
}

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ void reset_tile(int32_t *words, int parts) {
    __hip_atomic_store(words + kFusedPartsDone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(words + kFusedPastWait, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int p = 0; p < parts; ++p) __hip_atomic_store(words + kFusedFlags + p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LoRAKernelMeta._reset + prepare_tensors ("lora_kernel_metadata" page) for a
// batch of at most kPrepMaxTokens tokens inside one workgroup of kThreads: the
// stable counting sort of the prepare kernel (each wave ranks the tokens of its
// contiguous slice with match masks and per-wave LDS counts; a scan over the
// keys gives segment starts and slice bases; every token is placed at
// base + rank), with 4 waves instead of 16.  The results land where
// build_tile_table leaves them -- the tile table of `tile_tokens`-token tiles
// followed by the sorted indices -- so the rest of the kernel is unchanged.
// Workgroup `writer` also writes the metadata arrays, exactly as the prepare
// kernel does.  Returns the number of tiles (0 for a no-LoRA batch).
constexpr int kPrepMaxTokens = 2048;

__device__ int prepare_in_lds(const PrepareArgs &p, int tile_tokens, int *smem, int *s_scan, int *s_flag,
                              bool writer) {
    constexpr int kSteps = kPrepMaxTokens / (kThreads);   // 64-token steps per wave at most
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int n = p.num_tokens;
    const int nkeys = p.max_loras + 1;   // = slots
    const int nbits = 32 - __clz(nkeys - 1);
    int *pre = smem, *sid = pre + nkeys + 1, *sst = sid + nkeys, *scn = sst + nkeys;
    int *ssorted = scn + nkeys;
    int *cnt = ssorted + n;   // [key][wave]: running counts, then slice bases

    for (int k = tid; k < nkeys * kWaves; k += kThreads) cnt[k] = 0;
    if (tid == 0) {
        s_flag[0] = 0;   // any id other than -1
        s_flag[1] = 0;   // an id out of range
    }
    const int steps = (n + kWaves * kWave - 1) / (kWaves * kWave);
    const int t0 = wave * steps * kWave;
    int ids[kSteps];
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {   // one round trip (addresses clamped)
        const int t = t0 + q * kWave + lane;
        ids[q] = p.mapping[t < n ? t : n - 1];
    }
    __syncthreads();

    // ---- 1. ranks within the wave's slice
    int keys[kSteps], ranks[kSteps];
    bool any = false, bad = false;
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
        keys[q] = 0;
        ranks[q] = 0;
        if (q >= steps) continue;   // uniform
        const int t = t0 + q * kWave + lane;
        const bool valid = t < n;
        int id = valid ? ids[q] : -1;
        if (id < -1 || id >= p.max_loras) {
            bad = true;
            id = -1;
        }
        const int key = id + 1;
        any |= valid && id != -1;
        const uint64_t m = match_key(key, valid, nbits);
        const bool leader = valid && (m & lanemask_lt()) == 0;
        keys[q] = key;
        ranks[q] = cnt[key * kWaves + wave] + __popcll(m & lanemask_lt());
        if (leader) cnt[key * kWaves + wave] += __popcll(m);   // this wave's column only
    }
    if (ballot(any) && lane == 0) atomicOr(&s_flag[0], 1);
    if (ballot(bad) && lane == 0) atomicOr(&s_flag[1], 1);
    __syncthreads();
    const bool no_lora = s_flag[0] == 0;

    // ---- 2. per key (contiguous keys per thread): count, non-empty, tiles; one scan of the three
    const int per = (nkeys + kThreads - 1) / kThreads;   // <= 4
    const int beg = tid * per;
    int c[4], tl[4], sc = 0, sne = 0, stl = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = beg + i;
        c[i] = 0;
        tl[i] = 0;
        if (i < per && k < nkeys) {
            for (int w = 0; w < kWaves; ++w) c[i] += cnt[k * kWaves + w];
            tl[i] = (k >= 1 && c[i] > 0 && !no_lora) ? (c[i] + tile_tokens - 1) / tile_tokens : 0;
        }
        sc += c[i];
        sne += c[i] > 0 ? 1 : 0;
        stl += tl[i];
    }
    const int ic = wave_inclusive_scan(sc), ine = wave_inclusive_scan(sne), itl = wave_inclusive_scan(stl);
    if (lane == kWave - 1) {
        s_scan[wave] = ic;
        s_scan[kWaves + wave] = ine;
        s_scan[2 * kWaves + wave] = itl;
    }
    __syncthreads();
    int start = ic - sc, slot = ine - sne, tpre = itl - stl, n_active = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        start += w < wave ? s_scan[w] : 0;
        slot += w < wave ? s_scan[kWaves + w] : 0;
        tpre += w < wave ? s_scan[2 * kWaves + w] : 0;
        n_active += s_scan[kWaves + w];
        total += s_scan[2 * kWaves + w];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = beg + i;
        if (i < per && k < nkeys) {
            if (c[i] > 0) {
                sid[slot] = k - 1;
                scn[slot] = c[i];
                sst[slot] = tl[i] ? start : 0;
                pre[slot] = tpre;
                if (writer && !no_lora) {
                    p.active_ids[slot] = k - 1;
                    p.counts[slot] = c[i];
                    p.start_loc[slot + 1] = start + c[i];
                }
                ++slot;
            }
            int run = start;
            for (int w = 0; w < kWaves; ++w) {
                const int v = cnt[k * kWaves + w];
                cnt[k * kWaves + w] = run;
                run += v;
            }
            start += c[i];
            tpre += tl[i];
        }
    }
    // padding slots own no tiles; the metadata gets the _reset values there
    for (int k = tid; k < nkeys; k += kThreads) {
        if (k >= n_active) {
            sid[k] = -1;
            scn[k] = 0;
            sst[k] = 0;
            pre[k] = total;
        }
        if (writer && (no_lora || k >= n_active)) {
            p.active_ids[k] = -1;
            p.counts[k] = 0;
        }
    }
    if (writer)
        for (int k = tid; k < nkeys + 1; k += kThreads)
            if (no_lora || k == 0 || k > n_active) p.start_loc[k] = 0;
    if (tid == 0) {
        pre[nkeys] = total;
        if (writer) {
            *p.no_lora = no_lora ? 1 : 0;
            *p.status = s_flag[1] ? LORA_ERR_ID_RANGE : 0;
        }
    }
    __syncthreads();

    // ---- 3. stable scatter into LDS (and the metadata's copies)
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
        const int t = t0 + q * kWave + lane;
        if (q < steps && t < n) {
            const int pos = cnt[keys[q] * kWaves + wave] + ranks[q];
            ssorted[pos] = t;
            if (writer && !no_lora) {
                p.sorted[pos] = t;
                p.mapping_copy[t] = keys[q] - 1;
            }
        }
    }
    __syncthreads();
    return total;
}

}  // namespace

// LoRA-major launch (lora_decode.hip): hipErrorNotSupported when the batch is
// outside its range, so the caller can take the tile-major kernel.  f.p holds
// the batch's ids, count and max_loras; with `prepare` the launch also writes
// the metadata arrays of f.p (its ids are then the raw mapping).
hipError_t launch_lora_major(const FusedArgs &f, bool prepare, hipStream_t stream);

}  // namespace lora
