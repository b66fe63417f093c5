// lora_prepare.hip -- per-batch LoRA kernel metadata on one workgroup.
//
// Computes what LoRAKernelMeta._reset + prepare_tensors compute ("lora_kernel_metadata"
// page): the all(-1) no-LoRA flag with its early exit, the mapping copy, the
// stable sort of token indices by id, the ascending distinct ids with their
// counts (torch.unique(sorted=True, return_counts=True)) and their running
// sums (torch.cumsum) shifted by one slot.  The sort is a counting sort over
// the <= 1024 keys (key = id + 1), stable and bit-exact by construction.
//
// The batch is cut into 16 contiguous slices, one per wave, so a token's
// sorted position is
//   start[key] + sum over earlier slices of count[slice][key]
//              + number of equal keys before it in its own slice.
//   1. Each wave walks its slice 64 tokens at a time with no barrier: the
//      equal keys of a step are grouped with one ballot per key bit (match
//      mask), a token's rank in the slice is the slice's running count of its
//      key plus the popcount of the match mask below its lane, and one lane
//      per group bumps the running count (an LDS row owned by the wave).
//   2. One thread per key adds up its 16 slice counts (the histogram), a
//      block scan over the keys gives the segment starts and the compacted
//      id list, and each key's 16 counts become 16 slice bases.
//   3. Every token is written to base[key][slice] + rank.
// A slice's keys are loaded in one batch and kept in registers with their
// ranks when the slice has at most kSteps steps of 64 tokens; longer slices
// park (key, rank) in the mapping-copy array between steps 1 and 3.
#include "lora_internal.h"

namespace lora {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxKeys = LORA_MAX_LORAS + 1;
constexpr int kSteps = 16;     // steps of 64 tokens per wave held in registers
constexpr int kRankBits = 21;  // (key << 21) | rank: keys < 1024, ranks < 2^21 tokens
constexpr int kRankMask = (1 << kRankBits) - 1;
// Batches whose ranks stay in registers (kSteps steps of 64 tokens per wave)
// also stage the sorted indices in LDS and write them out coalesced: a direct
// scatter from one workgroup costs a partial cache-line write per token.
constexpr int kLdsSorted = kSteps * kThreads;

// 16-byte groups per tile of the fused call's counters: the exit count, the
// done count and the part flags.
constexpr int kSyncGroups = 2 + kFusedMaxParts / 4;

// Workgroups 1.. of the launch: the fused call's counters and accumulation
// area start every batch at zero (each fused call also leaves them zero),
// cleared next to the sort instead of by the sorting workgroup.
__device__ __forceinline__ void clear_fused_area(const PrepareArgs &a, int32_t *sk_counters, int sk_words) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int stride = (gridDim.x - 1) * kThreads;
    const int first = (blockIdx.x - 1) * kThreads + threadIdx.x;
    for (int k = first; k < a.sync_tiles * kSyncGroups; k += stride) {
        const int tile = k / kSyncGroups, w = k % kSyncGroups;
        const int word = w == 0 ? kFusedPastWait : w == 1 ? kFusedPartsDone : kFusedFlags + 4 * (w - 2);
        *reinterpret_cast<u32x4 *>(a.sync + kFusedTileWords * tile + word) = z;
    }
    for (int k = first; k < a.acc_floats / 4; k += stride) reinterpret_cast<u32x4 *>(a.acc)[k] = z;
    for (int k = first; k < sk_words / 4; k += stride) reinterpret_cast<u32x4 *>(sk_counters)[k] = z;
}

__global__ __launch_bounds__(kThreads) void prepare_kernel(PrepareArgs a, int32_t *sk_counters, int sk_words) {
    prefetch_kernargs<PrepareArgs>();
    if (blockIdx.x > 0) {
        clear_fused_area(a, sk_counters, sk_words);
        return;
    }
    // per wave and key: the running count of the wave's slice (later its
    // base).  Wave-major, so the lanes of a step, which hold different keys,
    // reach different banks.
    __shared__ __attribute__((aligned(16))) int s_cnt[kWaves][kMaxKeys];
    __shared__ int s_wa[kWaves], s_wb[kWaves];
    __shared__ int s_any, s_bad;
    __shared__ __attribute__((aligned(16))) int s_sorted[kLdsSorted];

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int n = a.num_tokens;
    const int nkeys = a.max_loras + 1;
    const int nbits = 32 - __clz(nkeys - 1);   // keys 0 .. nkeys-1 fit in nbits
    const int steps = (n + kThreads - 1) / kThreads;   // 64-token steps per wave
    const int slice = steps * kWave;                    // tokens per wave
    const int t0 = wave * slice;
    const bool in_regs = steps <= kSteps;

    for (int k = tid; k < kWaves * nkeys; k += kThreads) s_cnt[k / nkeys][k % nkeys] = 0;
    if (tid == 0) {
        s_any = 0;
        s_bad = 0;
    }
    __syncthreads();

    // _reset values and the no-LoRA flag, then the pages' early return
    // (sorted indices untouched; the mapping copy too unless it served as
    // scratch for a long batch)
    auto no_lora_exit = [&]() {
        if (tid == 0) {
            *a.no_lora = 1;
            *a.status = s_bad ? LORA_ERR_ID_RANGE : 0;
        }
        for (int k = tid; k < nkeys; k += kThreads) {
            a.active_ids[k] = -1;
            a.counts[k] = 0;
        }
        for (int k = tid; k < nkeys + 1; k += kThreads) a.start_loc[k] = 0;
    };

    // ---- 1. ranks within the wave's slice
    int packed[kSteps];
    int ids[kSteps];
    bool any = false, bad = false;
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int q = 0; q < kSteps; ++q) {   // one round trip for the chunk (addresses clamped)
            const int t = t0 + (c0 + q) * kWave + lane;
            if (c0 + q < steps) ids[q] = a.mapping[t < n ? t : n - 1];   // uniform
        }
    };
    for (int c0 = 0; c0 < steps; c0 += kSteps) {
        load_chunk(c0);
#pragma unroll
        for (int q = 0; q < kSteps; ++q) {
            if (c0 + q >= steps) break;   // uniform
            const int t = t0 + (c0 + q) * kWave + lane;
            const bool valid = t < n;
            int id = valid ? ids[q] : -1;
            if (id < -1 || id >= a.max_loras) {
                bad = true;
                id = -1;
            }
            const int key = id + 1;
            any |= valid && id != -1;
            // a step whose valid tokens all share one key (an all -1 stretch, a
            // run of one id) needs no per-bit ballots: they all match each other
            const int k0 = __builtin_amdgcn_readfirstlane(key);
            const uint64_t m = ballot(valid && key != k0) == 0 ? ballot(valid) : match_key(key, valid, nbits);
            const bool leader = valid && (m & lanemask_lt()) == 0;
            const int rank = s_cnt[wave][key] + __popcll(m & lanemask_lt());
            packed[q] = (key << kRankBits) | rank;
            if (leader) s_cnt[wave][key] += __popcll(m);   // this wave's row only
        }
        if (!in_regs) {
#pragma unroll
            for (int q = 0; q < kSteps; ++q) {
                const int t = t0 + (c0 + q) * kWave + lane;
                if (c0 + q < steps && t < n) a.mapping_copy[t] = packed[q];
            }
        }
    }
    if (ballot(any) && lane == 0) atomicOr(&s_any, 1);
    if (ballot(bad) && lane == 0) atomicOr(&s_bad, 1);
    __syncthreads();

    if (s_any == 0) {
        no_lora_exit();
        return;
    }
    if (tid == 0) {
        *a.no_lora = 0;
        *a.status = s_bad ? LORA_ERR_ID_RANGE : 0;
    }

    // ---- 2. histogram, scan over keys (nkeys <= kThreads: one key per thread), slice bases
    int col[kWaves];
    int c = 0;
    if (tid < nkeys) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            col[w] = s_cnt[w][tid];
            c += col[w];
        }
    }
    const int ne = c > 0 ? 1 : 0;
    const int ic = wave_inclusive_scan(c), ine = wave_inclusive_scan(ne);
    if (lane == kWave - 1) {
        s_wa[wave] = ic;
        s_wb[wave] = ine;
    }
    __syncthreads();
    int start = ic - c, slot = ine - ne, n_active = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int va = s_wa[w], vb = s_wb[w];
        start += w < wave ? va : 0;
        slot += w < wave ? vb : 0;
        n_active += vb;
    }
    if (ne) {
        a.active_ids[slot] = tid - 1;
        a.counts[slot] = c;
        a.start_loc[slot + 1] = start + c;
    }
    if (tid < nkeys) {
        int run = start;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            s_cnt[w][tid] = run;
            run += col[w];
        }
    }
    for (int k = tid; k < nkeys; k += kThreads) {
        if (k >= n_active) {
            a.active_ids[k] = -1;
            a.counts[k] = 0;
        }
    }
    for (int k = tid; k < nkeys + 1; k += kThreads)
        if (k == 0 || k > n_active) a.start_loc[k] = 0;
    __syncthreads();

    // ---- 3. stable scatter
    if (in_regs) {   // n <= kLdsSorted: into LDS, then one coalesced pass
#pragma unroll
        for (int q = 0; q < kSteps; ++q) {
            const int t = t0 + q * kWave + lane;
            if (q < steps && t < n) {
                const int key = (int)((unsigned)packed[q] >> kRankBits), rank = packed[q] & kRankMask;
                const int pos = s_cnt[wave][key] + rank;
                if ((unsigned)pos < (unsigned)n) s_sorted[pos] = t;
                a.mapping_copy[t] = key - 1;
            }
        }
        __syncthreads();
        int k0 = 0;
        if ((reinterpret_cast<uintptr_t>(a.sorted) & 15) == 0) {
            k0 = n & ~3;
            for (int k = 4 * tid; k < k0; k += 4 * kThreads)
                *reinterpret_cast<u32x4 *>(a.sorted + k) = *reinterpret_cast<const u32x4 *>(&s_sorted[k]);
        }
        for (int k = k0 + tid; k < n; k += kThreads) a.sorted[k] = s_sorted[k];
    } else {
        for (int s = 0; s < steps; ++s) {
            const int t = t0 + s * kWave + lane;
            if (t < n) {
                const int v = a.mapping_copy[t];
                const int key = (int)((unsigned)v >> kRankBits), rank = v & kRankMask;
                const int pos = s_cnt[wave][key] + rank;
                if ((unsigned)pos < (unsigned)n) a.sorted[pos] = t;
                a.mapping_copy[t] = key - 1;
            }
        }
    }
}

// ---- Several workgroups, for batches of at least kMultiMin tokens.  The
// batch is cut into G contiguous chunks, one per workgroup, and the sort
// runs in two launches:
//   rank: each workgroup ranks its chunk as above (per-wave slices, match
//         masks) and turns the ranks into ranks within the chunk; it writes
//         (key, rank) per token and its chunk's count per key to scratch,
//         and whether the chunk holds a valid id or an id out of range;
//   place: every workgroup adds, per key, the counts of the chunks before
//         its own and scans the keys' totals (the same scan on every
//         workgroup), so a token's position is
//           start[key] + counts of key in earlier chunks + rank in chunk;
//         workgroup 0 also writes the distinct ids, counts, segment starts,
//         flag and status.
// The stable order is that of the single workgroup: chunks, then slices,
// then lanes, all in token order.  Scratch: the library-owned stream-K slot
// area (N + G * (max_loras + 2) words).
constexpr int kMultiMin = 4096;
constexpr int kMultiWork = 64;
constexpr int kMultiMaxGroups = 64;

__device__ __forceinline__ int *multi_packed(int32_t *scratch) { return scratch; }
__device__ __forceinline__ int *multi_hist(int32_t *scratch, int n, int nkeys, int g) {
    return scratch + n + g * (nkeys + 1);
}

__global__ __launch_bounds__(kThreads) void prepare_rank_kernel(PrepareArgs a, int32_t *scratch, int chunk) {
    __shared__ __attribute__((aligned(16))) int s_cnt[kWaves][kMaxKeys];
    __shared__ int s_any, s_bad;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int n = a.num_tokens, g = blockIdx.x;
    const int nkeys = a.max_loras + 1;
    const int nbits = 32 - __clz(nkeys - 1);
    const int c0 = g * chunk, len = min(chunk, n - c0);
    const int steps = (len + kThreads - 1) / kThreads;
    const int slice = steps * kWave;
    const int t0 = c0 + wave * slice, tend = c0 + len;
    const bool in_regs = steps <= kSteps;
    int *packed_out = multi_packed(scratch);

    for (int k = tid; k < kWaves * nkeys; k += kThreads) s_cnt[k / nkeys][k % nkeys] = 0;
    if (tid == 0) {
        s_any = 0;
        s_bad = 0;
    }
    __syncthreads();

    int packed[kSteps];
    int ids[kSteps];
    bool any = false, bad = false;
    for (int cs = 0; cs < steps; cs += kSteps) {
#pragma unroll
        for (int q = 0; q < kSteps; ++q) {
            const int t = t0 + (cs + q) * kWave + lane;
            if (cs + q < steps) ids[q] = a.mapping[t < tend ? t : tend - 1];   // uniform
        }
#pragma unroll
        for (int q = 0; q < kSteps; ++q) {
            if (cs + q >= steps) break;   // uniform
            const int t = t0 + (cs + q) * kWave + lane;
            const bool valid = t < tend;
            int id = valid ? ids[q] : -1;
            if (id < -1 || id >= a.max_loras) {
                bad = true;
                id = -1;
            }
            const int key = id + 1;
            any |= valid && id != -1;
            const int k0 = __builtin_amdgcn_readfirstlane(key);
            const uint64_t m = ballot(valid && key != k0) == 0 ? ballot(valid) : match_key(key, valid, nbits);
            const bool leader = valid && (m & lanemask_lt()) == 0;
            const int rank = s_cnt[wave][key] + __popcll(m & lanemask_lt());
            packed[q] = (key << kRankBits) | rank;
            if (leader) s_cnt[wave][key] += __popcll(m);
        }
        if (!in_regs) {
#pragma unroll
            for (int q = 0; q < kSteps; ++q) {
                const int t = t0 + (cs + q) * kWave + lane;
                if (cs + q < steps && t < tend) packed_out[t] = packed[q];
            }
        }
    }
    if (ballot(any) && lane == 0) atomicOr(&s_any, 1);
    if (ballot(bad) && lane == 0) atomicOr(&s_bad, 1);
    __syncthreads();
    // per key: the chunk's count, and each wave's base within the chunk
    int *hist = multi_hist(scratch, n, nkeys, g);
    if (tid < nkeys) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int c = s_cnt[w][tid];
            s_cnt[w][tid] = run;
            run += c;
        }
        hist[tid] = run;
    }
    if (tid == 0) hist[nkeys] = s_any | (s_bad << 1);
    __syncthreads();
    // ranks within the chunk
    if (in_regs) {
#pragma unroll
        for (int q = 0; q < kSteps; ++q) {
            const int t = t0 + q * kWave + lane;
            if (q < steps && t < tend) {
                const int key = (int)((unsigned)packed[q] >> kRankBits);
                packed_out[t] = packed[q] + s_cnt[wave][key];
            }
        }
    } else {
        for (int q = 0; q < steps; ++q) {
            const int t = t0 + q * kWave + lane;
            if (t < tend) {
                const int v = packed_out[t];
                packed_out[t] = v + s_cnt[wave][(int)((unsigned)v >> kRankBits)];
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void prepare_place_kernel(PrepareArgs a, int32_t *scratch, int chunk, int groups,
                                                                 int32_t *sk_counters, int sk_words) {
    if ((int)blockIdx.x >= groups) {
        // the remaining workgroups clear the fused calls' and the stream-K
        // shrink's counters (the clearing below indexes from workgroup 1)
        PrepareArgs c = a;
        const u32x4 z = {0u, 0u, 0u, 0u};
        const int stride = (gridDim.x - groups) * kThreads;
        const int first = (blockIdx.x - groups) * kThreads + threadIdx.x;
        for (int k = first; k < c.sync_tiles * kSyncGroups; k += stride) {
            const int tile = k / kSyncGroups, w = k % kSyncGroups;
            const int word = w == 0 ? kFusedPastWait : w == 1 ? kFusedPartsDone : kFusedFlags + 4 * (w - 2);
            *reinterpret_cast<u32x4 *>(c.sync + kFusedTileWords * tile + word) = z;
        }
        for (int k = first; k < c.acc_floats / 4; k += stride) reinterpret_cast<u32x4 *>(c.acc)[k] = z;
        for (int k = first; k < sk_words / 4; k += stride) reinterpret_cast<u32x4 *>(sk_counters)[k] = z;
        return;
    }
    __shared__ int s_base[kMaxKeys];
    __shared__ int s_wa[kWaves], s_wb[kWaves];
    __shared__ int s_flags;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int n = a.num_tokens, g = blockIdx.x;
    const int nkeys = a.max_loras + 1;
    const int c0 = g * chunk, tend = min(c0 + chunk, n);
    const int *packed = multi_packed(scratch);
    // this thread's first token, loaded now so that its round trip overlaps
    // the counts' (a chunk holds at most kThreads tokens when g < kMultiMaxGroups)
    const int v0 = c0 + tid < tend ? packed[c0 + tid] : 0;
    if (tid == 0) s_flags = 0;
    __syncthreads();
    if (tid < groups) {
        const int f = multi_hist(scratch, n, nkeys, tid)[nkeys];
        if (f) atomicOr(&s_flags, f);
    }
    // per key: counts in the chunks before this one, and in all chunks
    // (16 loads in flight at a time)
    int before = 0, c = 0;
    if (tid < nkeys) {
        for (int k0 = 0; k0 < groups; k0 += 16) {
            int h[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) h[q] = k0 + q < groups ? multi_hist(scratch, n, nkeys, k0 + q)[tid] : 0;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                before += k0 + q < g ? h[q] : 0;
                c += h[q];
            }
        }
    }
    __syncthreads();
    const bool any = s_flags & 1, bad = (s_flags >> 1) & 1;
    if (!any) {   // the pages' early return: reset values and the flag only
        if (g == 0) {
            if (tid == 0) {
                *a.no_lora = 1;
                *a.status = bad ? LORA_ERR_ID_RANGE : 0;
            }
            for (int k = tid; k < nkeys; k += kThreads) {
                a.active_ids[k] = -1;
                a.counts[k] = 0;
            }
            for (int k = tid; k < nkeys + 1; k += kThreads) a.start_loc[k] = 0;
        }
        return;
    }
    const int ne = c > 0 ? 1 : 0;
    const int ic = wave_inclusive_scan(c), ine = wave_inclusive_scan(ne);
    if (lane == kWave - 1) {
        s_wa[wave] = ic;
        s_wb[wave] = ine;
    }
    __syncthreads();
    int start = ic - c, slot = ine - ne, n_active = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int va = s_wa[w], vb = s_wb[w];
        start += w < wave ? va : 0;
        slot += w < wave ? vb : 0;
        n_active += vb;
    }
    if (tid < nkeys) s_base[tid] = start + before;
    if (g == 0) {
        if (tid == 0) {
            *a.no_lora = 0;
            *a.status = bad ? LORA_ERR_ID_RANGE : 0;
        }
        if (ne) {
            a.active_ids[slot] = tid - 1;
            a.counts[slot] = c;
            a.start_loc[slot + 1] = start + c;
        }
        for (int k = tid; k < nkeys; k += kThreads) {
            if (k >= n_active) {
                a.active_ids[k] = -1;
                a.counts[k] = 0;
            }
        }
        for (int k = tid; k < nkeys + 1; k += kThreads)
            if (k == 0 || k > n_active) a.start_loc[k] = 0;
    }
    __syncthreads();
    for (int t = c0 + tid; t < tend; t += kThreads) {
        const int v = t == c0 + tid ? v0 : packed[t];
        const int key = (int)((unsigned)v >> kRankBits), rank = v & kRankMask;
        const int pos = s_base[key] + rank;
        if ((unsigned)pos < (unsigned)n) a.sorted[pos] = t;
        a.mapping_copy[t] = key - 1;
    }
}

}  // namespace

// The single workgroup's ranking takes about (64-token steps per wave) x
// (key bits + 2) units of work: several workgroups pay for a second launch
// once that passes kMultiWork (about 4 us of ranking; measured crossover).
bool multi_prepare(int n, int max_loras) {
    const int nkeys = max_loras + 1;
    const int nbits = nkeys > 1 ? 32 - __builtin_clz((unsigned)(nkeys - 1)) : 0;
    const long steps = (n + kThreads - 1) / kThreads;
    return n >= kMultiMin && steps * (nbits + 2) >= kMultiWork;
}

int prepare_launches(int n, int max_loras) { return multi_prepare(n, max_loras) ? 2 : 1; }

// One sorting workgroup, plus workgroups that clear the fused call's area
// (about 4 16-byte stores per thread) when the batch can use it.
hipError_t launch_prepare(const PrepareArgs &a, int32_t *sk_counters, int sk_words, hipStream_t s) {
    if (!sk_counters) sk_words = 0;
    const long groups = (long)a.sync_tiles * kSyncGroups + a.acc_floats / 4 + sk_words / 4;
    long clear = (groups + 4L * kThreads - 1) / (4L * kThreads);
    if (clear > 64) clear = 64;
    if (multi_prepare(a.num_tokens, a.max_loras) && sk_counters) {
        // several sorting workgroups; scratch in the stream-K slot area
        int32_t *scratch = sk_counters + kSkCounterWords;
        int g = (a.num_tokens + kThreads - 1) / kThreads;
        if (g > kMultiMaxGroups) g = kMultiMaxGroups;
        const int chunk = (a.num_tokens + g - 1) / g;
        g = (a.num_tokens + chunk - 1) / chunk;
        hipLaunchKernelGGL(prepare_rank_kernel, dim3((unsigned)g), dim3(kThreads), 0, s, a, scratch, chunk);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(prepare_place_kernel, dim3((unsigned)(g + clear)), dim3(kThreads), 0, s, a, scratch, chunk, g,
                           sk_counters, sk_words);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)(1 + clear)), dim3(kThreads), 0, s, a, sk_counters, sk_words);
    return hipGetLastError();
}

}  // namespace lora
