// lora_prepare.hip -- per-batch LoRA kernel metadata on one workgroup.
//
// Computes what LoRAKernelMeta._reset + prepare_tensors compute ("lora_kernel_metadata"
// page): the all(-1) no-LoRA flag with its early exit, the mapping copy, the
// stable sort of token indices by id, the ascending distinct ids with their
// counts (torch.unique(sorted=True, return_counts=True)) and their running
// sums (torch.cumsum) shifted by one slot.  The sort is a counting sort over
// the <= 1024 keys (id + 1), so it is stable and bit-exact by construction:
//
//   pass 1: histogram of keys; each wave groups equal keys with one ballot
//           per key bit, and one lane per group adds the group size (LDS).
//   scan:   one thread per key; block-wide exclusive scans give each
//           non-empty key its slot and its first sorted position.
//   pass 2: tiles of 1024 tokens in order; a token's position is its key's
//           running cursor + the count of equal keys in earlier waves of the
//           tile (per-wave table in LDS) + its rank among equal keys of its
//           own wave (popcount of the match mask below its lane).
#include "lora_internal.h"

namespace lora {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxKeys = LORA_MAX_LORAS + 1;

// Block-wide exclusive scan of two values; returns the totals too.
__device__ __forceinline__ void block_scan2(int a, int b, int &ea, int &eb, int &ta, int &tb,
                                            int *s_wa, int *s_wb) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    int ia = wave_inclusive_scan(a);
    int ib = wave_inclusive_scan(b);
    if (lane == kWave - 1) {
        s_wa[wave] = ia;
        s_wb[wave] = ib;
    }
    __syncthreads();
    int pa = 0, pb = 0;
    ta = 0;
    tb = 0;
    for (int w = 0; w < kWaves; ++w) {
        int va = s_wa[w], vb = s_wb[w];
        if (w < wave) {
            pa += va;
            pb += vb;
        }
        ta += va;
        tb += vb;
    }
    ea = pa + ia - a;
    eb = pb + ib - b;
}

__global__ __launch_bounds__(kThreads) void prepare_kernel(PrepareArgs a) {
    __shared__ int s_cnt[kMaxKeys];
    __shared__ int s_cur[kMaxKeys];
    __shared__ uint16_t s_wt[kWaves][kMaxKeys];
    __shared__ int s_wa[kWaves], s_wb[kWaves];
    __shared__ int s_any, s_bad;

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int n = a.num_tokens;
    const int nkeys = a.max_loras + 1;
    const int nbits = 32 - __clz(nkeys - 1);   // keys 0 .. nkeys-1 fit in nbits

    for (int k = tid; k < nkeys; k += kThreads) s_cnt[k] = 0;
    for (int k = tid; k < kWaves * kMaxKeys; k += kThreads) (&s_wt[0][0])[k] = 0;
    if (tid == 0) {
        s_any = 0;
        s_bad = 0;
    }
    __syncthreads();

    // ---- pass 1: histogram, any-active, bad ids
    bool any = false, bad = false;
    for (int base = 0; base < n; base += kThreads) {
        const int t = base + tid;
        const bool valid = t < n;
        int id = valid ? a.mapping[t] : -1;
        if (id < -1 || id >= a.max_loras) {
            bad = true;
            id = -1;
        }
        const int key = id + 1;
        any |= valid && id != -1;
        const uint64_t m = match_key(key, valid, nbits);
        if (valid && (m & lanemask_lt()) == 0) atomicAdd(&s_cnt[key], __popcll(m));
    }
    if (ballot(any) && lane == 0) atomicOr(&s_any, 1);
    if (ballot(bad) && lane == 0) atomicOr(&s_bad, 1);
    __syncthreads();

    const bool no_lora = (s_any == 0);
    if (tid == 0) {
        *a.no_lora = no_lora ? 1 : 0;
        *a.status = s_bad ? LORA_ERR_ID_RANGE : 0;
    }
    if (no_lora) {
        // _reset values, then the pages' early return
        for (int k = tid; k < nkeys; k += kThreads) {
            a.active_ids[k] = -1;
            a.counts[k] = 0;
        }
        for (int k = tid; k < nkeys + 1; k += kThreads) a.start_loc[k] = 0;
        return;
    }

    // ---- scan over keys (nkeys <= kThreads: one key per thread)
    const int c = tid < nkeys ? s_cnt[tid] : 0;
    const int ne = c > 0 ? 1 : 0;
    int start, slot, total, n_active;
    block_scan2(c, ne, start, slot, total, n_active, s_wa, s_wb);
    if (ne) {
        a.active_ids[slot] = tid - 1;
        a.counts[slot] = c;
        a.start_loc[slot + 1] = start + c;
    }
    if (tid < nkeys) s_cur[tid] = start;
    for (int k = tid; k < nkeys; k += kThreads) {
        if (k >= n_active) {
            a.active_ids[k] = -1;
            a.counts[k] = 0;
        }
    }
    for (int k = tid; k < nkeys + 1; k += kThreads)
        if (k == 0 || k > n_active) a.start_loc[k] = 0;
    __syncthreads();

    // ---- pass 2: stable scatter, tile by tile
    for (int base = 0; base < n; base += kThreads) {
        const int t = base + tid;
        const bool valid = t < n;
        int id = valid ? a.mapping[t] : -1;
        if (id < -1 || id >= a.max_loras) id = -1;
        const int key = id + 1;
        const uint64_t m = match_key(key, valid, nbits);
        const bool leader = valid && (m & lanemask_lt()) == 0;
        const int rank = __popcll(m & lanemask_lt());
        if (leader) s_wt[wave][key] = (uint16_t)__popcll(m);
        __syncthreads();
        if (valid) {
            int pos = s_cur[key] + rank;
            for (int w = 0; w < wave; ++w) pos += s_wt[w][key];
            if ((unsigned)pos < (unsigned)n) a.sorted[pos] = t;
            a.mapping_copy[t] = id;
        }
        __syncthreads();
        if (leader) {
            atomicAdd(&s_cur[key], __popcll(m));
            s_wt[wave][key] = 0;
        }
        // the next tile's first barrier orders these updates before any read
    }
}

}  // namespace

hipError_t launch_prepare(const PrepareArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(prepare_kernel, dim3(1), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace lora
