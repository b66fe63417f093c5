// lora_decode.hip -- prepare + shrink + expand of a decode batch in one launch,
// with the work laid out by LoRA id rather than by sorted segment.
//
// The tile-major one-launch kernel can only start reading weights once the
// batch is sorted, because a workgroup learns which LoRA its tile holds from
// the sort.  Here workgroup L + max_loras * idx serves LoRA id L in role idx,
// so its weight addresses are known at entry: a shrink part requests its
// weights with its ids, an expander as soon as its ids are in.  It needs no
// sort: it picks out its own tokens with one ballot per 64 tokens, in batch
// order (the order the stable sort gives them within the segment).
//
// Roles of id L:
//   - idx < parts: shrink part idx -- K chunk idx of all S*r weight rows, for
//     every token of L (the chunk's weights stay in registers across the
//     16-token tiles); its partial sums are stored in part slot idx (plain
//     stores, no atomics: each slot has one writer) and the part is counted
//     done on L's counter words;
//   - idx >= parts: expand block idx - parts (and every (W - parts)-th after
//     it) -- waits until L's parts are all done, adds up each tile's rows of
//     the part slots in part order (so buf is deterministic), multiplies them
//     by the block's weights and adds the result into y; the expander of each
//     slice's first block writes the rows to buf, which the call writes as a
//     fresh buffer ("=").
// Counter words, the wait, the help path of a waiter that sees no progress
// and the reset by the last workgroup out are those of the tile-major kernel,
// with the words of id L in place of those of tile L.
//
// With the prepare in the launch (lora_prepare_shrink_expand) the ids are the
// raw mapping, and the metadata arrays (LoRAKernelMeta.prepare_tensors on the
// "lora_kernel_metadata" page), which nothing in this launch reads, are
// written piecewise by the first expander of every id: its slot and its
// stretch of the sorted indices, whose place follows from counting smaller
// keys and present keys with ballots and a presence bitmap in LDS.  Without
// it (lora_shrink_expand on a prepared batch) the ids are the prepared copy,
// gated by the no-LoRA flag, and the metadata is left alone.
//
// Weights of an id the batch does not use are read for nothing, so the
// launcher takes this kernel only for batches of at least 4 tokens per id
// (a uniform batch then leaves about 2% of the ids unused).
#include "lora_fused.h"

#include <stdlib.h>

namespace lora {
namespace {

constexpr int kFilterSteps = kPrepMaxTokens / kThreads;   // 64-token steps per wave
constexpr int kMaxChunk = 2 * kWaves * 64;                // K per part: two 64-wide steps per wave
constexpr int kKeyWords = (LORA_MAX_LORAS + 1 + 31) / 32;   // presence bits of keys 0..max_loras
constexpr int kRowsStride = 64 + 4;                         // fp32 per staged row (rank <= 64), padded
constexpr int kSlotElems = (kTile * 64 + kThreads - 1) / kThreads;   // tile elements per thread, at most
constexpr int kSlotBatch = 8;                               // part slots loaded per round trip

// The batch's ids, one round trip: wave w holds the contiguous run of steps*64
// tokens from t0 (so wave order is batch order), lane l token t0 + 64 q + l.
struct Ids {
    int v[kFilterSteps];
    int t0, steps;
};

__device__ __forceinline__ void load_ids(const int32_t *mapping, int n, Ids &ids) {
    ids.steps = (n + kThreads - 1) / kThreads;
    ids.t0 = wave_id() * ids.steps * kWave;
#pragma unroll
    for (int q = 0; q < kFilterSteps; ++q) {   // addresses clamped
        // only the wave's own steps: every workgroup of the launch reads
        // these few lines, and clamped loads past the batch would pile onto
        // the one holding its last id
        const int t = ids.t0 + q * kWave + lane_id();
        ids.v[q] = 0;
        if (q < ids.steps) ids.v[q] = mapping[t < n ? t : n - 1];   // uniform
    }
}

// Tokens whose id satisfies `pred`, counted (and, with a list, written to it
// in batch order).  Every thread of the workgroup calls it; the count is the
// same in all of them.
template <bool LIST, typename Pred>
__device__ __forceinline__ int pick_tokens(const Ids &ids, int n, Pred pred, int *list, int *s_wcnt) {
    const int lane = lane_id(), wave = wave_id();
    uint64_t m[kFilterSteps];
    int wc = 0;
#pragma unroll
    for (int q = 0; q < kFilterSteps; ++q) {
        const int t = ids.t0 + q * kWave + lane;
        m[q] = ballot(q < ids.steps && t < n && pred(ids.v[q]));
        wc += __popcll(m[q]);
    }
    if (lane == 0) s_wcnt[wave] = wc;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        base += v < wave ? s_wcnt[v] : 0;
        total += s_wcnt[v];
    }
    if (LIST) {
#pragma unroll
        for (int q = 0; q < kFilterSteps; ++q) {
            if ((m[q] >> lane) & 1) list[base + __popcll(m[q] & lanemask_lt())] = ids.t0 + q * kWave + lane;
            base += __popcll(m[q]);
        }
    }
    __syncthreads();
    return total;
}

// The metadata arrays of prepare_tensors ("lora_kernel_metadata" page),
// written piecewise instead of by one sorting workgroup.  A key is id + 1
// (ids outside [-1, max_loras) count as -1, key 0); slots hold the keys
// present in ascending order.  The first expander of id L writes L's slot
// (active id, count, end of its segment) and its tokens' stretch of the
// sorted indices, which starts after every token of a smaller key; the first
// expander of id 0 also writes what belongs to no id: the key-0 slot, the
// padding slots, start_loc[0], the no-LoRA flag, the status and the id copy.
__device__ __forceinline__ int key_of(int id, int ml) { return (id >= 0 && id < ml) ? id + 1 : 0; }

__device__ void write_meta(const PrepareArgs &p, const Ids &ids, int n, int L, int cnt, const int *list, int *list0,
                           int *s_wcnt, uint32_t *s_bits) {
    const int tid = threadIdx.x;
    const int ml = p.max_loras, nkeys = ml + 1;
    const int words = (nkeys + 31) / 32;
    for (int w = tid; w < words; w += kThreads) s_bits[w] = 0u;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kFilterSteps; ++q) {
        const int t = ids.t0 + q * kWave + lane_id();
        if (q < ids.steps && t < n) {
            const int k = key_of(ids.v[q], ml);
            atomicOr(&s_bits[k >> 5], 1u << (k & 31));
        }
    }
    __syncthreads();
    auto present_below = [&](int key) {   // keys present among 0 .. key-1
        int c = 0;
        for (int w = 0; w < (key >> 5); ++w) c += __popc(s_bits[w]);
        if (key & 31) c += __popc(s_bits[key >> 5] & ((1u << (key & 31)) - 1u));
        return c;
    };
    if (cnt > 0) {
        const int off = pick_tokens<false>(ids, n, [&](int id) { return key_of(id, ml) < L + 1; }, nullptr, s_wcnt);
        const int slot = present_below(L + 1);
        for (int j = tid; j < cnt; j += kThreads) p.sorted[off + j] = list[j];
        if (tid == 0) {
            p.active_ids[slot] = L;
            p.counts[slot] = cnt;
            p.start_loc[slot + 1] = off + cnt;
        }
    }
    if (L != 0) return;
    const int n_active = present_below(nkeys);
    const bool key0 = s_bits[0] & 1u;
    const bool no_lora = n_active - (key0 ? 1 : 0) == 0;
    const int bad = pick_tokens<false>(ids, n, [&](int id) { return id < -1 || id >= ml; }, nullptr, s_wcnt);
    if (tid == 0) {
        *p.no_lora = no_lora ? 1 : 0;
        *p.status = bad ? LORA_ERR_ID_RANGE : 0;
    }
    const int pad = no_lora ? 0 : n_active;
    for (int k = pad + tid; k < nkeys; k += kThreads) {
        p.active_ids[k] = -1;
        p.counts[k] = 0;
    }
    for (int k = tid; k <= nkeys; k += kThreads)
        if (no_lora || k == 0 || k > n_active) p.start_loc[k] = 0;
    if (no_lora) return;
    if (key0) {
        const int c0 = pick_tokens<true>(ids, n, [&](int id) { return key_of(id, ml) == 0; }, list0, s_wcnt);
        for (int j = tid; j < c0; j += kThreads) p.sorted[j] = list0[j];
        if (tid == 0) {
            p.active_ids[0] = -1;
            p.counts[0] = c0;
            p.start_loc[1] = c0;
        }
    }
#pragma unroll
    for (int q = 0; q < kFilterSteps; ++q) {
        const int t = ids.t0 + q * kWave + lane_id();
        if (q < ids.steps && t < n) p.mapping_copy[t] = key_of(ids.v[q], ml) - 1;
    }
}

// Four waves per SIMD (at most 128 registers) keep 1024 workgroups resident;
// the shapes whose registers do not fit that (rank above 32, more than 48
// weight rows) would spill and keep the default.
template <int MT, int KS>
constexpr int kLmWavesPerSimd = (KS == 1 && MT <= 3) ? 4 : 1;

// PREP: the launch also prepares the batch (f.p.mapping is the raw mapping and
// the metadata arrays are written); otherwise f.p.mapping is the prepared id
// copy and the metadata is left alone.
template <int MT, int KS, bool ADD, bool PREP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kLmWavesPerSimd<MT, KS>)))
void lora_major_kernel(FusedArgs f) {
    extern __shared__ int smem[];
    __shared__ int s_wcnt[kWaves];
    __shared__ int s_claim;
    __shared__ uint32_t s_bits[kKeyWords];
    __shared__ floatx4 red[kWaves * MT * kWave];
    __shared__ __attribute__((aligned(16))) float s_rows[kTile * kRowsStride];   // a tile's rows of one slice

    prefetch_kernargs<FusedArgs>();
    const ShrinkArgs &a = f.s;
    const ExpandArgs &e = f.e;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int n16 = lane & 15, g = lane >> 4;
    const int rank = a.rank;
    const int n = a.num_tokens;
    const int ml = f.p.max_loras;
    const int L = (int)blockIdx.x % ml, idx = (int)blockIdx.x / ml;
    const int W = (int)gridDim.x / ml;   // roles per id: parts, then expand blocks
    const int nparts = a.k_splits;
    int *const s_list = smem;         // this id's tokens
    int *const s_list0 = smem + n;    // key-0 tokens (metadata only)

    // Weights, x and y are touched once per launch: their loads (and the y
    // stores) are nontemporal, so the stream does not evict the ids, buffer
    // rows and counters that the launch reuses (measured 14.1 -> 13.3 us on
    // the decode shape).
    //
    // the ids first: memory counters complete in order, so the token filter
    // then waits for them only, not for the weights issued after them.  A
    // prepared no-LoRA batch keeps the previous batch's id copy (prepare
    // returns before copying), so without a prepare the flag decides.
    Ids ids;
    load_ids(f.p.mapping, n, ids);
    const int no_lora = PREP ? 0 : *a.meta.no_lora;
    auto mine = [&](int id) { return id == L && !no_lora; };

    int32_t *const words = f.sync + kFusedTileWords * L;
    int32_t *const parts_done = words + kFusedPartsDone;
    int32_t *const past_wait = words + kFusedPastWait;
    int32_t *const flags = words + kFusedFlags;

    // part slot p of this call: [p][S][N][r]
    const int nsl = a.rows / rank;
    auto slot_at = [&](int p, int i, int tok) { return f.slots + (((int64_t)p * nsl + i) * n + tok) * rank; };

    if (idx < nparts) {
        // ================ shrink part idx: K chunk idx of all weight rows of L
        const int kbeg = idx * a.k_chunk;
        const int kend = min(kbeg + a.k_chunk, a.hidden);
        const int nsteps = (kend - kbeg + 63) / 64;   // <= 2 * kWaves
        // this wave's two K steps (wave and wave + kWaves); a step past the
        // chunk, or an 8-wide group past its end, reads the row start and is
        // masked where it is multiplied
        u32x4 av[2][MT][2];
        {
            const uint16_t *arow[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                int row = mt * 16 + n16;
                row = row < a.rows ? row : a.rows - 1;
                const int i = row / rank, j = row - i * rank;
                arow[mt] = lane_slice_ptr(a.a, i) + ((int64_t)L * rank + j) * a.hidden;
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int kk = kbeg + (wave + kWaves * s2) * 64 + g * 16;
                const int o0 = kk + 8 <= kend ? kk : 0, o1 = kk + 16 <= kend ? kk + 8 : 0;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    av[s2][mt][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(arow[mt] + o0));
                    av[s2][mt][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(arow[mt] + o1));
                }
            }
        }
        const int cnt = pick_tokens<true>(ids, n, mine, s_list, s_wcnt);
        if (cnt == 0) return;   // the whole workgroup: no word of L is touched by anyone
        int got = 0;
        if (!f.owners_skip) {
            const int ntiles = (cnt + kTile - 1) / kTile;
            for (int t = 0; t < ntiles; ++t) {
                const int pidx = t * kTile + n16;
                const bool tv = pidx < cnt;
                const int tok = s_list[tv ? pidx : cnt - 1];
                const uint16_t *xrow = a.x + (int64_t)tok * a.ldx;
                u32x4 xv[2][2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int kk = kbeg + (wave + kWaves * s2) * 64 + g * 16;
                    const int o0 = kk + 8 <= kend ? kk : 0, o1 = kk + 16 <= kend ? kk + 8 : 0;
                    xv[s2][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xrow + o0));
                    xv[s2][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xrow + o1));
                }
                // the part's flag after the first loads, which then do not wait for it
                if (t == 0 && tid == 0)
                    got = __hip_atomic_exchange(&flags[idx], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                floatx4 acc[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
                const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int st = wave + kWaves * s2;
                    if (st >= nsteps) continue;   // uniform in the wave
                    const int kk = kbeg + st * 64 + g * 16;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const bool in = kk + 8 * h + 8 <= kend;
                        const u32x4 xh = in ? xv[s2][h] : z;
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            acc[mt] = mfma16x16x32(as_bf16x8(in ? av[s2][mt][h] : z), as_bf16x8(xh), acc[mt]);
                    }
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * kWave + lane] = acc[mt];
                if (t == 0 && tid == 0) s_claim = got;
                __syncthreads();
                // each thread sums one output element per m-tile over the 4 waves
                // and adds it into buf (D layout: lane l holds rows 4(l/16)..+3 of
                // its m-tile for token column l % 16)
                if (s_claim == 0) {
                    const int l = tid >> 2, c = tid & 3;
                    const int pr = t * kTile + (l & 15);
                    const int tk = s_list[pr < cnt ? pr : cnt - 1];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const float *rp = reinterpret_cast<const float *>(red) + ((size_t)mt * kWave + l) * 4 + c;
                        float v = 0.f;
#pragma unroll
                        for (int q = 0; q < kWaves; ++q) v += rp[(size_t)q * MT * kWave * 4];
                        const int row = mt * 16 + 4 * (l >> 4) + c;
                        if (pr < cnt && row < a.rows) {
                            const int i = row / rank, j = row - i * rank;
                            __hip_atomic_store(slot_at(idx, i, tk) + j, v * a.scale, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                }
                __syncthreads();   // `red` is reused
            }
            // every thread's additions have completed before the part is counted
            __builtin_amdgcn_s_waitcnt(kVmcntZero);
            asm volatile("" ::: "memory");
            __syncthreads();
            if (tid == 0 && got == 0) __hip_atomic_fetch_add(parts_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // done with L's words: the count has landed before this workgroup counts out
        if (tid == 0) {
            __builtin_amdgcn_s_waitcnt(kVmcntZero);
            asm volatile("" ::: "memory");
            const int d = __hip_atomic_fetch_add(past_wait, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (d == W - 1) reset_tile(words, nparts);
        }
        return;
    }

    // ================ expand blocks idx - nparts, + (W - nparts), ... of L
    const int e0 = idx - nparts, we = W - nparts;
    struct Block {
        int i, grp, ycol, width;
        bool has_cols;
        const uint16_t *wslice, *bptr;
    };
    auto block_at = [&](int blk) {
        Block bk;
        int i = 0;
#pragma unroll
        for (int s = 1; s < LORA_MAX_SLICES; ++s)
            if (s < e.num_slices && blk >= f.block_begin[s]) i = s;
        bk.i = i;
        bk.width = select_slice(e.width, i);
        const int c0 = (blk - select_slice(f.block_begin, i)) * kBlockCols + wave * kWaveCols;
        bk.has_cols = c0 < bk.width;
        bk.grp = clamp_group((bk.has_cols ? c0 : 0) + 4 * n16, bk.width);
        bk.wslice = select_slice(e.b, i) + (int64_t)L * bk.width * rank;
        bk.bptr = select_slice(e.bias, i);
        bk.ycol = select_slice(e.col_off, i) + bk.grp;
        return bk;
    };
    u32x4 w[4][KS];
    u32x2 braw;
    auto load_weights = [&](const Block &bk) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const uint16_t *row = bk.wslice + (int64_t)(bk.grp + qq) * rank;
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const int kk = k * 32 + 8 * g;
                w[qq][k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + (kk < rank ? kk : 0)));
            }
        }
        braw = bk.bptr ? *reinterpret_cast<const u32x2 *>(bk.bptr + (int64_t)L * bk.width + bk.grp)
                       : u32x2{0u, 0u};
    };
    // the weights are requested once the ids are in: loads return in order,
    // so weight loads issued first would hold up this compute unit's later
    // id loads (the shrink parts' among them); an id with no tokens then
    // reads none
    Block bk = block_at(e0);

    const int cnt = pick_tokens<true>(ids, n, mine, s_list, s_wcnt);
    if (cnt > 0) load_weights(bk);
    auto token_at = [&](int pidx) { return s_list[pidx < cnt ? pidx : cnt - 1]; };
    // y rows of tile `t` for the current block (no dependence on buf)
    u32x2 yv[4];
    int ytok[4];
    auto load_y = [&](int t) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            ytok[r4] = token_at(t * kTile + 4 * g + r4);
            yv[r4] = ADD ? __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(e.y + (int64_t)ytok[r4] * e.ldy + bk.ycol))
                         : u32x2{0u, 0u};
        }
    };
    if (cnt > 0) load_y(0);
    if (PREP && e0 == 0 && (cnt > 0 || L == 0)) write_meta(f.p, ids, n, L, cnt, s_list, s_list0, s_wcnt, s_bits);
    if (cnt == 0) return;   // the whole workgroup: no word of L is touched by anyone
    const int ntiles = (cnt + kTile - 1) / kTile;

    // Rows of tile t of slice i (16 tokens x rank fp32): each thread takes
    // up to kSlotElems (token, k) elements and adds up their part slots in
    // part order; the loads of up to kSlotBatch parts are issued before the
    // first add (indices past the last part re-read the last part's slot and
    // add zero).
    auto sum_slots = [&](int i, int t, bool writer) {
        __syncthreads();   // the previous tile's rows have been read
        const int elems = kTile * rank;
#pragma unroll
        for (int q = 0; q < kSlotElems; ++q) {
            const int e = tid + q * kThreads;
            if (e < elems) {
                const int row = e / rank, j = e - row * rank;
                const int pr = t * kTile + row;
                const int tk = token_at(pr);
                float v = 0.f;
                for (int p0 = 0; p0 < nparts; p0 += kSlotBatch) {   // one round for up to 8 parts
                    float vals[kSlotBatch];
#pragma unroll
                    for (int p = 0; p < kSlotBatch; ++p) {
                        const int pp = p0 + p < nparts ? p0 + p : nparts - 1;
                        vals[p] = __hip_atomic_load(slot_at(pp, i, tk) + j, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
                    }
#pragma unroll
                    for (int p = 0; p < kSlotBatch; ++p) v += p0 + p < nparts ? vals[p] : 0.f;
                }
                s_rows[row * kRowsStride + j] = v;
                if (writer && pr < cnt) a.buf[((int64_t)i * n + tk) * rank + j] = v;
            }
        }
        __syncthreads();
    };

    // A waiter's copy of part `ks` (rare; kept small so that it costs the main
    // path no registers): one fp32 dot product per (token, weight row).
    auto help_part = [&](int ks) {
        const int hb = ks * a.k_chunk;
        const int he = min(hb + a.k_chunk, a.hidden);   // he - hb is a multiple of 8
        for (int o = tid; o < cnt * a.rows; o += kThreads) {
            const int pr = o / a.rows, row = o - pr * a.rows;
            const int tok = s_list[pr];
            const int i = row / rank, j = row - i * rank;
            const uint16_t *xr = a.x + (int64_t)tok * a.ldx;
            const uint16_t *ar = lane_slice_ptr(a.a, i) + ((int64_t)L * rank + j) * a.hidden;
            float sum = 0.f;
            for (int k = hb; k < he; k += 8) {
                const u32x4 xq = ld16(xr + k), aq = ld16(ar + k);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    sum += bf16_bits_to_float(xq[c] & 0xffffu) * bf16_bits_to_float(aq[c] & 0xffffu);
                    sum += bf16_bits_to_float(xq[c] >> 16) * bf16_bits_to_float(aq[c] >> 16);
                }
            }
            __hip_atomic_store(slot_at(ks, i, tok) + j, sum * a.scale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // every thread's additions have completed before the part is counted
        __builtin_amdgcn_s_waitcnt(kVmcntZero);
        asm volatile("" ::: "memory");
        __syncthreads();
        if (tid == 0) __hip_atomic_fetch_add(parts_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    // wait for every part of L; after help_after polls without them, take and
    // run every part still free, then wait for the rest
    for (int round = 0;; ++round) {
        if (tid == 0) {
            const int limit = round == 0 ? f.help_after : kSpinLimit;
            int polls = 0;
            bool ok;
            while (!(ok = __hip_atomic_load(parts_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= nparts) &&
                   polls < limit) {
                ++polls;
                __builtin_amdgcn_s_sleep(8);
            }
            s_claim = ok ? 1 : (round == 0 ? 2 : 3);
            if (s_claim == 3)
                __hip_atomic_store(f.status, (int)LORA_ERR_SYNC, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        const int verdict = s_claim;
        __syncthreads();
        if (verdict != 2) break;
        for (int ks = 0; ks < nparts; ++ks) {
            if (tid == 0) s_claim = __hip_atomic_exchange(&flags[ks], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const int taken = s_claim;
            __syncthreads();
            if (!taken) help_part(ks);
        }
    }
    // done with L's words (every count it waited for has landed): count out
    // now, act on the result at the end so the round trip overlaps the work
    int out = 0;
    if (tid == 0) out = __hip_atomic_fetch_add(past_wait, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    for (int blk = e0; blk < f.blocks; blk += we) {
        if (blk != e0) {
            bk = block_at(blk);
            load_weights(bk);
        }
        const u32x4 z4 = {0u, 0u, 0u, 0u};
        u32x4 wm[4][KS];
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const bool kin = k * 32 + 8 * g < rank;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) wm[qq][k] = kin ? w[qq][k] : z4;
        }
        const float bias0 = bf16_bits_to_float(braw[0] & 0xffffu), bias1 = bf16_bits_to_float(braw[0] >> 16);
        const float bias2 = bf16_bits_to_float(braw[1] & 0xffffu), bias3 = bf16_bits_to_float(braw[1] >> 16);
        for (int t = 0; t < ntiles; ++t) {
            if (blk != e0 || t != 0) load_y(t);
            // the tile's rows of this block's slice: the sum of the parts' slots in
            // part order (so buf is deterministic), gathered once per workgroup
            // with device-coherent loads (other workgroups stored them) and
            // shared through LDS; the expander of the slice's first block also
            // writes them to the caller's buffer (buf = shrink)
            sum_slots(bk.i, t, blk == f.block_begin[bk.i]);
            u32x4 ah[KS], al[KS];
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const int kk = k * 32 + 8 * g;
                float v[8];
                if (kk < rank) {
                    const floatx4 lo4 = *reinterpret_cast<const floatx4 *>(&s_rows[n16 * kRowsStride + kk]);
                    const floatx4 hi4 = *reinterpret_cast<const floatx4 *>(&s_rows[n16 * kRowsStride + kk + 4]);
                    v[0] = lo4[0]; v[1] = lo4[1]; v[2] = lo4[2]; v[3] = lo4[3];
                    v[4] = hi4[0]; v[5] = hi4[1]; v[6] = hi4[2]; v[7] = hi4[3];
                } else {
#pragma unroll
                    for (int c = 0; c < 8; ++c) v[c] = 0.f;
                }
                uint32_t h[8], l[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    h[c] = float_to_bf16_bits(v[c]);
                    l[c] = float_to_bf16_bits(v[c] - bf16_bits_to_float(h[c]));
                }
                ah[k] = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
                al[k] = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
            }
            if (!bk.has_cols) continue;   // uniform in the wave
            floatx4 acc[4];
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) acc[t4] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KS; ++k)
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) {
                    acc[t4] = mfma16x16x32(as_bf16x8(ah[k]), as_bf16x8(wm[t4][k]), acc[t4]);
                    acc[t4] = mfma16x16x32(as_bf16x8(al[k]), as_bf16x8(wm[t4][k]), acc[t4]);
                }
            // acc[t4][r4]: token row 4g + r4 of the tile, column grp + t4
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const u32x2 yy = yv[r4];
                const float r0 = bf16_bits_to_float(yy[0] & 0xffffu) + (acc[0][r4] + bias0);
                const float r1 = bf16_bits_to_float(yy[0] >> 16) + (acc[1][r4] + bias1);
                const float r2 = bf16_bits_to_float(yy[1] & 0xffffu) + (acc[2][r4] + bias2);
                const float r3 = bf16_bits_to_float(yy[1] >> 16) + (acc[3][r4] + bias3);
                __builtin_nontemporal_store(u32x2{pack2(float_to_bf16_bits(r0), float_to_bf16_bits(r1)),
                                                  pack2(float_to_bf16_bits(r2), float_to_bf16_bits(r3))},
                                            reinterpret_cast<u32x2 *>(e.y + (int64_t)ytok[r4] * e.ldy + bk.ycol));
            }
        }
    }
    // the last of L's workgroups out resets L's words
    if (tid == 0 && out == W - 1) reset_tile(words, nparts);
}

typedef void (*LoraMajorFn)(FusedArgs);

template <int MT, bool PREP>
LoraMajorFn pick_ks(int ks, bool add) {
    if (ks == 1) return add ? lora_major_kernel<MT, 1, true, PREP> : lora_major_kernel<MT, 1, false, PREP>;
    return add ? lora_major_kernel<MT, 2, true, PREP> : lora_major_kernel<MT, 2, false, PREP>;
}

template <bool PREP>
LoraMajorFn pick(int mt, int ks, bool add) {
    switch (mt) {
        case 1: return pick_ks<1, PREP>(ks, add);
        case 2: return pick_ks<2, PREP>(ks, add);
        case 3: return pick_ks<3, PREP>(ks, add);
        default: return pick_ks<4, PREP>(ks, add);
    }
}

}  // namespace

// Range (beyond the tile-major kernel's, which the caller has checked): at
// least 4 tokens per LoRA id, at most kPrepMaxTokens tokens, K split into
// parts of at most kMaxChunk (a part's weights stay in registers), and every
// role of every id resident at once (max_loras * (parts + blocks) workgroups).
// The counter words of id L are those of tile L, which the metadata region
// holds for every id when the batch has more tokens than ids.
hipError_t launch_lora_major(const FusedArgs &fin, bool prepare, hipStream_t stream) {
    const int n = fin.s.num_tokens;
    const int max_loras = fin.p.max_loras;
    if (n > kPrepMaxTokens || n < 4 * max_loras || n <= max_loras) return hipErrorNotSupported;
    if (fin.s.rows > 64 || fin.s.rank > 64) return hipErrorNotSupported;
    FusedArgs f = fin;
    int parts = (fin.s.hidden + kMaxChunk - 1) / kMaxChunk;
    if (const char *v = getenv("LORA_LM_PARTS")) {   // tuning: more, shorter parts
        const int want = atoi(v);
        if (want > parts) parts = want;
    }
    if (parts > kLmMaxParts) return hipErrorNotSupported;   // the part slots hold this many
    int chunk = (fin.s.hidden + parts - 1) / parts;
    chunk = (chunk + 63) / 64 * 64;
    parts = (fin.s.hidden + chunk - 1) / chunk;
    f.s.k_splits = parts;
    f.s.k_chunk = chunk;

    const int mt = (fin.s.rows + 15) / 16;
    const int kse = (fin.s.rank + 31) / 32;
    const bool add = fin.e.add_inputs != 0;
    const LoraMajorFn fn = prepare ? pick<true>(mt, kse, add) : pick<false>(mt, kse, add);
    const size_t lds = sizeof(int) * (size_t)((prepare ? 2 : 1) * n);   // the id's tokens (, the key-0 tokens)
    long expanders = f.blocks;   // one expand block per workgroup
    if (const char *v = getenv("LORA_LM_EXPANDERS")) {   // tuning: expanders walking several blocks
        const int want = atoi(v);
        if (want > 0 && want < expanders) expanders = want;
    }
    const long grid = (long)max_loras * (parts + expanders);
    if (grid > resident_grid(reinterpret_cast<const void *>(fn), kThreads, lds)) return hipErrorNotSupported;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kThreads), lds, stream, f);
    return hipGetLastError();
}

}  // namespace lora
