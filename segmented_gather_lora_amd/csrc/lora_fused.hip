// lora_fused.hip -- lora_shrink followed by lora_expand in one launch, for
// batches of short segments (PunicaWrapperGPU.add_lora_linear on the
// "punica_gpu" page chains add_shrink into an fp32 buffer and add_expand of
// that buffer; decode batches give each LoRA a handful of tokens, where two
// launches and two metadata round trips cost more than the data).
//
// Work is cut into 16-token tiles of the segments, as in the two kernels.
// Each tile gets W workgroups (grid / tiles, or one workgroup walks several
// tiles when tiles outnumber the grid); workgroup idx of a tile
//   1. runs the tile's shrink parts idx, idx + W, ... (a part is a K chunk of
//      all S*r <= 64 weight rows; its partial sums are added into buf with
//      float atomics), marking each part taken (an exchange on its flag,
//      issued as the part starts and checked before its adds) and counting
//      it done;
//   2. takes the tile's 256-column expand blocks idx, idx + W, ..., issues
//      the first block's weight and y loads, waits until the done counter
//      shows every part, stages the tile's buffer rows of all slices in LDS
//      once, and runs its blocks.
// The wait cannot deadlock, whatever is resident: a waiter that sees no
// progress for a while (about 0.1 ms) takes every part whose flag is still
// clear and runs it itself, so it only ever waits for parts that a running
// workgroup has taken, and a part never waits.  An owner that finds its part
// taken skips the adds.  Expand blocks have no dependants.
//
// Ordering without cache maintenance: buf is only written here with
// device-scope atomic adds, which are performed at the device's coherence
// point; a part's writer waits until its adds have completed (vmcnt) before
// it counts the part; readers load buf with device-coherent loads after they
// see the count.  (A device-scope release / acquire fence would instead write
// back / invalidate the XCD's whole L2 at every part and every reader.)
//
// Counters (in the caller's metadata region, zeroed by prepare), per tile T
// in kFusedTileWords words of their own:
//   +kFusedPastWait   workgroups done with parts and waits;
//   +kFusedPartsDone  parts done (its own 128-byte line: it is polled);
//   +kFusedFlags + p  part p taken.
// The W-th workgroup done with parts and waits resets the tile's words, so a
// call leaves every counter at zero.
#include "lora_fused.h"

#include <stdlib.h>
#include <string.h>

namespace lora {

namespace {

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
__device__ int prepare_in_lds(const PrepareArgs &p, int tile_tokens, int *smem, int *s_scan, int *s_flag,
                              bool writer) {
    constexpr int kSteps = kPrepMaxTokens / (kThreads);   // 64-token steps per wave at most
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int n = p.num_tokens;
    const int nkeys = p.max_loras + 1;   // = slots
    const int nbits = 32 - __clz(nkeys - 1);
    int *pre = smem, *sid = pre + nkeys + 1, *sst = sid + nkeys, *scn = sst + nkeys;
    int *ssorted = scn + nkeys;
    int *cnt = ssorted + n;   // [wave][key]: running counts, then slice bases (wave-major: no bank conflicts)

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
        // only the wave's own steps: every workgroup of the launch reads
        // these few lines, and clamped loads past the batch would pile onto
        // the one holding its last id
        const int t = t0 + q * kWave + lane;
        ids[q] = 0;
        if (q < steps) ids[q] = p.mapping[t < n ? t : n - 1];   // uniform
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
        ranks[q] = cnt[wave * nkeys + key] + __popcll(m & lanemask_lt());
        if (leader) cnt[wave * nkeys + key] += __popcll(m);   // this wave's row only
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
            for (int w = 0; w < kWaves; ++w) c[i] += cnt[w * nkeys + k];
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
                const int v = cnt[w * nkeys + k];
                cnt[w * nkeys + k] = run;
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
            const int pos = cnt[wave * nkeys + keys[q]] + ranks[q];
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

// MT: 16-row tiles of weight rows (S*r <= 16*MT); KS: 32-wide K steps of the
// expand (rank <= 32*KS); PREP: the kernel also prepares the batch (the tile
// table comes from the mapping instead of the metadata).
template <int MT, int KS, bool ADD, bool PREP>
__global__ __launch_bounds__(kThreads) void fused_kernel(FusedArgs f) {
    constexpr int kRowK = 32 * KS;
    constexpr int kRowStride = kRowK + 8;
    constexpr int kMaxSlices = (16 * MT) / 8;   // S * r <= 16*MT with r >= 8
    extern __shared__ int smem[];
    __shared__ int s_wsum[kWaves];
    __shared__ int s_claim;
    __shared__ int s_tok[kTile];   // the tile's token indices, for the helper path
    __shared__ floatx4 red[(kWaves - 1) * MT * kWave];
    // buffer rows of the tile, every slice: [slice][token][k]
    __shared__ __attribute__((aligned(16))) uint16_t s_hi[kMaxSlices * kTile * kRowStride];
    __shared__ __attribute__((aligned(16))) uint16_t s_lo[kMaxSlices * kTile * kRowStride];

    prefetch_kernargs<FusedArgs>();
    const ShrinkArgs &a = f.s;
    const ExpandArgs &e = f.e;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int n16 = lane & 15, g = lane >> 4;
    const int rank = a.rank;

    const int nslots = a.meta.nslots;
    __shared__ int s_scan[3 * kWaves], s_flag[2];
    const int total = PREP ? prepare_in_lds(f.p, kTile, smem, s_scan, s_flag, blockIdx.x == 0)
                           : build_tile_table<kThreads>(a.meta, kTile, smem, s_wsum);
    if (total == 0) return;
    const int grid = gridDim.x, b = blockIdx.x;
    // this workgroup's tiles: one tile shared by W workgroups, or every grid-th tile alone
    const bool shared = grid >= total;
    const int first = shared ? b % total : b;
    const int step = shared ? total : grid;
    const int idx = shared ? b / total : 0;

    // A workgroup counts out of a tile (thread 0, `out` = the count before
    // its own) once it is done with the tile's parts, waits and reads of the
    // accumulation area, and acts on the result at the tile's end, so the
    // round trip overlaps its expand blocks.  The tile's last workgroup out
    // clears the tile's rows of that area (every add into them has completed:
    // each reader waited for all parts) and resets the tile's words, so the
    // call leaves both at zero.
    auto count_out = [&](int32_t *words) {
        return __hip_atomic_fetch_add(words + kFusedPastWait, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto finish_tile = [&](const TileRef &tr, int32_t *words, int W, int out) {
        if (tid == 0) s_claim = out == W - 1;
        __syncthreads();
        const bool last = s_claim;
        __syncthreads();
        if (!last) return;
        const int per_tok = rank / 4;   // 16-byte pieces per token row of a slice
        for (int x = tid; x < a.rows / 4 * kTile; x += kThreads) {
            const int prow = x / (a.rows / 4), rest = x % (a.rows / 4);
            const int si = rest / per_tok, piece = rest % per_tok;
            const int pp = tr.tile * kTile + prow;
            if (pp >= tr.seg_count) continue;
            const int tt = sorted_at(a.meta, smem, tr.seg_start + pp);
            if ((unsigned)tt >= (unsigned)a.num_tokens) continue;
            float *dst = f.acc + ((int64_t)si * a.num_tokens + tt) * rank + 4 * piece;
#pragma unroll
            for (int k = 0; k < 4; ++k) __hip_atomic_store(dst + k, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid == 0) reset_tile(words, a.k_splits);
    };

    for (int tile = first; tile < total; tile += step) {
        const int W = shared ? grid / total + (tile < grid % total ? 1 : 0) : 1;
        int32_t *const words = f.sync + kFusedTileWords * tile;
        int32_t *const parts_done = words + kFusedPartsDone;
        int32_t *const flags = words + kFusedFlags;
        const TileRef tr = lookup_tile(smem, nslots, tile);

        // One shrink part on the MFMA: K chunk `ks` of all weight rows for the
        // tile's tokens.  The owner takes the part's flag as it starts and
        // skips the adds if a waiter took it first.
        auto run_part = [&](int ks) {
            int got = 0;
            const int p = tr.tile * kTile + n16;
            bool tv = p < tr.seg_count;
            int tok = sorted_at(a.meta, smem, tr.seg_start + (tv ? p : tr.seg_count - 1));
            if ((unsigned)tok >= (unsigned)a.num_tokens) {
                tok = 0;
                tv = false;
            }
            const uint16_t *xrow = a.x + (int64_t)tok * a.ldx;
            const uint16_t *arow[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                int row = mt * 16 + n16;
                row = row < a.rows ? row : a.rows - 1;
                const int i = row / rank, j = row - i * rank;
                arow[mt] = select_slice(a.a, i) + ((int64_t)tr.lora_id * rank + j) * a.hidden;
            }
            const int kbeg = ks * a.k_chunk;
            const int kend = min(kbeg + a.k_chunk, a.hidden);
            const int nsteps = (kend - kbeg + 63) / 64;
            floatx4 acc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
            // K steps interleaved over the 4 waves, the next step in flight while
            // one is multiplied; loads are unconditional (past the end: the row
            // start, masked below)
            auto load = [&](int st, u32x4 (&av)[MT][2], u32x4 (&xv)[2]) {
                const int kk = kbeg + st * 64 + g * 16;
                const int o0 = kk + 8 <= kend ? kk : 0, o1 = kk + 16 <= kend ? kk + 8 : 0;
                xv[0] = ld16(xrow + o0);
                xv[1] = ld16(xrow + o1);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    av[mt][0] = ld16(arow[mt] + o0);
                    av[mt][1] = ld16(arow[mt] + o1);
                }
            };
            u32x4 av[MT][2], xv[2];
            load(min(wave, nsteps - 1), av, xv);
            // the flag exchange after the first loads: memory counters complete
            // in order, so the first step does not wait for its round trip
            if (tid == 0) got = __hip_atomic_exchange(&flags[ks], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int st = wave; st < nsteps; st += kWaves) {
                u32x4 an[MT][2], xn[2];
                load(min(st + kWaves, nsteps - 1), an, xn);
                const int kk = kbeg + st * 64 + g * 16;
                const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (kk + 8 * h + 8 > kend) {
                        xv[h] = z;
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) av[mt][h] = z;
                    }
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt] = mfma16x16x32(as_bf16x8(av[mt][h]), as_bf16x8(xv[h]), acc[mt]);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    xv[h] = xn[h];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) av[mt][h] = an[mt][h];
                }
            }
            if (wave > 0) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) red[((wave - 1) * MT + mt) * kWave + lane] = acc[mt];
            }
            __syncthreads();
            // wave 0 holds thread 0's exchange result in lane 0
            if (wave == 0 && __builtin_amdgcn_readfirstlane(got) == 0) {
#pragma unroll
                for (int w = 1; w < kWaves; ++w)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[mt] += red[((w - 1) * MT + mt) * kWave + lane];
                // D layout: lane holds rows 4g..4g+3 of m-tile mt for token column n16
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int row0 = mt * 16 + 4 * g;
                    if (!tv || row0 >= a.rows) continue;
                    const int i = row0 / rank, j = row0 - i * rank;
                    float *dst = f.acc + ((int64_t)i * a.num_tokens + tok) * rank + j;
                    const floatx4 v = acc[mt] * a.scale;
                    unsafeAtomicAdd(dst + 0, v[0]);
                    unsafeAtomicAdd(dst + 1, v[1]);
                    unsafeAtomicAdd(dst + 2, v[2]);
                    unsafeAtomicAdd(dst + 3, v[3]);
                }
                // this wave's additions have completed before the part is counted
                __builtin_amdgcn_s_waitcnt(kVmcntZero);
                asm volatile("" ::: "memory");
                if (lane == 0) __hip_atomic_fetch_add(parts_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();   // `red` is reused
        };

        // The same part for a waiter that took its flag (a rare path, kept
        // small so that it costs the main path no registers): one fp32 dot
        // product per (token, weight row) over the K chunk.
        auto help_part = [&](int ks) {
            const int kbeg = ks * a.k_chunk;
            const int kend = min(kbeg + a.k_chunk, a.hidden);   // kend - kbeg is a multiple of 8
            if (tid < kTile) {   // -1: no token at this tile row
                const int pp = tr.tile * kTile + tid;
                const int t = sorted_at(a.meta, smem, tr.seg_start + (pp < tr.seg_count ? pp : tr.seg_count - 1));
                s_tok[tid] = (pp < tr.seg_count && (unsigned)t < (unsigned)a.num_tokens) ? t : -1;
            }
            __syncthreads();
            for (int o = tid; o < kTile * a.rows; o += kThreads) {
                const int pr = o / a.rows, row = o - pr * a.rows;
                const int tok = s_tok[pr];
                if (tok < 0) continue;
                const int i = row / rank, j = row - i * rank;
                const uint16_t *xr = a.x + (int64_t)tok * a.ldx;
                const uint16_t *ar = select_slice(a.a, i) + ((int64_t)tr.lora_id * rank + j) * a.hidden;
                float sum = 0.f;
                for (int k = kbeg; k < kend; k += 8) {
                    const u32x4 xv = ld16(xr + k), av = ld16(ar + k);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        sum += bf16_bits_to_float(xv[c] & 0xffffu) * bf16_bits_to_float(av[c] & 0xffffu);
                        sum += bf16_bits_to_float(xv[c] >> 16) * bf16_bits_to_float(av[c] >> 16);
                    }
                }
                unsafeAtomicAdd(f.acc + ((int64_t)i * a.num_tokens + tok) * rank + j, sum * a.scale);
            }
            // every thread's additions have completed before the part is counted
            __builtin_amdgcn_s_waitcnt(kVmcntZero);
            asm volatile("" ::: "memory");
            __syncthreads();
            if (tid == 0) __hip_atomic_fetch_add(parts_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };

        // ---------------- 1. this workgroup's own shrink parts
        if (!f.owners_skip)
            for (int ks = idx; ks < a.k_splits; ks += W) run_part(ks);

        // ---------------- 2. expand blocks idx, idx + W, ... of the tile
        bool waited = false;
        int out = -1;   // thread 0: this workgroup's count-out result
        // this lane's y rows: tile rows 4g .. 4g + 3, the same for every block
        int ytok[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            int pp = tr.tile * kTile + 4 * g + r4;
            pp = pp < tr.seg_count ? pp : tr.seg_count - 1;
            const int tt = sorted_at(e.meta, smem, tr.seg_start + pp);
            ytok[r4] = (unsigned)tt < (unsigned)e.num_tokens ? tt : e.num_tokens - 1;
        }
        struct Block {
            int i, width, grp, ycol;
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
            bk.wslice = select_slice(e.b, i) + (int64_t)tr.lora_id * bk.width * rank;
            bk.bptr = select_slice(e.bias, i);
            bk.ycol = select_slice(e.col_off, i) + bk.grp;
            return bk;
        };
        // a block's weights, bias and y rows: they do not depend on buf
        u32x4 w[4][KS];
        u32x2 braw, yv[4];
        auto load_block = [&](const Block &bk) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const uint16_t *row = bk.wslice + (int64_t)(bk.grp + qq) * rank;
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    const int kk = k * 32 + 8 * g;
                    w[qq][k] = ld16(row + (kk < rank ? kk : 0));
                }
            }
            braw = bk.bptr ? *reinterpret_cast<const u32x2 *>(bk.bptr + (int64_t)tr.lora_id * bk.width + bk.grp)
                           : u32x2{0u, 0u};
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                yv[r4] = ADD ? *reinterpret_cast<const u32x2 *>(e.y + (int64_t)ytok[r4] * e.ldy + bk.ycol)
                             : u32x2{0u, 0u};
        };
        Block cur;
        if (idx < f.blocks) {
            cur = block_at(idx);
            load_block(cur);
        }
        for (int blk = idx; blk < f.blocks; blk += W) {
            const int i = cur.i;
            if (!waited) {   // uniform: the first block of this tile
                waited = true;
                // wait for every part; after help_after polls without them,
                // take and run every part still free, then wait for the rest
                for (int round = 0;; ++round) {
                    if (tid == 0) {
                        const int limit = round == 0 ? f.help_after : kSpinLimit;
                        int n = 0;
                        bool ok;
                        while (!(ok = __hip_atomic_load(parts_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                                      a.k_splits) && n < limit) {
                            ++n;
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
                    for (int ks = 0; ks < a.k_splits; ++ks) {
                        if (tid == 0) s_claim = __hip_atomic_exchange(&flags[ks], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        __syncthreads();
                        const int taken = s_claim;
                        __syncthreads();
                        if (!taken) help_part(ks);
                    }
                }
                // the tile's buffer rows of every slice (device-coherent loads), as bf16 hi / lo
                const int lanes_per_row = rank >> 2;
                const int per_slice = kTile * lanes_per_row;   // 16-byte pieces per slice
                for (int x = tid; x < e.num_slices * per_slice; x += kThreads) {
                    const int si = x / per_slice, rem = x % per_slice;
                    const int prow = rem / lanes_per_row, piece = rem % lanes_per_row;
                    int pp = tr.tile * kTile + prow;
                    pp = pp < tr.seg_count ? pp : tr.seg_count - 1;
                    int tt = sorted_at(e.meta, smem, tr.seg_start + pp);
                    const bool tok_ok = (unsigned)tt < (unsigned)e.num_tokens;
                    tt = tok_ok ? tt : e.num_tokens - 1;
                    const int64_t o_acc = ((int64_t)si * e.num_tokens + tt) * rank + 4 * piece;
                    floatx4 bv;
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        bv[k] = __hip_atomic_load(f.acc + o_acc + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    // the call's result in the caller's buffer (buf = shrink), written by
                    // one workgroup of the tile; rows past the segment repeat its last
                    // token and store the same values
                    if (idx == 0 && tok_ok) *reinterpret_cast<floatx4 *>(a.buf + o_acc) = bv;
                    uint32_t h[4], l[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        h[k] = float_to_bf16_bits(bv[k]);
                        l[k] = float_to_bf16_bits(bv[k] - bf16_bits_to_float(h[k]));
                    }
                    const int o = (si * kTile + prow) * kRowStride + 4 * piece;
                    *reinterpret_cast<u32x2 *>(&s_hi[o]) = u32x2{pack2(h[0], h[1]), pack2(h[2], h[3])};
                    *reinterpret_cast<u32x2 *>(&s_lo[o]) = u32x2{pack2(l[0], l[1]), pack2(l[2], l[3])};
                }
                if (rank < kRowK) {
                    for (int x = tid; x < e.num_slices * kTile * (kRowK - rank); x += kThreads) {
                        const int pr = x / (kRowK - rank), k = rank + x % (kRowK - rank);
                        s_hi[pr * kRowStride + k] = 0;
                        s_lo[pr * kRowStride + k] = 0;
                    }
                }
                __syncthreads();
                // done with parts, waits and reads of the accumulation area
                if (tid == 0) out = count_out(words);
            }

            u32x2 res[4];
            if (cur.has_cols) {
                const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    const bool kin = k * 32 + 8 * g < rank;
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) w[qq][k] = kin ? w[qq][k] : z4;
                }
                floatx4 acc[4];
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) acc[t4] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    const int off = (i * kTile + n16) * kRowStride + k * 32 + 8 * g;
                    const u32x4 ah = *reinterpret_cast<const u32x4 *>(&s_hi[off]);
                    const u32x4 al = *reinterpret_cast<const u32x4 *>(&s_lo[off]);
#pragma unroll
                    for (int t4 = 0; t4 < 4; ++t4) {
                        acc[t4] = mfma16x16x32(as_bf16x8(ah), as_bf16x8(w[t4][k]), acc[t4]);
                        acc[t4] = mfma16x16x32(as_bf16x8(al), as_bf16x8(w[t4][k]), acc[t4]);
                    }
                }
                float bias[4];
                bias[0] = bf16_bits_to_float(braw[0] & 0xffffu);
                bias[1] = bf16_bits_to_float(braw[0] >> 16);
                bias[2] = bf16_bits_to_float(braw[1] & 0xffffu);
                bias[3] = bf16_bits_to_float(braw[1] >> 16);
                // acc[t4][r4]: token row 4g + r4 of the tile, column grp + t4
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const u32x2 yy = yv[r4];
                    const float r0 = bf16_bits_to_float(yy[0] & 0xffffu) + (acc[0][r4] + bias[0]);
                    const float r1 = bf16_bits_to_float(yy[0] >> 16) + (acc[1][r4] + bias[1]);
                    const float r2 = bf16_bits_to_float(yy[1] & 0xffffu) + (acc[2][r4] + bias[2]);
                    const float r3 = bf16_bits_to_float(yy[1] >> 16) + (acc[3][r4] + bias[3]);
                    res[r4] = u32x2{pack2(float_to_bf16_bits(r0), float_to_bf16_bits(r1)),
                                    pack2(float_to_bf16_bits(r2), float_to_bf16_bits(r3))};
                }
            }
            // The next block's operands go out before this block's stores:
            // memory counters complete in order, so loads issued after the
            // stores would also wait for the stores to complete.
            const bool store = cur.has_cols;
            const int ycol = cur.ycol;
            if (blk + W < f.blocks) {
                cur = block_at(blk + W);
                load_block(cur);
            }
            if (store) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    *reinterpret_cast<u32x2 *>(e.y + (int64_t)ytok[r4] * e.ldy + ycol) = res[r4];
            }
        }
        // no expand block here: this workgroup is done with its parts, count it out
        if (!waited && tid == 0) out = count_out(words);
        finish_tile(tr, words, W, out);
        __syncthreads();   // the staged rows are rewritten for the next tile
    }
}

typedef void (*FusedFn)(FusedArgs);

template <int MT, bool PREP>
FusedFn pick_ks(int ks, bool add) {
    if (ks == 1) return add ? fused_kernel<MT, 1, true, PREP> : fused_kernel<MT, 1, false, PREP>;
    return add ? fused_kernel<MT, 2, true, PREP> : fused_kernel<MT, 2, false, PREP>;
}

template <bool PREP>
FusedFn pick(int mt, int ks, bool add) {
    switch (mt) {
        case 1: return pick_ks<1, PREP>(ks, add);
        case 2: return pick_ks<2, PREP>(ks, add);
        case 3: return pick_ks<3, PREP>(ks, add);
        default: return pick_ks<4, PREP>(ks, add);
    }
}

}  // namespace

// Range: expected tokens per segment below 24, S * rank <= 64, rank <= 64
// (and, with a prepare, at most kPrepMaxTokens tokens).  K is split into
// chunks of 64-multiples until about 256 shrink parts exist, as for the direct
// shrink kernel; the grid is what the device holds at once.
static hipError_t launch(const ShrinkArgs &sin, const ExpandArgs &ein, const PrepareArgs *prep,
                         const int32_t *mapping_copy, int max_loras, int32_t *sync, float *acc, float *slots,
                         int32_t *status, int help_after, int owners_skip, hipStream_t stream) {
    const int n = sin.num_tokens;
    const int nslots = sin.meta.nslots;
    const int segs = nslots < n ? nslots : n;
    if (!one_launch_range(n, nslots, sin.rows, sin.rank, prep != nullptr)) return hipErrorNotSupported;

    FusedArgs f;
    memset(&f, 0, sizeof f);
    f.s = sin;
    f.e = ein;
    if (prep) f.p = *prep;
    f.sync = sync;
    f.acc = acc;
    f.slots = slots;
    f.status = status;
    f.help_after = help_after;
    f.owners_skip = owners_skip;
    int blocks = 0;
    for (int i = 0; i < ein.num_slices; ++i) {
        f.block_begin[i] = blocks;
        blocks += (ein.width[i] + kBlockCols - 1) / kBlockCols;
    }
    for (int i = ein.num_slices; i <= LORA_MAX_SLICES; ++i) f.block_begin[i] = blocks;
    f.blocks = blocks;

    // batches with every LoRA id likely present: the LoRA-major kernel
    // (test and comparison knob LORA_FUSED_LAYOUT: "tile" keeps this kernel,
    // "lora" fails the launch when the LoRA-major kernel does not apply)
    {
        const char *layout = getenv("LORA_FUSED_LAYOUT");
        if (!layout || strcmp(layout, "tile") != 0) {
            FusedArgs g = f;
            if (!prep) {
                g.p.mapping = mapping_copy;
                g.p.num_tokens = n;
                g.p.max_loras = max_loras;
            }
            const hipError_t r = launch_lora_major(g, prep != nullptr, stream);
            if (r != hipErrorNotSupported) return r;
            if (layout && strcmp(layout, "lora") == 0) return hipErrorInvalidValue;
        }
    }

    const int max_ks = (sin.hidden + 255) / 256;
    const long busy = (n + kTile - 1) / kTile + (segs + 1) / 2;
    int ks = busy < 256 ? (int)((256 + busy - 1) / busy) : 1;
    if (ks > max_ks) ks = max_ks;
    if (ks > kFusedMaxParts) ks = kFusedMaxParts;
    if (ks < 1) ks = 1;
    int chunk = (sin.hidden + ks - 1) / ks;
    chunk = (chunk + 63) / 64 * 64;
    ks = (sin.hidden + chunk - 1) / chunk;
    f.s.k_splits = ks;
    f.s.k_chunk = chunk;
    f.s.row_blocks = 1;
    f.s.meta.lds_tokens = n <= kLdsTokensMax ? n : 0;
    if (prep) f.s.meta.lds_tokens = n;   // the kernel sorts into LDS itself
    f.e.meta.lds_tokens = f.s.meta.lds_tokens;

    const int mt = (sin.rows + 15) / 16;
    const int kse = (sin.rank + 31) / 32;
    const bool add = ein.add_inputs != 0;
    const FusedFn fn = prep ? pick<true>(mt, kse, add) : pick<false>(mt, kse, add);
    size_t lds = sizeof(int) * (size_t)(4 * nslots + 1 + f.s.meta.lds_tokens);
    if (prep) lds += sizeof(int) * (size_t)nslots * kWaves;   // the sort's per-wave counts
    // enough workgroups for every tile's parts and blocks, at most what is resident
    const long tiles_upper = (n + kTile - 1) / kTile + segs;
    long grid = resident_grid(reinterpret_cast<const void *>(fn), kThreads, lds);
    const long useful = tiles_upper * (blocks > ks ? blocks : ks);
    if (grid > useful) grid = useful;
    grid = grid / kNumXcd * kNumXcd;
    if (grid < kNumXcd) grid = kNumXcd;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kThreads), lds, stream, f);
    return hipGetLastError();
}

hipError_t launch_fused(const ShrinkArgs &sin, const ExpandArgs &ein, const int32_t *mapping_copy, int max_loras,
                        int32_t *sync, float *acc, float *slots, int32_t *status, int help_after, int owners_skip,
                        hipStream_t stream) {
    return launch(sin, ein, nullptr, mapping_copy, max_loras, sync, acc, slots, status, help_after, owners_skip,
                  stream);
}

hipError_t launch_prepare_fused(const PrepareArgs &prep, const ShrinkArgs &sin, const ExpandArgs &ein,
                                int32_t *sync, float *acc, float *slots, int32_t *status, int help_after,
                                int owners_skip, hipStream_t stream) {
    return launch(sin, ein, &prep, nullptr, prep.max_loras, sync, acc, slots, status, help_after, owners_skip,
                  stream);
}

}  // namespace lora
