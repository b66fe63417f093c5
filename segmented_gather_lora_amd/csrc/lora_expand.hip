// lora_expand.hip -- y[t, off_i + c] = bf16((add_inputs ? y : 0) + buf[i][t] @ B_i[id_t][c]
// + bias_i[id_t][c]) for tokens grouped by LoRA id (PunicaWrapperGPU.add_expand
// on the "punica_gpu" page; per-slice column offsets as in
// PunicaWrapperTPU.add_expand and the bias rule of PunicaWrapperTPU._apply_bias
// on the "punica_tpu" page, folded into one pass with a single rounding).
//
// Per segment and slice this is C[tokens][cols] = buf_seg[tokens][r] * B_id[cols][r]^T
// with K = r (8..128), on the bf16 MFMA (v_mfma_f32_16x16x32_bf16) with the
// tokens on the M side and the output columns on the N side:
//   - a work unit is (TT tiles of 16 tokens of one segment) x (256 columns of
//     one slice); each of the 4 waves owns 64 of the columns and keeps their
//     weights (64 x r bf16) in registers for the unit;
//   - the unit's fp32 buffer rows are read once per workgroup with coalesced
//     loads, split into bf16 hi = rne(v) and lo = rne(v - hi) and staged in
//     LDS; every wave reads its MFMA operands from there, and both parts go
//     through the MFMA, which keeps ~16 mantissa bits of the fp32 value;
//   - the 64 columns of a wave are spread over four 16-column MFMA tiles so
//     that lane n holds columns 4n..4n+3 of 4 tokens: every y load and store
//     instruction moves 128 contiguous bytes of 4 token rows;
//   - y is read and written once, with nontemporal loads and stores that keep
//     its stream from evicting the weight blocks that other token tiles of the
//     segment re-read (5-10 % on the prefill, Zipf, large and embedding shapes;
//     the weights themselves stay cached).
// Work units follow a canonical tile-major order cut into one chunk per XCD,
// walked by a persistent grid.
//
// No load or store is conditional.  A lane whose token is past the end of
// the segment works on the segment's last token, and a 4-column group past
// the end of the slice works on the slice's last 4 columns: it computes
// exactly the owner's values and stores them to the same address, so the
// duplicate store is harmless.  Tokens with id -1 own no tile and are never
// touched.
#include "lora_internal.h"

namespace lora {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kWaveCols = 64;
constexpr int kBlockCols = kWaves * kWaveCols;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return lo16 | (hi16 << 16); }

// Last valid 4-column group for a group starting at c (c % 4 == 0).
__device__ __forceinline__ int clamp_group(int c, int width) { return c < width ? c : width - 4; }

template <int KS, int TT, bool ADD, bool EARLY>
__global__ __launch_bounds__(kThreads) void expand_kernel(ExpandArgs a) {
    prefetch_kernargs<ExpandArgs>();
    constexpr int kUnitTokens = 16 * TT;
    constexpr bool kPipe = TT <= 2;             // next block's loads ahead of this block's stores
    constexpr int kRowK = 32 * KS;              // bf16 per staged row (rank padded to 32)
    constexpr int kRowStride = kRowK + 8;       // +16 bytes: rows start on different banks
    extern __shared__ int smem[];
    __shared__ int s_wsum[kWaves];
    __shared__ __attribute__((aligned(16))) uint16_t s_hi[kUnitTokens * kRowStride];
    __shared__ __attribute__((aligned(16))) uint16_t s_lo[kUnitTokens * kRowStride];

    const int nslots = a.meta.nslots;
    const int total = build_tile_table<kThreads>(a.meta, kUnitTokens, smem, s_wsum);

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int n16 = lane & 15, g = lane >> 4;
    const int rank = a.rank;
    const u32x4 z4 = {0u, 0u, 0u, 0u};

    // One piece of work: token tile `tr`, column blocks [cb0, cb0 + ncb) of slice i.
    auto run_piece = [&](const TileRef &tr, int i, int cb0, int ncb) {
        const int width = select_slice(a.width, i);
        const int pbase = tr.tile * kUnitTokens;
        const float *bufs = a.buf + (int64_t)i * a.num_tokens * rank;

        // ---- coalesced fp32 buffer loads for the unit's rows: rank/4 lanes per row
        const int lanes_per_row = rank >> 2;                 // 16-byte pieces per row
        const int rows_per_pass = kThreads / lanes_per_row;
        // rank <= 32*KS, so a pass covers at least kThreads / (8*KS) rows
        constexpr int kMinRowsPerPass = kThreads / (8 * KS);
        constexpr int kPasses = (kUnitTokens + kMinRowsPerPass - 1) / kMinRowsPerPass;
        floatx4 bvals[kPasses];
        int brow_p[kPasses];
#pragma unroll
        for (int ps = 0; ps < kPasses; ++ps) {
            int p = ps * rows_per_pass + tid / lanes_per_row;
            const int piece = tid % lanes_per_row;
            brow_p[ps] = p;
            p = p < kUnitTokens ? p : kUnitTokens - 1;
            int pp = pbase + p;
            pp = pp < tr.seg_count ? pp : tr.seg_count - 1;
            int t = sorted_at(a.meta, smem, tr.seg_start + pp);
            t = (unsigned)t < (unsigned)a.num_tokens ? t : a.num_tokens - 1;
            bvals[ps] = *reinterpret_cast<const floatx4 *>(bufs + (int64_t)t * rank + 4 * piece);
        }
        // ---- y rows of this lane: tile q, row 4g + e of the tile -> token index
        int ytok[TT][4];
#pragma unroll
        for (int q = 0; q < TT; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int pp = pbase + q * 16 + 4 * g + e;
                pp = pp < tr.seg_count ? pp : tr.seg_count - 1;
                const int t = sorted_at(a.meta, smem, tr.seg_start + pp);
                ytok[q][e] = (unsigned)t < (unsigned)a.num_tokens ? t : a.num_tokens - 1;
            }

        // ---- operands of one column block for this wave: weights (B operand of
        // n-tile q: lane (n16, g) -> column 4*n16 + q), bias and y rows.  With
        // EARLY (runs of one block) they are loaded before the buffer rows are
        // staged, in the same round trip; longer runs load them block by block
        // (fewer registers live across the staging).
        const uint16_t *wslice = select_slice(a.b, i) + (int64_t)tr.lora_id * width * rank;
        const uint16_t *bptr = select_slice(a.bias, i);
        const int slice_col = select_slice(a.col_off, i);
        u32x4 w[4][KS];
        u32x2 braw, yv[TT][4];
        // address of y[row][col], recomputed at every use: the opaque copy of
        // the row keeps the compiler from holding 16 64-bit row addresses
        // live across the column-block loop
        auto y_at = [&](int row, int col) {
            asm volatile("" : "+v"(row));
            return a.y + ((int64_t)row * a.ldy + col);
        };
        auto load_block = [&](int grp) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint16_t *row = wslice + (int64_t)(grp + q) * rank;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int k = ks * 32 + 8 * g;
                    w[q][ks] = *reinterpret_cast<const u32x4 *>(row + (k < rank ? k : 0));
                }
            }
            braw = bptr ? *reinterpret_cast<const u32x2 *>(bptr + (int64_t)tr.lora_id * width + grp) : u32x2{0u, 0u};
            const int ycol = slice_col + grp;
#pragma unroll
            for (int q = 0; q < TT; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    yv[q][e] = ADD ? __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(y_at(ytok[q][e], ycol)))
                                   : u32x2{0u, 0u};
        };
        // first of this lane's 4 columns in block cb0 + c (clamped to the slice)
        auto group_of = [&](int c) {
            return clamp_group((cb0 + c) * kBlockCols + wave * kWaveCols + 4 * n16, width);
        };
        if (EARLY) load_block(group_of(0));

        // ---- stage the buffer rows in LDS as bf16 hi / lo (rank tail stays zero),
        // once for all column blocks of the run
#pragma unroll
        for (int ps = 0; ps < kPasses; ++ps) {
            const int p = brow_p[ps];
            const int piece = tid % lanes_per_row;
            if (p < kUnitTokens) {
                uint32_t h[4], l[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = float_to_bf16_bits(bvals[ps][e]);
                    l[e] = float_to_bf16_bits(bvals[ps][e] - bf16_bits_to_float(h[e]));
                }
                *reinterpret_cast<u32x2 *>(&s_hi[p * kRowStride + 4 * piece]) = u32x2{pack2(h[0], h[1]), pack2(h[2], h[3])};
                *reinterpret_cast<u32x2 *>(&s_lo[p * kRowStride + 4 * piece]) = u32x2{pack2(l[0], l[1]), pack2(l[2], l[3])};
            }
        }
        if (rank < kRowK) {   // zero the rank padding once per unit
            for (int x = tid; x < kUnitTokens * (kRowK - rank); x += kThreads) {
                const int p = x / (kRowK - rank), k = rank + x % (kRowK - rank);
                s_hi[p * kRowStride + k] = 0;
                s_lo[p * kRowStride + k] = 0;
            }
        }
        __syncthreads();

        bool loaded = EARLY;   // this block's operands are in (EARLY, or fetched with the previous block)
        for (int c = 0; c < ncb; ++c) {
            // a wave past the slice's last column stays past it for the rest of the run
            if ((cb0 + c) * kBlockCols + wave * kWaveCols >= width) break;
            const int grp = group_of(c);
            if (!loaded) load_block(grp);

            // K positions >= rank: zero the weights (no NaN from stale data)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bool kin = ks * 32 + 8 * g < rank;
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q][ks] = kin ? w[q][ks] : z4;
            }
            float bias[4];
            bias[0] = bf16_bits_to_float(braw[0] & 0xffffu);
            bias[1] = bf16_bits_to_float(braw[0] >> 16);
            bias[2] = bf16_bits_to_float(braw[1] & 0xffffu);
            bias[3] = bf16_bits_to_float(braw[1] >> 16);
            const int ycol = slice_col + grp;

            u32x2 out[kPipe ? TT : 1][4];   // kPipe: the block's results, stored after the next block's loads
#pragma unroll
            for (int q = 0; q < TT; ++q) {
                floatx4 acc[4];
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) acc[t4] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int off = (q * 16 + n16) * kRowStride + ks * 32 + 8 * g;
                    const u32x4 ah = *reinterpret_cast<const u32x4 *>(&s_hi[off]);
                    const u32x4 al = *reinterpret_cast<const u32x4 *>(&s_lo[off]);
#pragma unroll
                    for (int t4 = 0; t4 < 4; ++t4) {
                        acc[t4] = mfma16x16x32(as_bf16x8(ah), as_bf16x8(w[t4][ks]), acc[t4]);
                        acc[t4] = mfma16x16x32(as_bf16x8(al), as_bf16x8(w[t4][ks]), acc[t4]);
                    }
                }
                // acc[t4][e]: token row 4g + e of tile q, column grp + t4
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const u32x2 yy = yv[q][e];
                    const float r0 = bf16_bits_to_float(yy[0] & 0xffffu) + (acc[0][e] + bias[0]);
                    const float r1 = bf16_bits_to_float(yy[0] >> 16) + (acc[1][e] + bias[1]);
                    const float r2 = bf16_bits_to_float(yy[1] & 0xffffu) + (acc[2][e] + bias[2]);
                    const float r3 = bf16_bits_to_float(yy[1] >> 16) + (acc[3][e] + bias[3]);
                    const u32x2 o = {pack2(float_to_bf16_bits(r0), float_to_bf16_bits(r1)),
                                     pack2(float_to_bf16_bits(r2), float_to_bf16_bits(r3))};
                    if constexpr (kPipe)
                        out[q][e] = o;
                    else
                        __builtin_nontemporal_store(o, reinterpret_cast<u32x2 *>(y_at(ytok[q][e], ycol)));
                }
            }
            // With tiles of at most 32 tokens, the next block's weights and y
            // rows go out before this block's stores: memory counters complete
            // in order, so loads issued after the stores would also wait for
            // the stores to complete.  (For 64-token tiles the registers this
            // holds cost more occupancy than the overlap gains.)
            if constexpr (kPipe) {
                loaded = c + 1 < ncb && (cb0 + c + 1) * kBlockCols + wave * kWaveCols < width;
                if (loaded) load_block(group_of(c + 1));
#pragma unroll
                for (int q = 0; q < TT; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_nontemporal_store(out[q][e], reinterpret_cast<u32x2 *>(y_at(ytok[q][e], ycol)));
            } else {
                loaded = false;
            }
        }
        __syncthreads();   // the staged rows are rewritten by the next piece
    };
    // the slice of (single-block or run) index b of a tile
    auto slice_of = [&](int b) {
        int i = 0;
#pragma unroll
        for (int s = 1; s < LORA_MAX_SLICES; ++s)
            if (s < a.num_slices && b >= a.run_begin[s]) i = s;
        return i;
    };

    // The pieces of this workgroup.  With a.share: equal shares of the (tile,
    // column block) list (runs are single blocks then), in XCD order, cut
    // anywhere, since column blocks need no combining, so every workgroup
    // gets the same number of blocks to within one.  Otherwise units of
    // a.run_blocks blocks of one slice, walked in one chunk per XCD.
    const long W = (long)total * a.runs;
    const int G = gridDim.x;
    const int share_id = (int)(blockIdx.x % kNumXcd) * (G / kNumXcd) + (int)(blockIdx.x / kNumXcd);
    const long end = a.share ? W * (share_id + 1) / G : 0;
    long cur = a.share ? W * share_id / G : 0;
    const UnitWalker walk(a.share ? 0 : (int)W);
    for (int jj = walk.first;;) {
        int t, i, cb0, ncb;
        if (a.share) {
            if (cur >= end) break;
            t = (int)(cur / a.runs);
            const int b = (int)(cur - (long)t * a.runs);
            i = slice_of(b);
            cb0 = b - select_slice(a.run_begin, i);
            const int blocks_i = (select_slice(a.width, i) + kBlockCols - 1) / kBlockCols;
            ncb = (int)min((long)(blocks_i - cb0), end - cur);
            cur += ncb;
        } else {
            const int u = walk.unit(jj);
            if (u < 0) break;
            jj += walk.stride;
            t = u / a.runs;
            const int run = u % a.runs;
            i = slice_of(run);
            cb0 = (run - select_slice(a.run_begin, i)) * a.run_blocks;
            const int blocks_i = (select_slice(a.width, i) + kBlockCols - 1) / kBlockCols;
            ncb = min(a.run_blocks, blocks_i - cb0);
        }
        run_piece(lookup_tile(smem, nslots, t), i, cb0, ncb);
    }
}

typedef void (*ExpandFn)(ExpandArgs);

template <int KS, int TT>
ExpandFn pick_add(bool add, bool early) {
    if (early) return add ? expand_kernel<KS, TT, true, true> : expand_kernel<KS, TT, false, true>;
    return add ? expand_kernel<KS, TT, true, false> : expand_kernel<KS, TT, false, false>;
}

template <int KS>
ExpandFn pick_tt(int tt, bool add, bool early) {
    switch (tt) {
        case 1: return pick_add<KS, 1>(add, early);
        case 2: return pick_add<KS, 2>(add, early);
        default: return pick_add<KS, 4>(add, early);
    }
}

ExpandFn pick(int ks, int tt, bool add, bool early) {
    switch (ks) {
        case 1: return pick_tt<1>(tt, add, early);
        case 2: return pick_tt<2>(tt, add, early);
        case 3: return pick_tt<3>(tt, add, early);
        default: return pick_tt<4>(tt, add, early);
    }
}

}  // namespace

// Launch geometry from host-known sizes only: 256 columns per column block,
// TT tiles of 16 tokens per unit following the expected segment length
// N / min(N, max_loras + 1), and runs of R column blocks of one slice per unit
// (the unit's buffer rows are staged once for its R blocks).  R is 1, with the
// block's loads issued in the staging round trip, when units of one block fill
// the resident grid at most twice or when a 64-token tile's buffer rows are
// small (rank <= 16); otherwise R = 4 (measured best or within a few percent
// on the prefill, Zipf, large and logits shapes).
hipError_t launch_expand(const ExpandArgs &in, const ExpandTuning &cfg, hipStream_t s) {
    ExpandArgs a = in;
    const int n = a.num_tokens;
    const int nslots = a.meta.nslots;
    const int segs = nslots < n ? nslots : n;
    const int ks = (a.rank + 31) / 32;
    const int avg = (n + segs - 1) / segs;
    int tt = cfg.tile_tokens > 0 ? cfg.tile_tokens / 16 : 4;
    if (cfg.tile_tokens <= 0) {
        while (tt > 1 && 16 * tt / 2 >= avg) tt /= 2;
        // up to rank 32, 32-token tiles measured faster than 64-token ones
        // (twice the units over the same y traffic, little buffer per unit)
        if (a.rank <= 32 && tt > 2) tt = 2;
    }
    tt = tt >= 4 ? 4 : (tt >= 2 ? 2 : 1);
    a.tile_tokens = 16 * tt;
    const bool add = a.add_inputs != 0;
    a.meta.lds_tokens = n <= kLdsTokensMax ? n : 0;
    const size_t lds = sizeof(int) * (size_t)(4 * nslots + 1 + a.meta.lds_tokens);
    const long tiles_upper = (n + a.tile_tokens - 1) / a.tile_tokens + segs;

    auto count_runs = [&](int r) {
        long runs = 0;
        for (int i = 0; i < a.num_slices; ++i) {
            a.run_begin[i] = (int)runs;
            runs += ((a.width[i] + kBlockCols - 1) / kBlockCols + r - 1) / r;
        }
        for (int i = a.num_slices; i <= LORA_MAX_SLICES; ++i) a.run_begin[i] = (int)runs;
        return runs;
    };
    // Run length: 16 blocks when segments are tiny (each unit then stages a
    // handful of buffer rows once for many weight blocks), else 4; halved
    // while fewer than kMinUnits units would be left to spread over the
    // device.  Fitted to sweeps over the decode, prefill, Zipf, large, logits
    // and embedding shapes.
    constexpr long kMinUnits = 800;
    int r = 1;
    if (cfg.run_blocks > 0) {
        r = cfg.run_blocks;
    } else {
        r = avg < 16 ? 16 : 4;
        while (r > 1 && tiles_upper * count_runs(r) < kMinUnits) r /= 2;
    }
    // Shares of the (tile, column block) list instead of units of r blocks
    // (LORA_EXPAND_SHARE=1 forces it, 2 turns it off), for ranks above 64:
    // there a unit is long (each block moves 16 KB of weights per wave) and
    // the uneven count of units per workgroup costs most (measured: large
    // 221 -> 200 us; no gain on the rank-64 prefill shape, a loss on the
    // rank-16 and rank-32 shapes).
    a.share = cfg.share == 1 || (cfg.share == 0 && cfg.run_blocks <= 0 && r > 1 && a.rank > 64);
    if (a.share) r = 1;
    a.run_blocks = r;
    a.runs = (int)count_runs(r);
    const ExpandFn fn = pick(ks, tt, add, r == 1 && !a.share);
    const long units_upper = tiles_upper * a.runs;
    a.num_units = (int)units_upper;
    long grid = persistent_grid(units_upper, cfg.grid_cap > 0 ? cfg.grid_cap : 2048,
                                reinterpret_cast<const void *>(fn), kThreads, lds);
    if (a.share && cfg.grid_cap <= 0) {
        // every resident workgroup, as long as each gets a few blocks
        long res = resident_grid(reinterpret_cast<const void *>(fn), kThreads, lds);
        const long by_work = units_upper / 4;
        if (res > by_work) res = by_work;
        grid = res / kNumXcd * kNumXcd;
        if (grid < kNumXcd) grid = kNumXcd;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace lora
