// lora_shrink.hip -- buf[i][t][:] += scale * x[t] @ A_i[id_t]^T for tokens
// grouped by LoRA id (PunicaWrapperGPU.add_shrink on the "punica_gpu" page).
//
// Each segment (the tokens of one id, contiguous in the sorted index list) is
// a skinny GEMM  C[rows = S*r][tokens] = A_id[rows][H] * X_seg[tokens][H]^T
// run on the bf16 MFMA (v_mfma_f32_16x16x32_bf16) with the weight rows on the
// M side and the gathered token rows on the N side, so that every lane ends up
// with 4 consecutive rank entries of one token: 16-byte stores into buf.
//
// Work unit = (token tile of a segment, block of weight rows, K chunk), in a
// canonical tile-major order that is cut into one contiguous chunk per XCD
// (neighbouring units share x rows or weight rows through that XCD's L2).
// The grid is persistent: each workgroup builds the tile table in LDS once and
// walks its chunk.  A workgroup has 4 waves laid out as WR (row groups) x WK
// (K interleave); each wave streams its weight rows and the tile's token rows
// from HBM straight into MFMA operand registers: every lane loads 32
// contiguous bytes of a row per 64-wide K step (4 lanes cover one 128-byte
// line), feeding two MFMAs (the same K permutation on both operands leaves
// the sum unchanged).
//
// All loads are unconditional: lanes of missing tokens or rows read a clamped
// valid row (their outputs are discarded), and only the last K step of a
// ragged K range is masked.  With a fixed number of loads per step the
// compiler can wait for exactly the step being multiplied while the next one
// is in flight.  Partial sums of the WK waves are added in LDS; K chunks are
// combined with float atomics, else the unit does a read-modify-write of buf.
#include "lora_internal.h"

#include <stdlib.h>

namespace lora {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ const uint16_t *select_ptr(const uint16_t *const (&p)[LORA_MAX_SLICES], int i) {
    const uint16_t *r = p[0];
#pragma unroll
    for (int s = 1; s < LORA_MAX_SLICES; ++s)
        if (i == s) r = p[s];
    return r;
}

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Loads of one 64-wide K step: 16 elements of each row at kk (clamped to the
// row start where the step runs past kend; those halves are masked later).
template <int N>
__device__ __forceinline__ void load_step(const uint16_t *const (&row)[N], int kk, int kend, u32x4 (&v)[N][2]) {
    const int o0 = kk + 8 <= kend ? kk : 0;
    const int o1 = kk + 16 <= kend ? kk + 8 : 0;
#pragma unroll
    for (int q = 0; q < N; ++q) {
        v[q][0] = ld16(row[q] + o0);
        v[q][1] = ld16(row[q] + o1);
    }
}

template <int N>
__device__ __forceinline__ void mask_step(int kk, int kend, u32x4 (&v)[N][2]) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bool ok0 = kk + 8 <= kend, ok1 = kk + 16 <= kend;
#pragma unroll
    for (int q = 0; q < N; ++q) {
        v[q][0] = ok0 ? v[q][0] : z;
        v[q][1] = ok1 ? v[q][1] : z;
    }
}

template <int NT, int MT, int WK>
__global__ __launch_bounds__(kThreads) void shrink_kernel(ShrinkArgs a) {
    constexpr int WR = 4 / WK;
    constexpr int kTileTokens = 16 * NT;
    extern __shared__ int smem[];
    __shared__ int s_wsum[kThreads / kWave];
    __shared__ floatx4 red[(WK > 1 ? WK - 1 : 1) * WR * MT * NT * kWave];

    if (*a.meta.no_lora) return;
    const int nslots = a.meta.nslots;
    const int total = build_tile_table(a.meta, kTileTokens, smem, s_wsum);

    const int lane = lane_id(), wave = wave_id();
    const int wk = wave % WK, wr = wave / WK;
    const int col = lane & 15, g = lane >> 4;
    const int rows_per_wg = WR * MT * 16;
    const bool atomic = a.k_splits > 1;

    const UnitWalker walk(total * a.row_blocks * a.k_splits);
    for (int jj = walk.first;; jj += walk.stride) {
        const int u = walk.unit(jj);
        if (u < 0) break;
        const int ks = u % a.k_splits;
        const int rest = u / a.k_splits;
        const int rb = rest % a.row_blocks;
        const TileRef tr = lookup_tile(smem, nslots, rest / a.row_blocks);

        // token rows (N side); missing tokens repeat the segment's last token
        const uint16_t *xrow[NT];
        int tok[NT];
        bool tv[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int p = tr.tile * kTileTokens + nt * 16 + col;
            tv[nt] = p < tr.seg_count;
            int t = a.meta.sorted[tr.seg_start + (tv[nt] ? p : tr.seg_count - 1)];
            if ((unsigned)t >= (unsigned)a.num_tokens) {   // metadata not from this batch
                t = 0;
                tv[nt] = false;
            }
            tok[nt] = t;
            xrow[nt] = a.x + (int64_t)t * a.ldx;
        }
        // weight rows (M side); rows past S*r repeat the last row
        const uint16_t *arow[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            int row = rb * rows_per_wg + (wr * MT + mt) * 16 + col;
            row = row < a.rows ? row : a.rows - 1;
            const int i = row / a.rank, j = row - i * a.rank;
            arow[mt] = select_ptr(a.a, i) + ((int64_t)tr.lora_id * a.rank + j) * a.hidden;
        }

        const int kbeg = ks * a.k_chunk;
        const int kend = min(kbeg + a.k_chunk, a.hidden);
        const int nsteps = (kend - kbeg + 63) / 64;
        const bool ragged = ((kend - kbeg) & 63) != 0;

        floatx4 acc[MT][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

        u32x4 av[MT][2], xv[NT][2];
        {
            const int kk = kbeg + min(wk, nsteps - 1) * 64 + g * 16;
            load_step<MT>(arow, kk, kend, av);
            load_step<NT>(xrow, kk, kend, xv);
        }
        for (int s = wk; s < nsteps; s += WK) {
            // prefetch the next step (the last step is re-read, never skipped)
            u32x4 an[MT][2], xn[NT][2];
            const int kn = kbeg + min(s + WK, nsteps - 1) * 64 + g * 16;
            load_step<MT>(arow, kn, kend, an);
            load_step<NT>(xrow, kn, kend, xn);
            if (ragged && s == nsteps - 1) {
                const int kk = kbeg + s * 64 + g * 16;
                mask_step<MT>(kk, kend, av);
                mask_step<NT>(kk, kend, xv);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        acc[mt][nt] = mfma16x16x32(as_bf16x8(av[mt][h]), as_bf16x8(xv[nt][h]), acc[mt][nt]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                av[mt][0] = an[mt][0];
                av[mt][1] = an[mt][1];
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                xv[nt][0] = xn[nt][0];
                xv[nt][1] = xn[nt][1];
            }
        }

        bool writer = true;
        if constexpr (WK > 1) {
            if (wk > 0) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        red[(((wk - 1) * WR + wr) * MT * NT + mt * NT + nt) * kWave + lane] = acc[mt][nt];
            }
            __syncthreads();
            if (wk == 0) {
#pragma unroll
                for (int w = 1; w < WK; ++w)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            acc[mt][nt] += red[(((w - 1) * WR + wr) * MT * NT + mt * NT + nt) * kWave + lane];
            }
            __syncthreads();   // `red` is rewritten by the next unit
            writer = wk == 0;
        }

        // D layout: lane holds rows 4g..4g+3 of the m-tile for token column `col`.
        if (writer) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row0 = rb * rows_per_wg + (wr * MT + mt) * 16 + 4 * g;
                if (row0 >= a.rows) continue;
                const int i = row0 / a.rank, j = row0 - i * a.rank;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if (!tv[nt]) continue;
                    float *dst = a.buf + ((int64_t)i * a.num_tokens + tok[nt]) * a.rank + j;
                    const floatx4 v = acc[mt][nt] * a.scale;
                    if (atomic) {
                        unsafeAtomicAdd(dst + 0, v[0]);
                        unsafeAtomicAdd(dst + 1, v[1]);
                        unsafeAtomicAdd(dst + 2, v[2]);
                        unsafeAtomicAdd(dst + 3, v[3]);
                    } else {
                        floatx4 o = *reinterpret_cast<floatx4 *>(dst);
                        o += v;
                        *reinterpret_cast<floatx4 *>(dst) = o;
                    }
                }
            }
        }
    }
}

typedef void (*ShrinkFn)(ShrinkArgs);

template <int NT, int WK>
ShrinkFn pick_mt(int mt) {
    switch (mt) {
        case 1: return shrink_kernel<NT, 1, WK>;
        case 2: return shrink_kernel<NT, 2, WK>;
        case 3: return shrink_kernel<NT, 3, WK>;
        default: return shrink_kernel<NT, 4, WK>;
    }
}

template <int NT>
ShrinkFn pick_wk(int wk, int mt) {
    switch (wk) {
        case 1: return pick_mt<NT, 1>(mt);
        case 2: return pick_mt<NT, 2>(mt);
        default: return pick_mt<NT, 4>(mt);
    }
}

ShrinkFn pick(int nt, int wk, int mt) {
    switch (nt) {
        case 1: return pick_wk<1>(wk, mt);
        case 2: return pick_wk<2>(wk, mt);
        case 4: return pick_wk<4>(wk, mt);
        default: return pick_wk<8>(wk, mt);
    }
}

}  // namespace

// Tile selection from host-known sizes only (no device sync): tokens per
// tile follow the expected segment length N / min(N, max_loras + 1); rows
// are split over the 4 waves when there are enough 16-row MFMA tiles, else
// K is interleaved over the waves; K chunks are added only when the units
// would not cover the GPU.  `cfg` fields > 0 override the choice (tuning).
hipError_t launch_shrink(const ShrinkArgs &in, const ShrinkTuning &cfg, hipStream_t s) {
    ShrinkArgs a = in;
    const int n = a.num_tokens;
    const int nslots = a.meta.nslots;
    const int mtiles = (a.rows + 15) / 16;
    const int segs = nslots < n ? nslots : n;
    const int avg = (n + segs - 1) / segs;

    int nt = cfg.tile_tokens > 0 ? cfg.tile_tokens / 16 : (avg <= 16 ? 1 : (avg <= 32 ? 2 : (avg <= 64 ? 4 : 8)));
    if (nt != 1 && nt != 2 && nt != 4) nt = 8;
    int wk = cfg.waves_k;
    if (wk != 1 && wk != 2 && wk != 4) wk = mtiles >= 8 ? 1 : (mtiles >= 4 ? 2 : 4);
    const int wr = 4 / wk;
    int mt = cfg.mtiles_per_wave > 0 ? cfg.mtiles_per_wave : (mtiles + wr - 1) / wr;
    if (mt > 4) mt = 4;
    if (nt == 8 && mt > 2) mt = 2;
    const int rows_per_wg = wr * mt * 16;
    a.row_blocks = (a.rows + rows_per_wg - 1) / rows_per_wg;

    const int tile_tokens = 16 * nt;
    const int tiles_upper = (n + tile_tokens - 1) / tile_tokens + segs;
    const int busy = ((n + tile_tokens - 1) / tile_tokens + (segs + 1) / 2) * a.row_blocks;
    int ks = 1;
    const int target = 2 * 256;
    if (busy < target) ks = (target + busy - 1) / busy;
    const int max_ks = (a.hidden + 255) / 256;
    if (cfg.k_splits > 0) ks = cfg.k_splits;
    if (ks > max_ks) ks = max_ks;
    if (ks < 1) ks = 1;
    int chunk = (a.hidden + ks - 1) / ks;
    chunk = (chunk + 63) / 64 * 64;
    ks = (a.hidden + chunk - 1) / chunk;
    a.k_splits = ks;
    a.k_chunk = chunk;
    const long units_upper = (long)tiles_upper * a.row_blocks * ks;
    const int cap = cfg.grid_cap > 0 ? cfg.grid_cap : 1024;
    long grid = units_upper < cap ? units_upper : cap;
    grid = (grid + kNumXcd - 1) / kNumXcd * kNumXcd;
    a.num_units = (int)units_upper;

    ShrinkFn fn = pick(nt, wk, mt);
    const size_t lds = sizeof(int) * (size_t)(4 * nslots + 1);
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace lora
