// lora_shrink.hip -- buf[i][t][:] += scale * x[t] @ A_i[id_t]^T for tokens
// grouped by LoRA id (PunicaWrapperGPU.add_shrink on the "punica_gpu" page).
//
// Each segment (the tokens of one id, contiguous in the sorted index list) is
// a skinny GEMM  C[rows = S*r][tokens] = A_id[rows][H] * X_seg[tokens][H]^T
// run on the bf16 MFMA (v_mfma_f32_16x16x32_bf16) with the weight rows on the
// M side and the gathered token rows on the N side, so that every lane ends up
// with 4 consecutive rank entries of one token: 16-byte stores into buf.
//
// Work unit = (token tile of the segment, block of weight rows, K chunk).
// A workgroup has 4 waves laid out as WR (row groups) x WK (K interleave);
// each wave streams its weight rows and the tile's token rows straight from
// HBM into MFMA operand registers: every lane loads 32 contiguous bytes per
// row per 64-wide K step (4 lanes cover one 128-byte line), which feeds two
// MFMAs (the same K permutation is applied to both operands, so the sum is
// unchanged).  The next K step is loaded while the current one is multiplied.
// Partial sums of the WK waves are added in LDS; K chunks (split-K) are
// combined with float atomics, or a plain read-modify-write when the unit
// covers all of K.
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

// 16 bf16 of one row starting at element k, zero past `end` (8-element granularity).
__device__ __forceinline__ void load_row32(const uint16_t *row, bool valid, int k, int end, u32x4 &lo, u32x4 &hi) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    lo = z;
    hi = z;
    if (valid) {
        if (k + 8 <= end) lo = *reinterpret_cast<const u32x4 *>(row + k);
        if (k + 16 <= end) hi = *reinterpret_cast<const u32x4 *>(row + k + 8);
    }
}

template <int NT, int MT, int WK>
__global__ __launch_bounds__(kThreads) void shrink_kernel(ShrinkArgs a) {
    constexpr int WR = 4 / WK;
    constexpr int kTileTokens = 16 * NT;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int wk = wave % WK, wr = wave / WK;

    if (*a.meta.no_lora) return;

    int unit = blockIdx.x;
    const int ks = unit % a.k_splits;
    unit /= a.k_splits;
    const int rb = unit % a.row_blocks;
    const int tile_u = unit / a.row_blocks;

    int slot, tile, seg_start, seg_count, lid;
    if (!find_tile(a.meta, kTileTokens, tile_u, slot, tile, seg_start, seg_count, lid)) return;

    const int col = lane & 15, g = lane >> 4;
    const int rows_per_wg = WR * MT * 16;

    // token rows (N side of the MFMA)
    const uint16_t *xrow[NT];
    bool xvalid[NT];
    int tok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int p = tile * kTileTokens + nt * 16 + col;
        xvalid[nt] = p < seg_count && seg_start + p < a.num_tokens;
        tok[nt] = xvalid[nt] ? a.meta.sorted[seg_start + p] : 0;
        // a token index outside the batch (metadata not from this batch) is skipped
        if ((unsigned)tok[nt] >= (unsigned)a.num_tokens) {
            xvalid[nt] = false;
            tok[nt] = 0;
        }
        xrow[nt] = a.x + (int64_t)tok[nt] * a.ldx;
    }
    // weight rows (M side)
    const uint16_t *arow[MT];
    bool avalid[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row = rb * rows_per_wg + (wr * MT + mt) * 16 + col;
        avalid[mt] = row < a.rows;
        const int r = avalid[mt] ? row : 0;
        const int i = r / a.rank, j = r - i * a.rank;
        arow[mt] = select_ptr(a.a, i) + ((int64_t)lid * a.rank + j) * a.hidden;
    }

    const int kbeg = ks * a.k_chunk;
    const int kend = min(kbeg + a.k_chunk, a.hidden);
    const int nsteps = (kend - kbeg + 63) / 64;

    floatx4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

    u32x4 av[MT][2], xv[NT][2];
    int s = wk;
    if (s < nsteps) {
        const int k = kbeg + s * 64 + g * 16;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) load_row32(arow[mt], avalid[mt], k, kend, av[mt][0], av[mt][1]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) load_row32(xrow[nt], xvalid[nt], k, kend, xv[nt][0], xv[nt][1]);
    }
    for (; s < nsteps; s += WK) {
        u32x4 an[MT][2], xn[NT][2];
        const bool more = s + WK < nsteps;
        if (more) {
            const int k = kbeg + (s + WK) * 64 + g * 16;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) load_row32(arow[mt], avalid[mt], k, kend, an[mt][0], an[mt][1]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) load_row32(xrow[nt], xvalid[nt], k, kend, xn[nt][0], xn[nt][1]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] = mfma16x16x32(as_bf16x8(av[mt][h]), as_bf16x8(xv[nt][h]), acc[mt][nt]);
        if (more) {
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
    }

    if constexpr (WK > 1) {
        __shared__ floatx4 red[(WK - 1) * WR * MT * NT * kWave];
        if (wk > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    red[(((wk - 1) * WR + wr) * MT * NT + mt * NT + nt) * kWave + lane] = acc[mt][nt];
        }
        __syncthreads();
        if (wk > 0) return;
#pragma unroll
        for (int w = 1; w < WK; ++w)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] += red[(((w - 1) * WR + wr) * MT * NT + mt * NT + nt) * kWave + lane];
    }

    // D layout: lane holds rows 4g..4g+3 of the m-tile for token column `col`.
    const bool atomic = a.k_splits > 1;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row0 = rb * rows_per_wg + (wr * MT + mt) * 16 + 4 * g;
        if (row0 >= a.rows) continue;
        const int i = row0 / a.rank, j = row0 - i * a.rank;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (!xvalid[nt]) continue;
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
        default: return pick_wk<4>(wk, mt);
    }
}

}  // namespace

// Tile selection from host-known sizes only.  `tokens_per_tile` and `waves_k`
// may be forced (> 0) for tuning; otherwise they follow the expected tokens
// per segment, N / min(N, max_loras + 1).
hipError_t launch_shrink(const ShrinkArgs &in, int tokens_per_tile, int waves_k, hipStream_t s) {
    ShrinkArgs a = in;
    const int n = a.num_tokens;
    const int nslots = a.meta.nslots;
    const int mtiles = (a.rows + 15) / 16;
    const int segs = nslots < n ? nslots : n;
    const int avg = (n + segs - 1) / segs;

    int nt = tokens_per_tile > 0 ? tokens_per_tile / 16 : (avg <= 16 ? 1 : (avg <= 32 ? 2 : 4));
    if (nt != 1 && nt != 2) nt = 4;
    int wk = waves_k;
    if (wk != 1 && wk != 2 && wk != 4) {
        // enough m-tiles for 4 row groups: split rows; otherwise interleave K
        wk = mtiles >= 4 * 2 ? 1 : (mtiles >= 2 * 2 ? 2 : 4);
    }
    const int wr = 4 / wk;
    int mt = (mtiles + wr - 1) / wr;
    if (mt > 4) mt = 4;
    const int rows_per_wg = wr * mt * 16;
    a.row_blocks = (a.rows + rows_per_wg - 1) / rows_per_wg;

    const int tile_tokens = 16 * nt;
    const int tiles_upper = (n + tile_tokens - 1) / tile_tokens + segs;
    // expected busy units without split-K
    const int busy = ((n + tile_tokens - 1) / tile_tokens + (segs + 1) / 2) * a.row_blocks;
    int ks = 1;
    const int target = 2 * 256;
    if (busy < target) ks = (target + busy - 1) / busy;
    const int max_ks = (a.hidden + 255) / 256;
    if (ks > max_ks) ks = max_ks;
    if (ks < 1) ks = 1;
    if (const char *e = getenv("LORA_SHRINK_KSPLIT")) {
        int v = atoi(e);
        if (v >= 1) ks = v < max_ks ? v : max_ks;
    }
    int chunk = (a.hidden + ks - 1) / ks;
    chunk = (chunk + 63) / 64 * 64;
    ks = (a.hidden + chunk - 1) / chunk;
    a.k_splits = ks;
    a.k_chunk = chunk;
    a.num_units = tiles_upper * a.row_blocks * ks;

    ShrinkFn fn = pick(nt, wk, mt);
    hipLaunchKernelGGL(fn, dim3(a.num_units), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace lora
