// lora_expand.hip -- y[t, off_i + c] = bf16((add_inputs ? y : 0) + buf[i][t] @ B_i[id_t][c]
// + bias_i[id_t][c]) for tokens grouped by LoRA id (PunicaWrapperGPU.add_expand
// on the "punica_gpu" page; per-slice column offsets as in
// PunicaWrapperTPU.add_expand and the bias rule of PunicaWrapperTPU._apply_bias
// on the "punica_tpu" page, folded into one pass with a single rounding).
//
// Per segment and slice this is C[cols][tokens] = B_id[cols][r] * buf_seg[tokens][r]^T
// with K = r (8..128), on the bf16 MFMA (v_mfma_f32_16x16x32_bf16):
//   - each wave owns 64 output columns of one slice; a workgroup (4 waves)
//     covers 256 columns, and a work unit is (TT tiles of 16 tokens of one
//     segment) x (256 columns);
//   - the wave loads its weights (64 x r) once per unit, then, for all TT
//     token tiles at once, the token indices and afterwards the fp32 buffer
//     rows and the y rows, so a unit costs two memory round trips;
//   - each fp32 buffer value is split into bf16 hi = rne(v) and lo = rne(v - hi)
//     and both parts go through the MFMA, keeping ~16 mantissa bits;
//   - the 64 columns are permuted onto the four 16-row MFMA tiles so that a
//     lane ends with 16 consecutive columns of one token: y is read and
//     written as 32 contiguous bytes per lane (128 per token row per wave).
// Work units follow a canonical tile-major order cut into one chunk per XCD,
// walked by a persistent grid.
//
// Loads are unconditional.  A lane whose token is past the end of the
// segment works on the segment's last token, and an 8-column group past the
// end of the slice works on the slice's last 8 columns: such a lane computes
// exactly the values of the lane that owns that data and stores them to the
// same address, so the duplicate store is harmless.  Tokens with id -1 own no
// tile and are never touched.
#include "lora_internal.h"

namespace lora {

namespace {

constexpr int kThreads = 256;
constexpr int kWaveCols = 64;
constexpr int kBlockCols = 4 * kWaveCols;

template <typename T, int N>
__device__ __forceinline__ T select_slice(const T (&p)[N], int i) {
    T r = p[0];
#pragma unroll
    for (int s = 1; s < N; ++s)
        if (i == s) r = p[s];
    return r;
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return lo16 | (hi16 << 16); }

// Split 8 floats into bf16 hi and lo operands.
__device__ __forceinline__ void split_bf16(const floatx4 &v0, const floatx4 &v1, u32x4 &hi, u32x4 &lo) {
    const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    uint32_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = float_to_bf16_bits(v[e]);
        l[e] = float_to_bf16_bits(v[e] - bf16_bits_to_float(h[e]));
    }
    hi = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
    lo = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
}

// Column a lane works on for slice column c: itself when inside the slice,
// else the same position in the slice's last 8-column group.
__device__ __forceinline__ int clamp_col(int c, int width) { return c < width ? c : width - 8 + (c & 7); }

template <int KS, int TT, bool ADD>
__global__ __launch_bounds__(kThreads) void expand_kernel(ExpandArgs a) {
    extern __shared__ int smem[];
    __shared__ int s_wsum[kThreads / kWave];

    if (*a.meta.no_lora) return;
    const int nslots = a.meta.nslots;
    constexpr int kUnitTokens = 16 * TT;
    const int total = build_tile_table(a.meta, kUnitTokens, smem, s_wsum);

    const int lane = lane_id(), wave = wave_id();
    const int col = lane & 15, g = lane >> 4;
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    const floatx4 zf = {0.f, 0.f, 0.f, 0.f};

    const UnitWalker walk(total * a.col_blocks);
    for (int jj = walk.first;; jj += walk.stride) {
        const int u = walk.unit(jj);
        if (u < 0) break;
        const int cb = u % a.col_blocks;
        const TileRef tr = lookup_tile(smem, nslots, u / a.col_blocks);

        int i = 0;
#pragma unroll
        for (int s = 1; s < LORA_MAX_SLICES; ++s)
            if (s < a.num_slices && cb >= a.block_begin[s]) i = s;
        const int width = select_slice(a.width, i);
        const int c0 = (cb - select_slice(a.block_begin, i)) * kBlockCols + wave * kWaveCols;
        if (c0 >= width) continue;   // this wave has no columns in the block (no barrier below)

        // token indices of the unit's TT tiles (past the end: the last token)
        int tok[TT];
#pragma unroll
        for (int q = 0; q < TT; ++q) {
            int p = tr.tile * kUnitTokens + q * 16 + col;
            p = p < tr.seg_count ? p : tr.seg_count - 1;
            tok[q] = a.meta.sorted[tr.seg_start + p];
        }

        // weights: MFMA row `col` of tile mt is output column 16*(col/4) + 4*mt + col%4
        const uint16_t *wbase = select_slice(a.b, i) + (int64_t)tr.lora_id * width * a.rank;
        u32x4 w[4][KS];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int c = clamp_col(c0 + 16 * (col >> 2) + 4 * mt + (col & 3), width);
            const uint16_t *row = wbase + (int64_t)c * a.rank;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int k = ks * 32 + 8 * g;
                w[mt][ks] = *reinterpret_cast<const u32x4 *>(row + (k < a.rank ? k : 0));
            }
        }
        // this lane's output columns: two groups of 8 starting at cl and cl + 8
        const int cl = c0 + 16 * g;
        const int cg0 = clamp_col(cl, width), cg1 = clamp_col(cl + 8, width);
        const uint16_t *bptr = select_slice(a.bias, i);
        u32x4 bias0 = z4, bias1 = z4;
        if (bptr) {
            const uint16_t *brow = bptr + (int64_t)tr.lora_id * width;
            bias0 = *reinterpret_cast<const u32x4 *>(brow + cg0);
            bias1 = *reinterpret_cast<const u32x4 *>(brow + cg1);
        }

        // guard against metadata that is not from this batch
        bool tv[TT];
#pragma unroll
        for (int q = 0; q < TT; ++q) {
            tv[q] = (unsigned)tok[q] < (unsigned)a.num_tokens;
            tok[q] = tv[q] ? tok[q] : 0;
        }

        // buffer rows and y rows of all tiles
        const float *bufs = a.buf + (int64_t)i * a.num_tokens * a.rank;
        const int ycol = select_slice(a.col_off, i);
        floatx4 bv[TT][KS][2];
        u32x4 yv[TT][2];
#pragma unroll
        for (int q = 0; q < TT; ++q) {
            const float *brow = bufs + (int64_t)tok[q] * a.rank;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int k = ks * 32 + 8 * g;
                const int kc = k < a.rank ? k : 0;
                bv[q][ks][0] = *reinterpret_cast<const floatx4 *>(brow + kc);
                bv[q][ks][1] = *reinterpret_cast<const floatx4 *>(brow + kc + 4);
            }
            if (ADD) {
                const uint16_t *yrow = a.y + (int64_t)tok[q] * a.ldy + ycol;
                yv[q][0] = *reinterpret_cast<const u32x4 *>(yrow + cg0);
                yv[q][1] = *reinterpret_cast<const u32x4 *>(yrow + cg1);
            } else {
                yv[q][0] = z4;
                yv[q][1] = z4;
            }
        }

        // rank tail: K positions >= r contribute nothing
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bool kin = ks * 32 + 8 * g < a.rank;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) w[mt][ks] = kin ? w[mt][ks] : z4;
#pragma unroll
            for (int q = 0; q < TT; ++q) {
                bv[q][ks][0] = kin ? bv[q][ks][0] : zf;
                bv[q][ks][1] = kin ? bv[q][ks][1] : zf;
            }
        }
        float bias[16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bias[2 * e] = bf16_bits_to_float(bias0[e] & 0xffffu);
            bias[2 * e + 1] = bf16_bits_to_float(bias0[e] >> 16);
            bias[8 + 2 * e] = bf16_bits_to_float(bias1[e] & 0xffffu);
            bias[8 + 2 * e + 1] = bf16_bits_to_float(bias1[e] >> 16);
        }

#pragma unroll
        for (int q = 0; q < TT; ++q) {
            floatx4 acc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) acc[mt] = zf;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 hi, lo;
                split_bf16(bv[q][ks][0], bv[q][ks][1], hi, lo);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    acc[mt] = mfma16x16x32(as_bf16x8(w[mt][ks]), as_bf16x8(hi), acc[mt]);
                    acc[mt] = mfma16x16x32(as_bf16x8(w[mt][ks]), as_bf16x8(lo), acc[mt]);
                }
            }
            // acc[mt][e] is column cl + 4*mt + e of token tok[q] (or its duplicate)
            uint16_t *yrow = a.y + (int64_t)tok[q] * a.ldy + ycol;
#pragma unroll
            for (int hgrp = 0; hgrp < 2; ++hgrp) {
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c_lo = 8 * hgrp + 2 * e, c_hi = c_lo + 1;
                    const float d_lo = acc[c_lo >> 2][c_lo & 3] + bias[c_lo];
                    const float d_hi = acc[c_hi >> 2][c_hi & 3] + bias[c_hi];
                    const float r_lo = bf16_bits_to_float(yv[q][hgrp][e] & 0xffffu) + d_lo;
                    const float r_hi = bf16_bits_to_float(yv[q][hgrp][e] >> 16) + d_hi;
                    o[e] = pack2(float_to_bf16_bits(r_lo), float_to_bf16_bits(r_hi));
                }
                if (tv[q]) *reinterpret_cast<u32x4 *>(yrow + (hgrp ? cg1 : cg0)) = u32x4{o[0], o[1], o[2], o[3]};
            }
        }
    }
}

typedef void (*ExpandFn)(ExpandArgs);

template <int KS, int TT>
ExpandFn pick_add(bool add) {
    return add ? expand_kernel<KS, TT, true> : expand_kernel<KS, TT, false>;
}

template <int KS>
ExpandFn pick_tt(int tt, bool add) {
    switch (tt) {
        case 1: return pick_add<KS, 1>(add);
        case 2: return pick_add<KS, 2>(add);
        default: return pick_add<KS, 4>(add);
    }
}

}  // namespace

// Launch geometry from host-known sizes only: 256 columns per workgroup,
// 16-token tiles per unit bounded by registers (TT * ceil(r/32) <= 4) and by
// the expected segment length N / min(N, max_loras + 1).
hipError_t launch_expand(const ExpandArgs &in, const ExpandTuning &cfg, hipStream_t s) {
    ExpandArgs a = in;
    int blocks = 0;
    for (int i = 0; i < a.num_slices; ++i) {
        a.block_begin[i] = blocks;
        blocks += (a.width[i] + kBlockCols - 1) / kBlockCols;
    }
    for (int i = a.num_slices; i <= LORA_MAX_SLICES; ++i) a.block_begin[i] = blocks;
    a.col_blocks = blocks;
    const int n = a.num_tokens;
    const int nslots = a.meta.nslots;
    const int segs = nslots < n ? nslots : n;
    const int ks = (a.rank + 31) / 32;
    int tt = cfg.tile_tokens > 0 ? cfg.tile_tokens / 16 : 4 / ks;
    if (cfg.tile_tokens <= 0) {
        const int avg = (n + segs - 1) / segs;
        while (tt > 1 && 16 * tt / 2 >= avg) tt /= 2;
    }
    tt = tt >= 4 ? 4 : (tt >= 2 ? 2 : 1);
    a.tile_tokens = 16 * tt;
    const long tiles_upper = (n + a.tile_tokens - 1) / a.tile_tokens + segs;
    const long units_upper = tiles_upper * a.col_blocks;
    const int cap = cfg.grid_cap > 0 ? cfg.grid_cap : 2048;
    long grid = units_upper < cap ? units_upper : cap;
    grid = (grid + kNumXcd - 1) / kNumXcd * kNumXcd;
    a.num_units = (int)units_upper;
    ExpandFn fn;
    const bool add = a.add_inputs != 0;
    switch (ks) {
        case 1: fn = pick_tt<1>(tt, add); break;
        case 2: fn = pick_tt<2>(tt, add); break;
        case 3: fn = pick_tt<3>(tt, add); break;
        default: fn = pick_tt<4>(tt, add); break;
    }
    const size_t lds = sizeof(int) * (size_t)(4 * nslots + 1);
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace lora
