// lora_expand.hip -- y[t, off_i + c] = bf16((add_inputs ? y : 0) + buf[i][t] @ B_i[id_t][c]
// + bias_i[id_t][c]) for tokens grouped by LoRA id (PunicaWrapperGPU.add_expand
// on the "punica_gpu" page; per-slice column offsets as in
// PunicaWrapperTPU.add_expand and the bias rule of PunicaWrapperTPU._apply_bias
// on the "punica_tpu" page, folded into one pass with a single rounding).
//
// Per segment and slice this is C[cols][tokens] = B_id[cols][r] * buf_seg[tokens][r]^T,
// with K = r (8..128).  Each wave owns 64 output columns of one slice and keeps
// their weights (64 x r bf16) in registers for the whole token range of its
// work unit, walking the segment's tokens 16 at a time:
//   - the fp32 buffer row of each token is split into bf16 hi + lo parts
//     (hi = rne(v), lo = rne(v - hi)) and both go through the MFMA, so the
//     product keeps ~16 mantissa bits of the fp32 input;
//   - the 64 columns are permuted onto the four 16-row MFMA tiles so that each
//     lane ends with 16 consecutive columns of one token: y is read and written
//     as 32 contiguous bytes per lane, 128 bytes per token row per wave.
// Rows of y are gathered through the sorted token index; tokens with id -1 own
// no tile and are never touched.
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
    float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    uint32_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = float_to_bf16_bits(v[e]);
        l[e] = float_to_bf16_bits(v[e] - bf16_bits_to_float(h[e]));
    }
    hi = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
    lo = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
}

template <int KS>
__global__ __launch_bounds__(kThreads) void expand_kernel(ExpandArgs a) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    if (*a.meta.no_lora) return;

    const int cb = blockIdx.x % a.col_blocks;
    const int tile_u = blockIdx.x / a.col_blocks;
    int slot, tile, seg_start, seg_count, lid;
    if (!find_tile(a.meta, a.tile_tokens, tile_u, slot, tile, seg_start, seg_count, lid)) return;

    int i = 0;
#pragma unroll
    for (int s = 1; s < LORA_MAX_SLICES; ++s)
        if (s < a.num_slices && cb >= a.block_begin[s]) i = s;
    const int width = select_slice(a.width, i);
    const int c0 = (cb - select_slice(a.block_begin, i)) * kBlockCols + wave * kWaveCols;
    if (c0 >= width) return;

    const int col = lane & 15, g = lane >> 4;
    const uint16_t *wbase = select_slice(a.b, i) + (int64_t)lid * width * a.rank;

    // weights: MFMA row `col` of tile mt is output column 16*(col/4) + 4*mt + col%4
    u32x4 w[4][KS];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int c = c0 + 16 * (col >> 2) + 4 * mt + (col & 3);
        const bool cv = c < width;
        const uint16_t *row = wbase + (int64_t)(cv ? c : 0) * a.rank;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k = ks * 32 + 8 * g;
            w[mt][ks] = (cv && k < a.rank) ? *reinterpret_cast<const u32x4 *>(row + k) : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // this lane's output columns: c0 + 16g .. c0 + 16g + 15 (two groups of 8)
    const int cl = c0 + 16 * g;
    const bool ok0 = cl < width, ok1 = cl + 8 < width;
    float bias[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) bias[e] = 0.f;
    const uint16_t *bptr = select_slice(a.bias, i);
    if (bptr) {
        const uint16_t *brow = bptr + (int64_t)lid * width + cl;
        u32x4 b0 = ok0 ? *reinterpret_cast<const u32x4 *>(brow) : u32x4{0u, 0u, 0u, 0u};
        u32x4 b1 = ok1 ? *reinterpret_cast<const u32x4 *>(brow + 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bias[2 * e] = bf16_bits_to_float(b0[e] & 0xffffu);
            bias[2 * e + 1] = bf16_bits_to_float(b0[e] >> 16);
            bias[8 + 2 * e] = bf16_bits_to_float(b1[e] & 0xffffu);
            bias[8 + 2 * e + 1] = bf16_bits_to_float(b1[e] >> 16);
        }
    }

    const int p_begin = tile * a.tile_tokens;
    const int p_end = min(p_begin + a.tile_tokens, seg_count);
    const int ycol = select_slice(a.col_off, i) + cl;
    const float *bufs = a.buf + (int64_t)i * a.num_tokens * a.rank;

    for (int p0 = p_begin; p0 < p_end; p0 += 16) {
        const int p = p0 + col;
        bool tv = p < p_end && seg_start + p < a.num_tokens;
        int tok = tv ? a.meta.sorted[seg_start + p] : 0;
        if ((unsigned)tok >= (unsigned)a.num_tokens) {
            tv = false;
            tok = 0;
        }
        const float *brow = bufs + (int64_t)tok * a.rank;

        floatx4 acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k = ks * 32 + 8 * g;
            floatx4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
            if (tv && k < a.rank) {
                v0 = *reinterpret_cast<const floatx4 *>(brow + k);
                v1 = *reinterpret_cast<const floatx4 *>(brow + k + 4);
            }
            u32x4 hi, lo;
            split_bf16(v0, v1, hi, lo);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                acc[mt] = mfma16x16x32(as_bf16x8(w[mt][ks]), as_bf16x8(hi), acc[mt]);
                acc[mt] = mfma16x16x32(as_bf16x8(w[mt][ks]), as_bf16x8(lo), acc[mt]);
            }
        }
        if (!tv) continue;

        // acc[mt][e] is column cl + 4*mt + e of token `tok`
        uint16_t *yrow = a.y + (int64_t)tok * a.ldy + ycol;
#pragma unroll
        for (int hgrp = 0; hgrp < 2; ++hgrp) {
            if (!(hgrp == 0 ? ok0 : ok1)) continue;
            u32x4 yv = {0u, 0u, 0u, 0u};
            if (a.add_inputs) yv = *reinterpret_cast<const u32x4 *>(yrow + 8 * hgrp);
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c_lo = 8 * hgrp + 2 * e, c_hi = c_lo + 1;
                const float d_lo = acc[c_lo >> 2][c_lo & 3] + bias[c_lo];
                const float d_hi = acc[c_hi >> 2][c_hi & 3] + bias[c_hi];
                const float r_lo = bf16_bits_to_float(yv[e] & 0xffffu) + d_lo;
                const float r_hi = bf16_bits_to_float(yv[e] >> 16) + d_hi;
                o[e] = pack2(float_to_bf16_bits(r_lo), float_to_bf16_bits(r_hi));
            }
            *reinterpret_cast<u32x4 *>(yrow + 8 * hgrp) = u32x4{o[0], o[1], o[2], o[3]};
        }
    }
}

}  // namespace

hipError_t launch_expand(const ExpandArgs &in, hipStream_t s) {
    ExpandArgs a = in;
    int blocks = 0;
    for (int i = 0; i < a.num_slices; ++i) {
        a.block_begin[i] = blocks;
        blocks += (a.width[i] + kBlockCols - 1) / kBlockCols;
    }
    for (int i = a.num_slices; i <= LORA_MAX_SLICES; ++i) a.block_begin[i] = blocks;
    a.col_blocks = blocks;
    const int n = a.num_tokens;
    const int segs = a.meta.nslots < n ? a.meta.nslots : n;
    if (a.tile_tokens <= 0) {
        int avg = (n + segs - 1) / segs;
        int tt = (avg + 15) / 16 * 16;
        if (tt < 16) tt = 16;
        if (tt > 128) tt = 128;
        a.tile_tokens = tt;
    }
    const int tiles_upper = (n + a.tile_tokens - 1) / a.tile_tokens + segs;
    a.num_units = tiles_upper * a.col_blocks;
    const int ks = (a.rank + 31) / 32;
    void (*fn)(ExpandArgs);
    switch (ks) {
        case 1: fn = expand_kernel<1>; break;
        case 2: fn = expand_kernel<2>; break;
        case 3: fn = expand_kernel<3>; break;
        default: fn = expand_kernel<4>; break;
    }
    hipLaunchKernelGGL(fn, dim3(a.num_units), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace lora
