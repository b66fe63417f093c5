// lora_internal.h -- device helpers and kernel argument blocks shared by the
// gfx950 kernels of liblora_mi355x.so (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_mi355x.h"

namespace lora {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (uint64_t(1) << lane_id()) - 1;
}

// Mask of the lanes whose `key` equals this lane's, among lanes with `valid`
// set: one ballot per key bit (keys are < 2^nbits).
__device__ __forceinline__ uint64_t match_key(int key, bool valid, int nbits) {
    uint64_t m = ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        bool bit = (key >> b) & 1;
        uint64_t bb = ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int o = __shfl_up(v, d, kWave);
        if (lane_id() >= d) v += o;
    }
    return v;
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
    return __uint_as_float(h << 16);
}

// float -> bfloat16 bit pattern, round to nearest, ties to even (inputs are
// finite or inf; NaN maps to a quiet NaN).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const floatx4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) {
    return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------- metadata view

struct MetaView {
    const int32_t *sorted;       // token_indices_sorted
    const int32_t *active_ids;   // [max_loras + 1]
    const int32_t *counts;       // [max_loras + 1]
    const int32_t *start_loc;    // [max_loras + 2]
    const int32_t *no_lora;      // [1]
    int32_t nslots;              // max_loras + 1
};

// Map a linear tile index `u` onto (slot, tile-within-slot) where every slot
// with an id other than -1 owns ceil(count / tile_tokens) tiles, in slot
// order.  Computed by each wave on its own from the metadata (no barrier).
// Returns false when `u` is past the last tile.
__device__ __forceinline__ bool find_tile(const MetaView &m, int tile_tokens, int u,
                                          int &slot, int &tile, int &seg_start, int &seg_count, int &lora_id) {
    int base = 0;
    const int lane = lane_id();
    for (int c0 = 0; c0 < m.nslots; c0 += kWave) {
        int k = c0 + lane;
        int n_tiles = 0;
        int cnt = 0, id = -1;
        if (k < m.nslots) {
            cnt = m.counts[k];
            id = m.active_ids[k];
            if (id >= 0) n_tiles = (cnt + tile_tokens - 1) / tile_tokens;
        }
        int incl = wave_inclusive_scan(n_tiles);
        int excl = incl - n_tiles;
        bool hit = (n_tiles > 0) && (u >= base + excl) && (u < base + incl);
        uint64_t hm = ballot(hit);
        if (hm) {
            int src = __ffsll((long long)hm) - 1;
            slot = c0 + src;
            int e = __shfl(excl, src, kWave);
            tile = u - base - e;
            seg_count = __shfl(cnt, src, kWave);
            lora_id = __shfl(id, src, kWave);
            seg_start = m.start_loc[slot];
            return true;
        }
        base += __shfl(incl, kWave - 1, kWave);
    }
    return false;
}

// ---------------------------------------------------------------- kernel args

struct PrepareArgs {
    const int32_t *mapping;
    int32_t *mapping_copy;
    int32_t *sorted;
    int32_t *active_ids;
    int32_t *counts;
    int32_t *start_loc;
    int32_t *no_lora;
    int32_t *status;
    int32_t num_tokens;
    int32_t max_loras;
};

struct ShrinkArgs {
    MetaView meta;
    const uint16_t *x;
    int64_t ldx;
    const uint16_t *a[LORA_MAX_SLICES];
    float *buf;
    int32_t num_tokens;
    int32_t hidden;
    int32_t rank;
    int32_t rows;         // num_slices * rank
    int32_t row_blocks;   // row blocks per tile
    int32_t k_splits;     // K chunks per tile
    int32_t k_chunk;      // elements of K per chunk (multiple of 64)
    int32_t num_units;    // tiles upper bound * row_blocks * k_splits
    float scale;
};

struct ExpandArgs {
    MetaView meta;
    const float *buf;
    const uint16_t *b[LORA_MAX_SLICES];
    const uint16_t *bias[LORA_MAX_SLICES];
    uint16_t *y;
    int64_t ldy;
    int32_t width[LORA_MAX_SLICES];
    int32_t col_off[LORA_MAX_SLICES];      // first y column of each slice
    int32_t block_begin[LORA_MAX_SLICES + 1];  // prefix of column blocks per slice
    int32_t num_slices;
    int32_t num_tokens;
    int32_t rank;
    int32_t col_blocks;   // total column blocks
    int32_t tile_tokens;  // tokens per work unit (multiple of 16)
    int32_t num_units;
    int32_t add_inputs;
};

// Host-side launchers (defined next to their kernels).
hipError_t launch_prepare(const PrepareArgs &a, hipStream_t s);
hipError_t launch_shrink(const ShrinkArgs &a, int tokens_per_tile, int waves_k, hipStream_t s);
hipError_t launch_expand(const ExpandArgs &a, hipStream_t s);

}  // namespace lora
