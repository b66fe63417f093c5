// lora_fused.h -- the argument block, constants and device helpers shared by
// the two one-launch shrink->expand kernels: the tile-major kernel (work
// follows the sorted segments) and the LoRA-major kernel (work follows the
// LoRA ids, so weights are read before the batch is sorted).
#pragma once

#include "lora_internal.h"

namespace lora {

struct FusedArgs {
    ShrinkArgs s;
    ExpandArgs e;
    PrepareArgs p;          // the batch's mapping and metadata outputs (PREP kernels)
    int32_t *sync;
    float *acc;             // the accumulation area (zero on entry; left zero)
    float *slots;           // the LoRA-major kernel's part slots [part][S][N][r]
    int32_t *status;
    int32_t blocks;         // expand column blocks per tile (all slices)
    int32_t block_begin[LORA_MAX_SLICES + 1];   // prefix of column blocks per slice
    int32_t help_after;     // polls without progress before a waiter takes free parts
    int32_t owners_skip;    // test only: owners leave their parts to the waiters
};

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 16;            // tokens per tile
constexpr int kBlockCols = 256;      // expand columns per unit
constexpr int kWaveCols = 64;
constexpr int kSpinLimit = 1 << 18;  // polls about 0.5 us apart: ~0.1 s
// s_waitcnt vmcnt(0) with the other counters left at their maximum
constexpr int kVmcntZero = (7 << 4) | (15 << 8);

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return lo16 | (hi16 << 16); }
__device__ __forceinline__ int clamp_group(int c, int width) { return c < width ? c : width - 4; }

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ void reset_tile(int32_t *words, int parts) {
    __hip_atomic_store(words + kFusedPartsDone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(words + kFusedPastWait, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int p = 0; p < parts; ++p) __hip_atomic_store(words + kFusedFlags + p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Batches the one-launch kernels prepare themselves: at most this many tokens.
constexpr int kPrepMaxTokens = (int)kPrepMaxTokensHost;

}  // namespace

// LoRA-major launch (lora_decode.hip): hipErrorNotSupported when the batch is
// outside its range, so the caller can take the tile-major kernel.  f.p holds
// the batch's ids, count and max_loras; with `prepare` the launch also writes
// the metadata arrays of f.p (its ids are then the raw mapping).
hipError_t launch_lora_major(const FusedArgs &f, bool prepare, hipStream_t stream);

}  // namespace lora
