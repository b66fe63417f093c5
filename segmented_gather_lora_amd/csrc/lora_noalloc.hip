// lora_noalloc.hip -- lora_shrink_expand for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc): the fp32 buffer between the shrink and the expand
// lives in a file-scope device array of the library instead of a caller
// argument.  Each GPU the library runs on holds its own copy of the array
// until the process ends.
#include <mutex>

#include "lora_internal.h"

namespace {

// 32 MiB: S * N * rank floats of one call (the large shape, 3 x 16384 x 128,
// takes 24 MiB).
constexpr size_t kScratchFloats = (size_t)8 << 20;
static __device__ __align__(256) float scratch[kScratchFloats];

// The array's address on each device, taken once per device with that device
// current (in host code the name `scratch` is only a stand-in for the symbol,
// not a device address).
constexpr int kMaxDevices = 64;
std::mutex g_mu;
float *g_scratch[kMaxDevices];

int scratch_on_current_device(float **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LORA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LORA_ERR_LAUNCH;
        g_scratch[dev] = static_cast<float *>(p);
    }
    *out = g_scratch[dev];
    return LORA_OK;
}

}  // namespace

extern "C" int lora_shrink_expand_noalloc(const void *x, int64_t ldx, int num_tokens, int hidden,
                                          const void *const *lora_a, const void *const *lora_b,
                                          const void *const *bias, const int *slice_widths, int num_slices,
                                          int rank, void *y, int64_t ldy, int offset_start, int add_inputs,
                                          const lora_meta_t *meta, float scale, hipStream_t stream) {
    if (num_slices < 1 || num_slices > LORA_MAX_SLICES) return LORA_ERR_SLICES;
    if (rank < 8 || rank > LORA_MAX_RANK || rank % 8) return LORA_ERR_SHAPE;
    if (num_tokens < 0) return LORA_ERR_NUM_TOKENS;
    if ((size_t)num_slices * (size_t)num_tokens * (size_t)rank > kScratchFloats) return LORA_ERR_SCRATCH;
    float *buf = nullptr;
    const int st = scratch_on_current_device(&buf);
    if (st) return st;
    // the buffer is written as a fresh one: whatever an earlier call left in
    // the array does not matter, and nothing in it needs clearing
    return lora_shrink_expand(x, ldx, num_tokens, hidden, lora_a, lora_b, bias, slice_widths, num_slices, rank, buf,
                              y, ldy, offset_start, add_inputs, meta, scale, stream);
}
