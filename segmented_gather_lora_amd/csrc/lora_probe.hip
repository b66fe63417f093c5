// lora_probe.hip -- measurement aids, not part of the method: a streaming
// read of a device buffer and a launch that does nothing.  bench.py times
// them next to the hot path, on the same bytes and launch shapes, as the
// practical ceilings the kernels are compared with (how fast this part reads
// a step's bytes when nothing depends on anything, and what a launch of that
// many workgroups costs by itself).
#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // independent 16-byte loads in flight per lane

// Workgroup b reads the b-th contiguous share of the buffer, lanes on
// consecutive 16-byte pieces (every wave instruction covers 1 KB), with
// nontemporal loads.  The loaded words are folded into one value that decides
// a store, so no load can be dropped; the store happens only for a pattern
// the probe's callers never hold.
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4 *src, long n16, float *sink) {
    const long per = (n16 + gridDim.x - 1) / gridDim.x;
    const long beg = (long)blockIdx.x * per;
    const long end = beg + per < n16 ? beg + per : n16;
    uint32_t acc = 0;
    for (long i = beg + threadIdx.x; i < end; i += (long)kThreads * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const long j = i + (long)u * kThreads;
            v[u] = __builtin_nontemporal_load(src + (j < end ? j : i));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == 0x7fc00001u) sink[blockIdx.x] = 1.0f;
}

__global__ __launch_bounds__(kThreads) void probe_empty_kernel() {}

}  // namespace
}  // namespace lora

extern "C" {

int lora_probe_read(const void *src, size_t bytes, int workgroups, float *sink, hipStream_t stream) {
    if (!src || !sink) return LORA_ERR_NULL;
    if (workgroups < 1 || bytes < 16 || bytes % 16) return LORA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0) return LORA_ERR_ALIGN;
    hipLaunchKernelGGL(lora::probe_read_kernel, dim3((unsigned)workgroups), dim3(lora::kThreads), 0, stream,
                       static_cast<const lora::u32x4 *>(src), (long)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_LAUNCH;
}

int lora_probe_empty(int workgroups, hipStream_t stream) {
    if (workgroups < 1) return LORA_ERR_SHAPE;
    hipLaunchKernelGGL(lora::probe_empty_kernel, dim3((unsigned)workgroups), dim3(lora::kThreads), 0, stream);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_LAUNCH;
}

}  // extern "C"
