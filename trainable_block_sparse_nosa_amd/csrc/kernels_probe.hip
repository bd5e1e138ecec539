// Streaming-read probe: the achievable HBM read bandwidth on this part, the
// second denominator (besides the 8 TB/s peak) for the HBM-bound kernels.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace nosa {

constexpr int PROBE_THREADS = 256, PROBE_UNROLL = 8;

// Every 16-byte vector of src once: eight loads in flight per thread, a
// grid-stride loop over chunks of 256 * 8 vectors, each load instruction of a
// wave 1 KiB of whole cache lines, non-temporal (streamed once, not kept in
// the caches: 7.1 TB/s on a 2 GiB buffer, against 6.35 with cached loads).
// What was read is folded into one word per thread; the (practically never
// taken) store on a magic value keeps the loads without a write per thread.
__global__ void __launch_bounds__(PROBE_THREADS)
read_probe_kernel(const u32x4 *__restrict__ src, int64_t n_vec, uint32_t *__restrict__ sink) {
    uint32_t acc = 0u;
    const int64_t chunk = (int64_t)PROBE_THREADS * PROBE_UNROLL;
    for (int64_t base = (int64_t)blockIdx.x * chunk + threadIdx.x; base < n_vec;
         base += (int64_t)gridDim.x * chunk) {
        u32x4 v[PROBE_UNROLL];
#pragma unroll
        for (int j = 0; j < PROBE_UNROLL; ++j) {
            const int64_t i = base + (int64_t)j * PROBE_THREADS;
            v[j] = i < n_vec ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < PROBE_UNROLL; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, int wgs,
                             hipStream_t st) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(wgs), dim3(PROBE_THREADS), 0, st,
                       static_cast<const u32x4 *>(src), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace nosa
