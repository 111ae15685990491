// Streaming-read probe for bench.py: the HBM read rate a plain kernel reaches
// on this chip, recorded beside the attention kernels' rates as their practical
// ceiling (the nominal 8 TB/s is not reachable by reads alone).
//
// Each work group of 256 threads reads one contiguous slice of the buffer with
// 16-byte loads, four in flight per thread, plain or non-temporal (the load the
// attention kernels use for K and V), and folds the words into one value that
// is stored only if it matches a constant (so the loads are not removed and
// nothing is written in practice). Measurement only: not part of the library.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *p, int64_t n16_per_block, uint32_t *sink) {
    const u32x4 *base = p + blockIdx.x * n16_per_block;
    uint32_t acc = 0;
    for (int64_t i = threadIdx.x; i < n16_per_block; i += 256 * 4) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = i + u * 256;
            if (j < n16_per_block) v[u] = NT ? __builtin_nontemporal_load(base + j) : base[j];
            else v[u] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16 * blocks) from device memory `p` once with
// `blocks` work groups on `stream`; `sink` is device memory of at least
// blocks * 256 words (almost never written). nt != 0: non-temporal loads.
// Returns 0, or a HIP error code.
int probe_stream_read(const void *p, int64_t bytes, int blocks, int nt, void *sink, void *stream) {
    if (p == nullptr || sink == nullptr || blocks <= 0 || bytes <= 0 || bytes % (16LL * blocks) != 0)
        return (int)hipErrorInvalidValue;
    const int64_t per = bytes / 16 / blocks;
    if (nt)
        hipLaunchKernelGGL(stream_read_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                           (const u32x4 *)p, per, (uint32_t *)sink);
    else
        hipLaunchKernelGGL(stream_read_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                           (const u32x4 *)p, per, (uint32_t *)sink);
    return (int)hipGetLastError();
}

}  // extern "C"
