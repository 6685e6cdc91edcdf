// k_probe.hip -- a plain streaming read (libqmm_probe.so, a measurement tool
// outside the product library): every 16-byte chunk of a buffer is read once
// and nothing is computed but an XOR per workgroup, so the loads stay.  It is
// the floor a bandwidth-bound call of the same size is compared against, and
// a read of known size for calibrating the HBM traffic counters.
//
// Each lane keeps U independent 16-byte loads in flight: a workgroup reads
// blocks of 256 * U chunks, lane t taking chunks t, t + 256, ..., t + 256 (U-1)
// of the block (every load instruction of the workgroup covers 4 KiB of
// consecutive bytes), and blocks are spread over the grid by a grid stride.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void k_read_probe(const v4i *__restrict__ buf, int64_t n16,
                                                    int32_t *__restrict__ sink) {
    v4i acc = {0, 0, 0, 0};
    const int64_t nblk = (n16 + 256 * U - 1) / (256 * U);
    for (int64_t b = blockIdx.x; b < nblk; b += gridDim.x) {
        const int64_t c0 = b * 256 * U + threadIdx.x;
        if (c0 + 256 * (U - 1) < n16) {
            // whole block: all U loads issued before any is used
            v4i v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = buf[c0 + 256 * u];
#pragma unroll
            for (int u = 0; u < U; ++u) acc ^= v[u];
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c0 + 256 * u < n16) acc ^= buf[c0 + 256 * u];
        }
    }
    int v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int o = 32; o >= 1; o >>= 1) v ^= __shfl_xor(v, o);
    __shared__ int s[4];
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

}  // namespace

extern "C" int qmm_read_probe(const void *buf, size_t bytes, int32_t *sink, int64_t workgroups, int loads_per_lane,
                              void *stream) {
    if (!buf || !sink || bytes % 16 != 0 || ((uintptr_t)buf % 16) != 0 || workgroups <= 0 ||
        workgroups > (1 << 20))
        return 1;
    if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8) return 1;
    if (bytes == 0) return 0;
    const dim3 g((unsigned)workgroups), b(256);
    const hipStream_t s = (hipStream_t)stream;
    const v4i *p = (const v4i *)buf;
    const int64_t n = (int64_t)(bytes / 16);
    switch (loads_per_lane) {
        case 1: hipLaunchKernelGGL(k_read_probe<1>, g, b, 0, s, p, n, sink); break;
        case 2: hipLaunchKernelGGL(k_read_probe<2>, g, b, 0, s, p, n, sink); break;
        case 4: hipLaunchKernelGGL(k_read_probe<4>, g, b, 0, s, p, n, sink); break;
        default: hipLaunchKernelGGL(k_read_probe<8>, g, b, 0, s, p, n, sink); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
