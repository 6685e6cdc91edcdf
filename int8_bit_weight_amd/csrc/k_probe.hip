// k_probe.hip -- a plain streaming read, the measurement floor the
// bandwidth-bound calls are compared against: every byte of a buffer read
// once with 16-byte loads, nothing computed but an XOR per workgroup (so the
// loads are not removed).  Not part of any product path.
#include "qmm_internal.h"

namespace qmm {

namespace {

__global__ __launch_bounds__(256) void k_read_probe(const v4i *__restrict__ buf, int64_t n16,
                                                    int32_t *__restrict__ sink) {
    v4i acc = {0, 0, 0, 0};
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) acc ^= buf[i];
    int v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int o = 32; o >= 1; o >>= 1) v ^= __shfl_xor(v, o);
    __shared__ int s[4];
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

}  // namespace

}  // namespace qmm

using namespace qmm;

extern "C" qmm_status qmm_read_probe(const void *buf, size_t bytes, int32_t *sink, int64_t workgroups,
                                     void *stream) {
    if (!buf || !sink || bytes % 16 != 0 || ((uintptr_t)buf % 16) != 0 || workgroups <= 0 ||
        workgroups > (1 << 20))
        return QMM_ERR_INVALID;
    if (bytes == 0) return QMM_OK;
    hipLaunchKernelGGL(k_read_probe, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                       (const v4i *)buf, (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? QMM_OK : QMM_ERR_HIP;
}
