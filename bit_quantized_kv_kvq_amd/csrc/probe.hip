// probe.hip -- streaming-read probe: the bandwidth a plain read of device memory
// reaches on this device, the achievable ceiling beside the HBM peak for
// kernels that stream their input once.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kProbeDepth = 8;  // 16-byte loads in flight per thread

// Reads n16 16-byte words once (grid-strided, kProbeDepth loads in flight per
// thread) and folds them with XOR.  The fold is written only if it equals a
// fixed word, so the loads stay live without a write stream.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                          unsigned* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (; i + (kProbeDepth - 1) * stride < n16; i += kProbeDepth * stride) {
        uint4 v[kProbeDepth];
#pragma unroll
        for (int u = 0; u < kProbeDepth; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < kProbeDepth; ++u) {
            acc.x ^= v[u].x;
            acc.y ^= v[u].y;
            acc.z ^= v[u].z;
            acc.w ^= v[u].w;
        }
    }
    for (; i < n16; i += stride) {
        const uint4 v = p[i];
        acc.x ^= v.x;
        acc.y ^= v.y;
        acc.z ^= v.z;
        acc.w ^= v.w;
    }
    const unsigned r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == 0x9E3779B9u) *sink = r;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t n16, int blocks, unsigned* sink, hipStream_t stream) {
    stream_read_kernel<<<blocks, 256, 0, stream>>>(static_cast<const uint4*>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace kvq
