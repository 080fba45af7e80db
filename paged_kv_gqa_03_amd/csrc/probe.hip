// probe.hip -- pure-read HBM streaming probe: the measured ceiling that the
// decode kernels' achieved bandwidth is compared against.
//
// Every 16-byte word of the buffer is read exactly once with a non-temporal
// load.  The grid sweeps the buffer front to back: each pass of the grid
// reads one contiguous block of workgroups x 256 x 16 bytes (lane-consecutive
// words, workgroup-consecutive 4 KB blocks), eight such blocks in flight per
// thread.  Of the shapes swept on MI355X (grid-stride or one contiguous chunk
// per workgroup or per wave, 1 to 16 workgroups per CU, 4 to 32 loads in
// flight) this one read fastest at 1.26 GB (7.1 TB/s, one workgroup per
// CU).  Each wave leaves the XOR of the words it read in `sink`, so no load
// can be dropped and a test can check that every word was read once.
#include "device_common.hpp"
#include "kernels.hpp"

namespace pa {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p, uint64_t n16,
                                                          uint32_t *__restrict__ sink) {
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    // XOR over the wave, then one 16-byte store per wave.
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        acc.x ^= (uint32_t)__shfl_xor((int)acc.x, m);
        acc.y ^= (uint32_t)__shfl_xor((int)acc.y, m);
        acc.z ^= (uint32_t)__shfl_xor((int)acc.z, m);
        acc.w ^= (uint32_t)__shfl_xor((int)acc.w, m);
    }
    if ((threadIdx.x & 63) == 0)
        *reinterpret_cast<u32x4 *>(sink + ((uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4) = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *buf, uint64_t bytes, uint32_t *sink, int workgroups,
                              hipStream_t stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace pa
