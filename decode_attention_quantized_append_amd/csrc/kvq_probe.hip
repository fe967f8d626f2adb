// kvq_probe.hip -- libkvq_probe.so: a plain streaming read of a device
// buffer, for measuring the read bandwidth this device actually sustains.
// The benchmark reports the decode's bandwidth both against the nominal HBM
// peak and against this measured ceiling.  It is measurement tooling, not
// part of the append / decode path, and libkvq does not use it.
//
// Each thread reads U 16-byte pieces per pass, U passes apart by the grid's
// total thread count (all U loads in flight together), and folds what it
// read into an XOR so that the loads cannot be dropped; each wave stores one
// word.  The buffer must be 16-byte aligned and a multiple of 16 bytes.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

template <int U>
__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ src, uint64_t n16, uint32_t* sink) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) v[k] = src[i + k * stride];
#pragma unroll
        for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
    if ((threadIdx.x & 63) == 0) sink[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = acc;
}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 16) from buf with `blocks` workgroups of 256
// threads, `unroll` (1, 2, 4 or 8) loads in flight per thread; sink receives
// blocks * 4 words.  Returns 0, or -1 on bad arguments / a failed launch.
int kvq_probe_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, int blocks, int unroll, void* stream) {
    if (!buf || !sink || blocks < 1 || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15)) return -1;
    const hipStream_t st = (hipStream_t)stream;
    const uint4* src = static_cast<const uint4*>(buf);
    const uint64_t n16 = bytes / 16;
    switch (unroll) {
        case 1: hipLaunchKernelGGL(stream_read<1>, dim3(blocks), dim3(256), 0, st, src, n16, sink); break;
        case 2: hipLaunchKernelGGL(stream_read<2>, dim3(blocks), dim3(256), 0, st, src, n16, sink); break;
        case 4: hipLaunchKernelGGL(stream_read<4>, dim3(blocks), dim3(256), 0, st, src, n16, sink); break;
        case 8: hipLaunchKernelGGL(stream_read<8>, dim3(blocks), dim3(256), 0, st, src, n16, sink); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
