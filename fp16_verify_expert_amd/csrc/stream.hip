// Streaming read of a device buffer: the memory-bound ceiling the weight
// streaming kernels are measured against.  Every workgroup walks the buffer
// grid-stride with the same 16-byte non-temporal loads those kernels use and
// writes the XOR of the words it read (a checksum, so the loads are kept).
#include "common.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          size_t n16, uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    __shared__ uint32_t part[256];
    part[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < 64) {
        uint32_t a = part[threadIdx.x] ^ part[threadIdx.x + 64] ^ part[threadIdx.x + 128] ^
                     part[threadIdx.x + 192];
        for (int d = 32; d >= 1; d >>= 1) a ^= __shfl_xor(a, d);
        if (threadIdx.x == 0) sink[blockIdx.x] = a;
    }
}

}  // namespace

namespace smoe {
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                              hipStream_t s) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const u32x4*>(src), bytes / 16, sink);
    return hipGetLastError();
}
}  // namespace smoe
