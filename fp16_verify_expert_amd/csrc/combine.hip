// Weighted combine of the routed experts' outputs (plus shared expert and an
// optional residual).  The pages leave this step implicit; it is the usual
// routed-MoE weighted sum.  One thread owns 8 adjacent hidden elements of one
// token (16-byte loads and stores); sums are fp32 in a fixed order (slots in
// increasing j, then the shared term, then the residual), rounded once.
#include "common.h"

namespace {

constexpr int kCombThreads = 256;

__device__ __forceinline__ void add8(float (&acc)[8], uint4 v, float w) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] += w * h2f((uint16_t)(u[i] & 0xFFFFu));
        acc[2 * i + 1] += w * h2f((uint16_t)(u[i] >> 16));
    }
}

__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ pp, const float* __restrict__ w,
    const uint16_t* __restrict__ shared, const float* __restrict__ sscale,
    const uint16_t* resid, int k, int H, uint16_t* out) {
    const int t = blockIdx.y;
    const int c8 = blockIdx.x * kCombThreads + threadIdx.x;  // 8-element chunk
    if (c8 * 8 >= H) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const int r = pp[(size_t)t * k + j];
        if (r < 0) continue;
        const uint4 v = reinterpret_cast<const uint4*>(y + (size_t)r * H)[c8];
        add8(acc, v, w[(size_t)t * k + j]);
    }
    if (shared) {
        const float c = sscale ? sscale[t] : 1.0f;
        add8(acc, reinterpret_cast<const uint4*>(shared + (size_t)t * H)[c8], c);
    }
    if (resid) add8(acc, reinterpret_cast<const uint4*>(resid + (size_t)t * H)[c8], 1.0f);
    uint4 o;
    o.x = (uint32_t)f2h(acc[0]) | ((uint32_t)f2h(acc[1]) << 16);
    o.y = (uint32_t)f2h(acc[2]) | ((uint32_t)f2h(acc[3]) << 16);
    o.z = (uint32_t)f2h(acc[4]) | ((uint32_t)f2h(acc[5]) << 16);
    o.w = (uint32_t)f2h(acc[6]) | ((uint32_t)f2h(acc[7]) << 16);
    reinterpret_cast<uint4*>(out + (size_t)t * H)[c8] = o;
}

}  // namespace

namespace smoe {
hipError_t launch_combine(const uint16_t* y, const int32_t* pp, const float* w,
                          const uint16_t* shared, const float* sscale, const uint16_t* resid,
                          int T, int k, int H, uint16_t* out, hipStream_t s) {
    const int chunks = H / 8;
    const dim3 grid((chunks + kCombThreads - 1) / kCombThreads, T);
    combine_kernel<<<grid, dim3(kCombThreads), 0, s>>>(y, pp, w, shared, sscale, resid, k, H, out);
    return hipGetLastError();
}
}  // namespace smoe
