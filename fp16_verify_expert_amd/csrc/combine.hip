// Weighted combine of the routed experts' outputs (plus shared expert and an
// optional residual).  The pages leave this step implicit; it is the usual
// routed-MoE weighted sum.  A thread owns 8 adjacent hidden elements at a
// time (16-byte loads and stores); sums are fp32 in a fixed order (slots in
// increasing j, then the shared term, then the residual), rounded once.  The
// slots' row positions and weights are read first, 8 at a time, then their
// rows are requested together.  Without the norm epilogue a token's row is
// split over several workgroups (one chunk per thread); with it, one
// workgroup per token also writes the row RMS-normalised (the next pre-norm
// layer's input), from the rounded values.
#include "common.h"

namespace {

constexpr int kCombThreads = 256;
constexpr int kBatch = 8;  // slots whose rows are requested together

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
    const uint16_t* resid, int k, int H, uint16_t* out, uint16_t* __restrict__ norm_out,
    float eps) {
    __shared__ float red[kCombThreads / 64];
    const int t = blockIdx.x;
    const int nch = H / 8;
    float sq = 0.0f;  // sum of squares of the rounded outputs (norm_out only)
    for (int c8 = blockIdx.y * kCombThreads + threadIdx.x; c8 < nch;
         c8 += gridDim.y * kCombThreads) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < k; j0 += kBatch) {
            int r[kBatch];
            float wj[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                const int j = j0 + i;
                r[i] = (j < k) ? pp[(size_t)t * k + j] : -1;
                wj[i] = (j < k) ? w[(size_t)t * k + j] : 0.0f;
            }
            uint4 v[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                v[i] = (r[i] >= 0) ? reinterpret_cast<const uint4*>(y + (size_t)r[i] * H)[c8]
                                   : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                if (r[i] >= 0) add8(acc, v[i], wj[i]);
        }
        if (shared) {
            const float c = sscale ? sscale[t] : 1.0f;
            add8(acc, reinterpret_cast<const uint4*>(shared + (size_t)t * H)[c8], c);
        }
        if (resid) add8(acc, reinterpret_cast<const uint4*>(resid + (size_t)t * H)[c8], 1.0f);
        uint16_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            o[i] = f2h(acc[i]);
            const float r = h2f(o[i]);
            sq += r * r;
        }
        uint4 ov;
        ov.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
        ov.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
        ov.z = (uint32_t)o[4] | ((uint32_t)o[5] << 16);
        ov.w = (uint32_t)o[6] | ((uint32_t)o[7] << 16);
        reinterpret_cast<uint4*>(out + (size_t)t * H)[c8] = ov;
    }
    if (!norm_out) return;
    // row mean of squares (fixed-order tree over the block)
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) sq += __shfl_xor(sq, d);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sq;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < kCombThreads / 64; ++i) tot += red[i];
    const float inv = 1.0f / sqrtf(tot / (float)H + eps);
    for (int c8 = threadIdx.x; c8 < nch; c8 += kCombThreads) {
        const uint4 v = reinterpret_cast<const uint4*>(out + (size_t)t * H)[c8];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
        uint32_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint16_t lo = f2h(h2f((uint16_t)(u[i] & 0xFFFFu)) * inv);
            const uint16_t hi = f2h(h2f((uint16_t)(u[i] >> 16)) * inv);
            q[i] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
        reinterpret_cast<uint4*>(norm_out + (size_t)t * H)[c8] = make_uint4(q[0], q[1], q[2], q[3]);
    }
}

}  // namespace

namespace smoe {
hipError_t launch_combine(const uint16_t* y, const int32_t* pp, const float* w,
                          const uint16_t* shared, const float* sscale, const uint16_t* resid,
                          int T, int k, int H, uint16_t* out, uint16_t* norm_out, float eps,
                          hipStream_t s) {
    // the norm epilogue needs the whole row in one workgroup
    const int nch = H / 8;
    const int split = norm_out ? 1 : (nch + kCombThreads - 1) / kCombThreads;
    if (T == 0) return hipSuccess;
    combine_kernel<<<dim3(T, split), dim3(kCombThreads), 0, s>>>(y, pp, w, shared, sscale, resid,
                                                                  k, H, out, norm_out, eps);
    return hipGetLastError();
}
}  // namespace smoe
