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
#include "route_core.h"

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

// fp32 sums of one 8-element chunk c8 of token t's output, in the fixed
// order: slots j = 0..k-1 (pairs with pair_pos -1 skipped), then the shared
// term, then the residual.  The slots' row positions and weights are read
// kBatch at a time, then their rows are requested together.
__device__ __forceinline__ void combine_chunk(const uint16_t* __restrict__ y,
                                              const int32_t* __restrict__ pp,
                                              const float* __restrict__ w,
                                              const uint16_t* __restrict__ shared,
                                              const float* __restrict__ sscale,
                                              const uint16_t* resid, int t, int k, int H, int c8,
                                              float (&acc)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
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
}

// The chunk rounded to fp16 (packed), with the sum of squares of the rounded
// values added to sq.
__device__ __forceinline__ uint4 round_chunk(const float (&acc)[8], float& sq) {
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
    return ov;
}

// 1 / sqrt(mean of squares + eps) of a row whose per-thread partial sums of
// squares are sq (a workgroup of kCombThreads threads): a butterfly inside
// each wave, then the waves' sums in wave order.  Ends after a barrier.
__device__ __forceinline__ float row_inv_rms(float sq, int H, float eps, float* red) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) sq += __shfl_xor(sq, d);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sq;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < kCombThreads / 64; ++i) tot += red[i];
    return 1.0f / sqrtf(tot / (float)H + eps);
}

// A chunk of the rounded row scaled by inv, rounded to fp16 again.
__device__ __forceinline__ uint4 norm_chunk(uint4 v, float inv) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    uint32_t q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint16_t lo = f2h(h2f((uint16_t)(u[i] & 0xFFFFu)) * inv);
        const uint16_t hi = f2h(h2f((uint16_t)(u[i] >> 16)) * inv);
        q[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    return make_uint4(q[0], q[1], q[2], q[3]);
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
        float acc[8];
        combine_chunk(y, pp, w, shared, sscale, resid, t, k, H, c8, acc);
        reinterpret_cast<uint4*>(out + (size_t)t * H)[c8] = round_chunk(acc, sq);
    }
    if (!norm_out) return;
    const float inv = row_inv_rms(sq, H, eps, red);
    for (int c8 = threadIdx.x; c8 < nch; c8 += kCombThreads) {
        const uint4 v = reinterpret_cast<const uint4*>(out + (size_t)t * H)[c8];
        reinterpret_cast<uint4*>(norm_out + (size_t)t * H)[c8] = norm_chunk(v, inv);
    }
}

// One token: moe_combine of a layer's outputs (with the norm epilogue), then
// the next layer's router logits (and shared-gate logit) of the normalised
// row, one per wave in the pinned order of the routing kernels.  Every
// workgroup evaluates the combine itself (the row is a few KB, read from
// L2), keeps the normalised row in LDS for its waves' dot products, and
// workgroup 0 writes out and norm_out.  The same routines as combine_kernel
// and the routing kernels, so every value is bit-identical to those calls.
constexpr int kMaxFusedH = 8192;
__global__ __launch_bounds__(kCombThreads) void combine_logits_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ pp, const float* __restrict__ w,
    const uint16_t* __restrict__ shared, const float* __restrict__ sscale,
    const uint16_t* resid, int k, int H, uint16_t* out, uint16_t* __restrict__ norm_out,
    float eps, const uint16_t* __restrict__ wr, const uint16_t* __restrict__ wsg, int E,
    int nvec, float* __restrict__ lg) {
    __shared__ float red[kCombThreads / 64];
    __shared__ uint4 xs[kMaxFusedH / 8];
    const int nch = H / 8;
    const bool writer = blockIdx.x == 0;
    float sq = 0.0f;
    for (int c8 = threadIdx.x; c8 < nch; c8 += kCombThreads) {
        float acc[8];
        combine_chunk(y, pp, w, shared, sscale, resid, 0, k, H, c8, acc);
        const uint4 ov = round_chunk(acc, sq);
        xs[c8] = ov;
        if (writer) reinterpret_cast<uint4*>(out)[c8] = ov;
    }
    const float inv = row_inv_rms(sq, H, eps, red);
    for (int c8 = threadIdx.x; c8 < nch; c8 += kCombThreads) {
        const uint4 q = norm_chunk(xs[c8], inv);
        xs[c8] = q;
        if (writer) reinterpret_cast<uint4*>(norm_out)[c8] = q;
    }
    __syncthreads();
    const int wave = blockIdx.x * (kCombThreads / 64) + (threadIdx.x >> 6);
    smoe_route::wave_logits(reinterpret_cast<const uint16_t*>(xs), wr, wsg, H, E, nvec, wave,
                            nvec, gridDim.x * (kCombThreads / 64), lg, threadIdx.x & 63);
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

bool combine_logits_supported(int H) { return H <= kMaxFusedH; }

hipError_t launch_combine_logits(const uint16_t* y, const int32_t* pp, const float* w,
                                 const uint16_t* shared, const float* sscale,
                                 const uint16_t* resid, int k, int H, uint16_t* out,
                                 uint16_t* norm_out, float eps, const uint16_t* wr,
                                 const uint16_t* wsg, int E, float* lg, hipStream_t s) {
    const int nvec = E + (wsg ? 1 : 0);
    const int wg = (nvec + kCombThreads / 64 - 1) / (kCombThreads / 64);
    combine_logits_kernel<<<dim3(wg), dim3(kCombThreads), 0, s>>>(
        y, pp, w, shared, sscale, resid, k, H, out, norm_out, eps, wr, wsg, E, nvec, lg);
    return hipGetLastError();
}
}  // namespace smoe
