// Weighted combine of the routed experts' outputs (plus shared expert and an
// optional residual): the combine_core.h routines as launches of their own.
// Without the norm epilogue a token's row is split over several workgroups
// (one chunk per thread); with it, one workgroup per token also writes the
// row RMS-normalised (the next pre-norm layer's input), from the rounded
// values.
#include "combine_core.h"
#include "route_core.h"

namespace {

using namespace smoe_comb;

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
// Each wave first requests its router row (it does not depend on the combine),
// then evaluates the combine and the norm, then its logit against the row.
template <int CPL>
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
    const int wave = blockIdx.x * (kCombThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    uint4 wv[CPL];
    const bool has = wave < nvec;  // one logit per wave (the grid covers nvec)
    smoe_route::pinned_row<CPL>(has ? (wave < E ? wr + (size_t)wave * H : wsg) : wr, H, lane, wv);
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
    if (has) {
        const float s = smoe_route::pinned_dot_regs<CPL>(xs, wv, H, lane);
        if (lane == 0) lg[wave] = s;
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

bool combine_logits_supported(int H) { return H <= kMaxFusedH; }

hipError_t launch_combine_logits(const uint16_t* y, const int32_t* pp, const float* w,
                                 const uint16_t* shared, const float* sscale,
                                 const uint16_t* resid, int k, int H, uint16_t* out,
                                 uint16_t* norm_out, float eps, const uint16_t* wr,
                                 const uint16_t* wsg, int E, float* lg, hipStream_t s) {
    const int nvec = E + (wsg ? 1 : 0);
    const int wg = (nvec + kCombThreads / 64 - 1) / (kCombThreads / 64);
    const int cpl = (H / 8 + 63) / 64;  // chunks per lane of a row (H <= 8192: <= 16)
#define SMOE_CL(C) combine_logits_kernel<C><<<dim3(wg), dim3(kCombThreads), 0, s>>>( \
        y, pp, w, shared, sscale, resid, k, H, out, norm_out, eps, wr, wsg, E, nvec, lg)
    if (cpl <= 4) SMOE_CL(4);
    else if (cpl <= 8) SMOE_CL(8);
    else SMOE_CL(16);
#undef SMOE_CL
    return hipGetLastError();
}
}  // namespace smoe
