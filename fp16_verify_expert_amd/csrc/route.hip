// Top-k routing by the FP16 router, one workgroup per token.
//
// "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step Speculative
// Offloading" (AI summary), Key Contributions 3: routing decisions come from
// the target router; "Specter previews expert routing with an INT4 copy of the
// model itself", What shipped: the draft reuses that same FP16 router.
//
// The logit order and the selection rule live in route_core.h.
#include "route_core.h"

namespace {

constexpr int kRouteThreads = 1024;  // 16 waves; wave w takes experts w, w+16, ...

__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const uint16_t* __restrict__ wsg, int H, int E, int k, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ wout, float* __restrict__ gate) {
    __shared__ float logit[257];
    const int t = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int nvec = E + (wsg ? 1 : 0);
    // wave w takes vectors w, w + nw, ... of this token
    smoe_route::wave_logits(x + (size_t)t * H, wr, wsg, H, E, nvec, wave, nvec, nw, logit, lane);
    __syncthreads();
    if (wave != 0) return;
    smoe_route::topk_softmax_wave(logit, E, k, renorm, wsg != nullptr, lane, ids + (size_t)t * k,
                                  wout + (size_t)t * k, gate ? gate + t : nullptr, nullptr);
}

}  // namespace

namespace smoe {
hipError_t launch_route_topk(const uint16_t* x, const uint16_t* wr, const uint16_t* wsg, int T,
                             int H, int E, int k, int renorm, int32_t* ids, float* w, float* gate,
                             hipStream_t s) {
    route_topk_kernel<<<dim3(T), dim3(kRouteThreads), 0, s>>>(x, wr, wsg, H, E, k, renorm, ids,
                                                                w, gate);
    return hipGetLastError();
}
}  // namespace smoe
