// Fused routing plan of a decode-sized step: top-k routing, the Expert
// Lookahead Buffer update and the gather-by-expert maps in one launch.
//
// "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step Speculative
// Offloading" (AI summary), Key Contributions 3-4: the draft's expert choices
// come from the target router, are tallied in GPU counters, and the tokens are
// gathered by expert inside one fused launch.
//
// One workgroup of 1024 threads: the 16 waves share the T*(E+1) pinned-order
// dot products, then take the tokens' top-k selections, then the ELB update
// and the stable counting sort run on the ids held in LDS.  Every output is
// bit-identical to the separate routing, ELB and gather kernels (they run the
// same device routines).  One CU reads the whole router for every token, so
// beyond about one token's worth of dot products (T*(E+1)*H above 2^18) the
// plan runs as two launches instead: the routing kernel (a workgroup per
// token), then one workgroup for the ELB update and the maps (measured at the
// DeepSeek-V2-Lite shape, T = 16: 75 us in one workgroup).
#include "maps_core.h"
#include "route_core.h"

namespace {

constexpr int kPlanThreads = smoe_maps::kGatherThreads;
constexpr int kPlanWaves = kPlanThreads / 64;

__global__ __launch_bounds__(kPlanThreads) void route_plan_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const uint16_t* __restrict__ wsg, int T, int H, int E, int k, int renorm,
    int32_t* __restrict__ counters_row, int32_t* __restrict__ ids, float* __restrict__ wout,
    float* __restrict__ gate, int32_t* __restrict__ off, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, int32_t* __restrict__ err) {
    __shared__ float logit[smoe::kPlanMaxLogits];
    __shared__ int32_t ids_s[kPlanThreads];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nvec = E + (wsg ? 1 : 0);

    // 1. logits: item i = t * nvec + e, wave w takes items w, w + 16, ...
    smoe_route::wave_logits(x, wr, wsg, H, E, nvec, wave, T * nvec, kPlanWaves, logit, lane);
    __syncthreads();

    // 2. top-k and weights, wave w takes tokens w, w + 16, ...
    for (int t = wave; t < T; t += kPlanWaves)
        smoe_route::topk_softmax_wave(logit + t * nvec, E, k, renorm, wsg != nullptr, lane,
                                      ids + (size_t)t * k, wout + (size_t)t * k,
                                      gate ? gate + t : nullptr, ids_s + t * k);
    __syncthreads();

    // 3. ELB update and 4. the maps, from the ids in LDS (one token: its k
    //    ids are distinct and their sorted rows are their ranks by id)
    if (T == 1) {
        smoe_maps::one_token_maps(ids_s, k, E, counters_row, off, sorted_token, sorted_pair,
                                  pair_pos, active, n_active);
        return;
    }
    const int n = T * k;
    if (counters_row)
        smoe_maps::elb_accumulate(ids_s, n, threadIdx.x, kPlanThreads, E, counters_row, err);
    smoe_maps::gather_block(ids_s, n, k, E, off, sorted_token, sorted_pair, pair_pos, active,
                            n_active, err);
}

// The ELB update and the maps of a routed step (ids in memory).
__global__ __launch_bounds__(kPlanThreads) void plan_tail_kernel(
    const int32_t* __restrict__ ids, int n, int k, int E, int32_t* __restrict__ counters_row,
    int32_t* __restrict__ off, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, int32_t* __restrict__ err) {
    if (counters_row)
        smoe_maps::elb_accumulate(ids, n, threadIdx.x, kPlanThreads, E, counters_row, err);
    smoe_maps::gather_block(ids, n, k, E, off, sorted_token, sorted_pair, pair_pos, active,
                            n_active, err);
}

constexpr long long kPlanOneGroupElems = 1 << 18;  // T*(E+1)*H run in one workgroup

}  // namespace

namespace smoe {
hipError_t launch_route_plan(const uint16_t* x, const uint16_t* wr, const uint16_t* wsg, int T,
                             int H, int E, int k, int renorm, int layer, int32_t* counters,
                             int32_t* ids, float* w, float* gate, int32_t* off, int32_t* st,
                             int32_t* sp, int32_t* pp, int32_t* active, int32_t* n_active,
                             int32_t* err, hipStream_t s) {
    int32_t* counters_row = counters ? counters + (size_t)layer * E : nullptr;
    const int nvec = E + (wsg ? 1 : 0);
    if (T > 1 && (long long)T * nvec * H > kPlanOneGroupElems) {
        hipError_t e = launch_route_topk(x, wr, wsg, T, H, E, k, renorm, ids, w, gate, s);
        if (e != hipSuccess) return e;
        plan_tail_kernel<<<dim3(1), dim3(kPlanThreads), 0, s>>>(ids, T * k, k, E, counters_row,
                                                                 off, st, sp, pp, active,
                                                                 n_active, err);
        return hipGetLastError();
    }
    route_plan_kernel<<<dim3(1), dim3(kPlanThreads), 0, s>>>(x, wr, wsg, T, H, E, k, renorm,
                                                             counters_row, ids, w, gate, off, st,
                                                             sp, pp, active, n_active, err);
    return hipGetLastError();
}
}  // namespace smoe
