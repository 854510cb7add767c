// Fused routing plan of a decode-sized step: top-k routing, the Expert
// Lookahead Buffer update and the gather-by-expert maps.
//
// "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step Speculative
// Offloading" (AI summary), Key Contributions 3-4: the draft's expert choices
// come from the target router, are tallied in GPU counters, and the tokens are
// gathered by expert inside one fused launch.
//
// Small plans run in one workgroup of 1024 threads: the 16 waves share the
// T*(E+1) pinned-order dot products, then take the tokens' top-k selections,
// then the ELB update and the stable counting sort run on the ids held in
// LDS.  Every output is bit-identical to the separate routing, ELB and gather
// kernels (they run the same device routines).  That one CU reads the whole
// router for every token, and one CU keeps too few reads in flight to stream
// it (about 22 GB/s: 12 us for the 256 KB router of hidden 2048 and 64
// experts), so larger plans (T*(E+1)*H above 2^16) run as two launches when
// the caller gives a logits buffer: every (token, router row) dot product on
// a wave of its own across the chip, then one workgroup that takes the top k,
// the ELB update and the maps from those logits.  Without the buffer, plans
// above 2^18 run the routing kernel (a workgroup per token) and then one
// workgroup for the ELB update and the maps (at the DeepSeek-V2-Lite shape,
// T = 16, the single workgroup took 75 us).
#include "maps_core.h"
#include "route_core.h"

namespace {

constexpr int kPlanThreads = smoe_maps::kGatherThreads;
constexpr int kPlanWaves = kPlanThreads / 64;

// Steps 2-4 of a plan from the T*nvec logits in LDS (all threads of the
// workgroup call it; ids_s is LDS of kPlanThreads ids).
SMOE_DEV void plan_from_logits(const float* logit, int32_t* ids_s, int T, int E, int k,
                               int renorm, bool has_gate, int32_t* __restrict__ counters_row,
                               int32_t* __restrict__ ids, float* __restrict__ wout,
                               float* __restrict__ gate, int32_t* __restrict__ off,
                               int32_t* __restrict__ sorted_token,
                               int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
                               int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                               int32_t* __restrict__ err) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nvec = E + (has_gate ? 1 : 0);

    // 2. top-k and weights, wave w takes tokens w, w + 16, ...
    for (int t = wave; t < T; t += kPlanWaves)
        smoe_route::topk_softmax_wave(logit + t * nvec, E, k, renorm, has_gate, lane,
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
    smoe_maps::small_maps<true>(ids_s, T * k, k, E, counters_row, off, sorted_token,
                                sorted_pair, pair_pos, active, n_active, err);
}

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
    plan_from_logits(logit, ids_s, T, E, k, renorm, wsg != nullptr, counters_row, ids, wout, gate,
                     off, sorted_token, sorted_pair, pair_pos, active, n_active, err);
}

// Step 1 spread over the chip: item i = t * nvec + e on wave i of the grid,
// its logit into lg[i].
constexpr int kLogitThreads = 256;
__global__ __launch_bounds__(kLogitThreads) void plan_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const uint16_t* __restrict__ wsg, int T, int H, int E, int nvec, float* __restrict__ lg) {
    const int wave = blockIdx.x * (kLogitThreads / 64) + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * (kLogitThreads / 64);
    smoe_route::wave_logits(x, wr, wsg, H, E, nvec, wave, T * nvec, nwaves, lg, threadIdx.x & 63);
}

// Steps 2-4 from the logits plan_logits_kernel wrote.
__global__ __launch_bounds__(kPlanThreads) void plan_topk_kernel(
    const float* __restrict__ lg, int T, int E, int k, int renorm, int has_gate,
    int32_t* __restrict__ counters_row, int32_t* __restrict__ ids, float* __restrict__ wout,
    float* __restrict__ gate, int32_t* __restrict__ off, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, int32_t* __restrict__ err) {
    __shared__ float logit[smoe::kPlanMaxLogits];
    __shared__ int32_t ids_s[kPlanThreads];
    const int nl = T * (E + (has_gate ? 1 : 0));
    for (int i = threadIdx.x; i < nl; i += kPlanThreads) logit[i] = lg[i];
    __syncthreads();
    plan_from_logits(logit, ids_s, T, E, k, renorm, has_gate != 0, counters_row, ids, wout, gate,
                     off, sorted_token, sorted_pair, pair_pos, active, n_active, err);
}

// The ELB update and the maps of a routed step (n <= kPlanThreads ids in
// memory, read once into LDS).
__global__ __launch_bounds__(kPlanThreads) void plan_tail_kernel(
    const int32_t* __restrict__ ids, int n, int k, int E, int32_t* __restrict__ counters_row,
    int32_t* __restrict__ off, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, int32_t* __restrict__ err) {
    __shared__ int32_t ids_s[kPlanThreads];
    if ((int)threadIdx.x < n) ids_s[threadIdx.x] = ids[threadIdx.x];
    __syncthreads();
    smoe_maps::small_maps<true>(ids_s, n, k, E, counters_row, off, sorted_token, sorted_pair,
                                pair_pos, active, n_active, err);
}

#ifndef SMOE_PLAN_SPREAD_ELEMS
#define SMOE_PLAN_SPREAD_ELEMS (1 << 16)
#endif
constexpr long long kPlanSpreadElems = SMOE_PLAN_SPREAD_ELEMS;  // T*(E+1)*H above: spread logits
constexpr long long kPlanOneGroupElems = 1 << 18;  // without a logits buffer

}  // namespace

namespace smoe {
hipError_t launch_route_plan(const uint16_t* x, const uint16_t* wr, const uint16_t* wsg, int T,
                             int H, int E, int k, int renorm, int layer, int32_t* counters,
                             int32_t* ids, float* w, float* gate, int32_t* off, int32_t* st,
                             int32_t* sp, int32_t* pp, int32_t* active, int32_t* n_active,
                             int32_t* err, float* lg, hipStream_t s) {
    int32_t* counters_row = counters ? counters + (size_t)layer * E : nullptr;
    const int nvec = E + (wsg ? 1 : 0);
    const long long elems = (long long)T * nvec * H;
    if (lg && T > 0 && elems > kPlanSpreadElems) {
        const int items = T * nvec;
        const int wgs = (items + kLogitThreads / 64 - 1) / (kLogitThreads / 64);
        plan_logits_kernel<<<dim3(wgs), dim3(kLogitThreads), 0, s>>>(x, wr, wsg, T, H, E, nvec,
                                                                     lg);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        plan_topk_kernel<<<dim3(1), dim3(kPlanThreads), 0, s>>>(
            lg, T, E, k, renorm, wsg ? 1 : 0, counters_row, ids, w, gate, off, st, sp, pp, active,
            n_active, err);
        return hipGetLastError();
    }
    if (T > 1 && elems > kPlanOneGroupElems) {
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
