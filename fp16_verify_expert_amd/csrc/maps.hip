// Expert Lookahead Buffer counters and the stable gather-by-expert maps.
//
// Cited: "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step
// Speculative Offloading" (AI summary), Key Contributions 3-4 and Methodology
// in Plain English.  The Expert Lookahead Buffer is an int32 table indexed by
// (layer, expert) in device memory; every routing choice of a draft step adds
// one to its entry.  The gather maps order a step's (token, slot) pairs by
// expert, so both the draft and the verification FFN see each expert's rows
// as one contiguous block.
//
// The device routines live in maps_core.h.
#include "maps_core.h"

namespace {

__global__ __launch_bounds__(256) void elb_count_kernel(const int32_t* __restrict__ ids, int n,
                                                        int E, int32_t* __restrict__ row,
                                                        int32_t* __restrict__ err) {
    smoe_maps::elb_accumulate(ids, n, blockIdx.x * blockDim.x + threadIdx.x,
                              gridDim.x * blockDim.x, E, row, err);
}

__global__ __launch_bounds__(smoe_maps::kGatherThreads) void gather_kernel(
    const int32_t* __restrict__ ids, int n, int k, int E, int32_t* __restrict__ off,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    int32_t* __restrict__ err) {
    smoe_maps::gather_block(ids, n, k, E, off, sorted_token, sorted_pair, pair_pos, active,
                            n_active, err);
}

// At most kGatherThreads pairs: the ids are read once into LDS and sorted
// with the per-thread counting sort (no loops over a wave's distinct ids).
__global__ __launch_bounds__(smoe_maps::kGatherThreads) void gather_small_kernel(
    const int32_t* __restrict__ ids, int n, int k, int E, int32_t* __restrict__ off,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    int32_t* __restrict__ err) {
    __shared__ int32_t ids_s[smoe_maps::kGatherThreads];
    if ((int)threadIdx.x < n) ids_s[threadIdx.x] = ids[threadIdx.x];
    __syncthreads();
    smoe_maps::small_maps(ids_s, n, k, E, nullptr, off, sorted_token, sorted_pair, pair_pos,
                          active, n_active, err);
}

}  // namespace

namespace smoe {
hipError_t launch_elb_count(const int32_t* ids, int n, int E, int layer, int32_t* counters,
                            int32_t* err, hipStream_t s) {
    int blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    elb_count_kernel<<<dim3(blocks), dim3(256), 0, s>>>(ids, n, E, counters + (size_t)layer * E,
                                                         err);
    return hipGetLastError();
}

hipError_t launch_gather(const int32_t* ids, int n, int k, int E, int32_t* off, int32_t* st,
                         int32_t* sp, int32_t* pp, int32_t* active, int32_t* n_active,
                         int32_t* err, hipStream_t s) {
    if (n <= smoe_maps::kGatherThreads)
        gather_small_kernel<<<dim3(1), dim3(smoe_maps::kGatherThreads), 0, s>>>(
            ids, n, k, E, off, st, sp, pp, active, n_active, err);
    else
        gather_kernel<<<dim3(1), dim3(smoe_maps::kGatherThreads), 0, s>>>(
            ids, n, k, E, off, st, sp, pp, active, n_active, err);
    return hipGetLastError();
}
}  // namespace smoe
