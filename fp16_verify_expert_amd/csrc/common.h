// Internal helpers shared by the gfx950 kernels of libsmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smoe.h"

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

#define SMOE_DEV __device__ __forceinline__

SMOE_DEV float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
SMOE_DEV uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }  // RNE

// Pointers read from descriptor tables are generic; casting them to the
// global address space lets the compiler use global (not flat) loads.
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;
template <typename T>
SMOE_DEV gptr<T> as_global(const T* p) {
    return (gptr<T>)p;
}

SMOE_DEV void flag_error(int32_t* err, int32_t bit) {
    if (err) atomicOr(err, bit);
}

// Device-scope (agent) accesses: coherent across the XCDs' separate L2
// caches, for values one workgroup hands to another inside a launch.
template <typename T>
SMOE_DEV void st_dev(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
SMOE_DEV T ld_dev(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
SMOE_DEV uint4 ld_dev4(const void* p) {
    const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
    const uint64_t a = ld_dev(q), b = ld_dev(q + 1);
    return make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
}

// Number of sorted rows in [0, rows) that belong to expert slot bounds.
struct RowRange {
    int r0, r1;
};

// Launchers (one per kernel family), defined next to their kernels.
namespace smoe {
hipError_t launch_route_topk(const uint16_t* x, const uint16_t* wr, const uint16_t* wsg, int T,
                             int H, int E, int k, int renorm, int32_t* ids, float* w, float* gate,
                             hipStream_t s);
// Fused route + ELB + gather (one workgroup): limits on T*k and on the
// logits held in LDS.
constexpr int kPlanMaxPairs = 1024;
constexpr int kPlanMaxLogits = 4096;
hipError_t launch_route_plan(const uint16_t* x, const uint16_t* wr, const uint16_t* wsg, int T,
                             int H, int E, int k, int renorm, int layer, int32_t* counters,
                             int32_t* ids, float* w, float* gate, int32_t* off, int32_t* st,
                             int32_t* sp, int32_t* pp, int32_t* active, int32_t* n_active,
                             int32_t* err, float* lg, hipStream_t s);
hipError_t launch_elb_count(const int32_t* ids, int n, int E, int layer, int32_t* counters,
                            int32_t* err, hipStream_t s);
hipError_t launch_gather(const int32_t* ids, int n, int k, int E, int32_t* off, int32_t* st,
                         int32_t* sp, int32_t* pp, int32_t* active, int32_t* n_active,
                         int32_t* err, hipStream_t s);
int device_cu_count();
// The one-launch draft layer (T = 1): routing, routed INT4 FFN, optional
// FP16 shared expert, combine and the next layer's logits.
struct DraftLayerCall {
    const uint16_t* x;
    const uint16_t* wr;
    const uint16_t* wsg;
    const float* logits;
    int H, I, E, k, renorm;
    int32_t* counters_row;
    int32_t* ids;
    float* w;
    float* gate;
    int32_t* off;
    int32_t* st;
    int32_t* sp;
    int32_t* pp;
    int32_t* active;
    int32_t* n_active;
    const smoe_w4_expert* experts;
    uint16_t* y;
    const uint16_t* sw13;
    const uint16_t* sw2;
    int Is;
    uint16_t* sh_h;
    uint16_t* sh_out;
    const uint16_t* resid;
    uint16_t* out;
    uint16_t* norm_out;
    float eps;
    const uint16_t* wr_next;
    const uint16_t* wsg_next;
    int E_next;
    float* lg_next;
    void* ws;
    int32_t* err;
};
bool draft_layer_supported(int H, int I, int E, int k, int Is);
size_t draft_layer_workspace_bytes(int k, int I, int E);
hipError_t launch_draft_layer(const DraftLayerCall& c, hipStream_t s);
hipError_t launch_w4a16_ffn(const uint16_t* x, const int32_t* sorted_token, const int32_t* off,
                            const int32_t* active, const int32_t* n_active,
                            const smoe_w4_expert* experts, int T, int k, int H, int I, int E,
                            int bits, uint16_t* y, void* ws, int32_t* err, hipStream_t s,
                            const uint16_t* const* ascale = nullptr);
size_t w4a16_workspace_bytes(int T, int k, int H, int I, int E);
// w4a16_grouped_ffn (4-bit) and a dense FP16 shared expert over all T rows,
// the shared columns inside the multi-row launches where they fit
hipError_t launch_w4a16_ffn_shared(const uint16_t* x, const int32_t* sorted_token,
                                   const int32_t* off, const int32_t* active,
                                   const int32_t* n_active, const smoe_w4_expert* experts, int T,
                                   int k, int H, int I, int E, uint16_t* y, void* ws,
                                   const uint16_t* sw13, const uint16_t* sw2, int Is,
                                   uint16_t* sh_h, uint16_t* sh_out, int32_t* err,
                                   hipStream_t s);
// Waves per workgroup of the one-group (shared expert) ring launches, gate/up
// and down; each wave takes a contiguous range of the 128-K steps.
#ifndef SMOE_SH_GU_WAVES
#define SMOE_SH_GU_WAVES 2
#endif
#ifndef SMOE_SH_DN_WAVES
#define SMOE_SH_DN_WAVES 4
#endif
// the dense shared expert alone as verify_grouped_gemm's one-group ring
// launches over token rows 0..T-1 of x
hipError_t launch_dense_group(const uint16_t* x, int T, int H, const uint16_t* w13,
                              const uint16_t* w2, int Is, uint16_t* sh_h, uint16_t* sh_out,
                              int32_t* err, hipStream_t s);
// One-token draft step: the router logits, then routing, ELB, maps and the
// gate/up projection in one launch, then the down projection; an optional
// dense shared expert (sw13 non-null) computed in the same two launches.
bool draft_route_ffn_supported(int E, int k);
hipError_t launch_draft_route_ffn(const uint16_t* x, const uint16_t* wr, const uint16_t* wsg,
                                  int H, int E, int k, int renorm, int32_t* counters_row,
                                  int32_t* ids, float* w, float* gate, int32_t* off, int32_t* st,
                                  int32_t* sp, int32_t* pp, int32_t* active, int32_t* n_active,
                                  const smoe_w4_expert* experts, int I, uint16_t* y, void* ws,
                                  const uint16_t* sw13, const uint16_t* sw2, int Is,
                                  uint16_t* sh_h, uint16_t* sh_out, const float* logits_in,
                                  int32_t* err, hipStream_t s);
bool w4a16_shape_supported(int H, int I);
hipError_t launch_verify_ffn(const uint16_t* x, const int32_t* sorted_token, const int32_t* off,
                             const int32_t* active, const int32_t* n_active,
                             const smoe_f16_expert* experts, const uint8_t* mask, int T, int rows,
                             int H, int I, int E, uint16_t* y, void* ws, int32_t* err,
                             hipStream_t s);
hipError_t launch_verify_ffn_shared(const uint16_t* x, const int32_t* sorted_token,
                                    const int32_t* off, const int32_t* active,
                                    const int32_t* n_active, const smoe_f16_expert* experts,
                                    const uint8_t* mask, int T, int rows, int H, int I, int E,
                                    uint16_t* y, void* ws, const uint16_t* sw13,
                                    const uint16_t* sw2, int Is, uint16_t* sh_h,
                                    uint16_t* sh_out, int32_t* err, hipStream_t s);
size_t verify_workspace_bytes(int T, int rows, int H, int I, int E);
// dense regime of the verify FFN (many rows per expert)
size_t dense_plan_bytes(int E);
hipError_t launch_dense_ffn(const uint16_t* x, const int32_t* sorted_token, const int32_t* off,
                            const int32_t* active, const int32_t* n_active,
                            const smoe_f16_expert* experts, const uint8_t* mask, int rows, int H,
                            int I, int E, uint16_t* y, uint16_t* h, int32_t* plan, int32_t* err,
                            hipStream_t s);
hipError_t launch_combine(const uint16_t* y, const int32_t* pp, const float* w,
                          const uint16_t* shared, const float* sscale, const uint16_t* resid,
                          int T, int k, int H, uint16_t* out, uint16_t* norm_out, float eps,
                          hipStream_t s);
bool combine_logits_supported(int H);
hipError_t launch_combine_logits(const uint16_t* y, const int32_t* pp, const float* w,
                                 const uint16_t* shared, const float* sscale,
                                 const uint16_t* resid, int k, int H, uint16_t* out,
                                 uint16_t* norm_out, float eps, const uint16_t* wr,
                                 const uint16_t* wsg, int E, float* lg, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                              hipStream_t s);
}  // namespace smoe
