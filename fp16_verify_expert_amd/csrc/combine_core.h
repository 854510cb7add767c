// Device routines of the weighted combine (plus shared expert and an
// optional residual), shared by the combine kernels and the one-launch draft
// layer so that every value they produce is bit-identical.  The pages leave
// this step implicit; it is the usual routed-MoE weighted sum.  A thread owns
// 8 adjacent hidden elements at a time (16-byte loads and stores); sums are
// fp32 in a fixed order (slots in increasing j, then the shared term, then
// the residual), rounded once.
#pragma once
#include "common.h"

namespace smoe_comb {

constexpr int kCombThreads = 256;
constexpr int kBatch = 8;  // slots whose rows are requested together

SMOE_DEV void add8(float (&acc)[8], uint4 v, float w) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] += w * h2f((uint16_t)(u[i] & 0xFFFFu));
        acc[2 * i + 1] += w * h2f((uint16_t)(u[i] >> 16));
    }
}

// Plain 16-byte row loads (rows written by earlier launches).
struct PlainRows {
    SMOE_DEV uint4 operator()(const uint16_t* p) const { return *reinterpret_cast<const uint4*>(p); }
};

// fp32 sums of one 8-element chunk c8 of token t's output, in the fixed
// order: slots j = 0..k-1 (pairs with pair_pos -1 skipped), then the shared
// term, then the residual.  The slots' row positions and weights are read
// kBatch at a time, then their rows are requested together.  `ld` reads the
// expert and shared rows (the residual is always an earlier launch's).
template <typename Rows = PlainRows>
SMOE_DEV void combine_chunk(const uint16_t* __restrict__ y, const int32_t* __restrict__ pp,
                            const float* __restrict__ w, const uint16_t* __restrict__ shared,
                            const float* __restrict__ sscale, const uint16_t* resid, int t, int k,
                            int H, int c8, float (&acc)[8], Rows ld = Rows()) {
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
            v[i] = (r[i] >= 0) ? ld(y + (size_t)r[i] * H + 8 * c8) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (r[i] >= 0) add8(acc, v[i], wj[i]);
    }
    if (shared) {
        const float c = sscale ? sscale[t] : 1.0f;
        add8(acc, ld(shared + (size_t)t * H + 8 * c8), c);
    }
    if (resid) add8(acc, reinterpret_cast<const uint4*>(resid + (size_t)t * H)[c8], 1.0f);
}

// The chunk rounded to fp16 (packed), with the sum of squares of the rounded
// values added to sq.
SMOE_DEV uint4 round_chunk(const float (&acc)[8], float& sq) {
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
// squares are sq, computed by the first kCombThreads threads of the
// workgroup (later threads pass 0): a butterfly inside each wave, then the
// first kCombThreads / 64 waves' sums in wave order.  red holds one float
// per wave of the workgroup.  Ends after a barrier.
SMOE_DEV float row_inv_rms(float sq, int H, float eps, float* red) {
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
SMOE_DEV uint4 norm_chunk(uint4 v, float inv) {
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

}  // namespace smoe_comb
