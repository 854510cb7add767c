// Top-k routing by the FP16 router, one workgroup per token.
//
// "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step Speculative
// Offloading" (AI summary), Key Contributions 3: routing decisions come from
// the target router; "Specter previews expert routing with an INT4 copy of the
// model itself", What shipped: the draft reuses that same FP16 router.
//
// The logit sum is taken in one pinned fp32 order so that the chosen ids are
// reproducible bit for bit: 8-element hidden chunks, chunk c owned by lane
// c mod 64 of the wave, each lane adding its exact fp16*fp16 products in
// increasing hidden index, then six xor-butterfly rounds (distance 32 .. 1).
// Contraction is switched off in this file: a fused multiply-add would give
// the same value (the products are exact), but the compiler must not fold two
// products into one dot instruction with a different rounding sequence.
#include "common.h"

#pragma clang fp contract(off)

namespace {

constexpr int kRouteThreads = 1024;  // 16 waves; wave w takes experts w, w+16, ...

__device__ __forceinline__ float acc_chunk(float s, uint4 xv, uint4 wv) {
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x0 = h2f((uint16_t)(xw[i] & 0xFFFFu));
        const float w0 = h2f((uint16_t)(ww[i] & 0xFFFFu));
        const float x1 = h2f((uint16_t)(xw[i] >> 16));
        const float w1 = h2f((uint16_t)(ww[i] >> 16));
        const float p0 = x0 * w0;  // exact: 11-bit x 11-bit significands
        s = s + p0;
        const float p1 = x1 * w1;
        s = s + p1;
    }
    return s;
}

// Pinned-order dot product of one fp16 row of x with one fp16 row of w,
// evaluated by a whole wave; every lane returns the same value.  Each lane
// first requests up to 8 of its chunks, then adds them in increasing order.
__device__ __forceinline__ float pinned_dot(const uint4* __restrict__ xr,
                                            const uint4* __restrict__ wrow, int nch, int lane) {
    float s = 0.0f;
    for (int c0 = 0; c0 < nch; c0 += 64 * 8) {
        uint4 xv[8], wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = c0 + lane + 64 * u;
            if (c < nch) {
                xv[u] = xr[c];
                wv[u] = wrow[c];
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = c0 + lane + 64 * u;
            if (c < nch) s = acc_chunk(s, xv[u], wv[u]);
        }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) s = s + __shfl_xor(s, d);
    return s;
}

// Ranking of (logit, expert id) pairs: larger logit first, NaN below every
// number, equal logits (or two NaNs) lower id first.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    const bool na = va != va, nb = vb != vb;
    if (na != nb) return nb;
    if (!na && va != vb) return va > vb;
    return ia < ib;
}

__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const uint16_t* __restrict__ wsg, int H, int E, int k, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ wout, float* __restrict__ gate) {
    __shared__ float logit[257];
    const int t = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int nch = H >> 3;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * H);
    const int nvec = E + (wsg ? 1 : 0);
    for (int e = wave; e < nvec; e += nw) {
        const uint16_t* row = (e < E) ? wr + (size_t)e * H : wsg;
        const float s = pinned_dot(xr, reinterpret_cast<const uint4*>(row), nch, lane);
        if (lane == 0) logit[e] = s;
    }
    __syncthreads();
    if (wave != 0) return;

    // ---- top-k by (logit desc, index asc), one wave ----
    float v[4];
    bool live[4];
    float mysel[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // lane j%64 keeps winner j
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        live[i] = e < E;
        v[i] = live[i] ? logit[e] : 0.0f;
    }
    float m = 0.0f;  // largest logit (the first winner)
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int bi = 0x7fffffff;  // no candidate
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (live[i] && (bi == 0x7fffffff || ranks_before(v[i], e, bv, bi))) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const float ov = __shfl_xor(bv, d);
            const int oi = __shfl_xor(bi, d);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || ranks_before(ov, oi, bv, bi))) {
                bv = ov;
                bi = oi;
            }
        }
        // every lane now holds the same winner
        if (j == 0) m = bv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if ((bi & 63) == lane && (bi >> 6) == i) live[i] = false;
            if ((j & 63) == lane && (j >> 6) == i) mysel[i] = bv;
        }
        if (lane == 0) ids[(size_t)t * k + j] = bi;
    }

    // ---- softmax over all E at the chosen ids ----
    float ssum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < E) ssum += expf(v[i] - m);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ssum = ssum + __shfl_xor(ssum, d);
    float p[4];
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = (lane + 64 * i < k) ? expf(mysel[i] - m) / ssum : 0.0f;
        part += p[i];
    }
    if (renorm) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) part = part + __shfl_xor(part, d);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        if (j < k) wout[(size_t)t * k + j] = renorm ? p[i] / part : p[i];
    }
    if (wsg && lane == 0) gate[t] = 1.0f / (1.0f + expf(-logit[E]));
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
