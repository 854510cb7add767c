// Device routines of the top-k router, shared by the routing kernel and the
// fused route + ELB + gather kernel (both must choose the same ids bit for
// bit, so they run the very same code).
//
// The logit sum is taken in one pinned fp32 order: 8-element hidden chunks,
// chunk c owned by lane c mod 64 of the wave, each lane adding its exact
// fp16*fp16 products in increasing hidden index, then six xor-butterfly
// rounds (distance 32 .. 1).  Contraction is switched off for every file that
// includes this header: a fused multiply-add would give the same value (the
// products are exact), but the compiler must not fold two products into one
// dot instruction with a different rounding sequence.  The pragma sits in
// each function so every file that includes this header compiles these
// routines the same way.
#pragma once

#include "common.h"

namespace smoe_route {

SMOE_DEV float acc_chunk(float s, uint4 xv, uint4 wv) {
#pragma clang fp contract(off)
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x0 = h2f((uint16_t)(xw[i] & 0xFFFFu));
        const float w0 = h2f((uint16_t)(ww[i] & 0xFFFFu));
        const float x1 = h2f((uint16_t)(xw[i] >> 16));
        const float w1 = h2f((uint16_t)(ww[i] >> 16));
        // x*w is exact in fp32 (11-bit x 11-bit significands, no underflow),
        // so a fused multiply-add rounds exactly like the separate add of the
        // product; it lets the hardware take the fp16 operands directly
        // (v_fma_mix), one instruction per element
        s = __builtin_fmaf(x0, w0, s);
        s = __builtin_fmaf(x1, w1, s);
    }
    return s;
}

// Pinned-order dot product of one fp16 row of x with one fp16 row of w,
// evaluated by a whole wave; every lane returns the same value.  Each lane
// first requests up to 8 of its chunks, then adds them in increasing order.
SMOE_DEV float pinned_dot(const uint4* __restrict__ xr, const uint4* __restrict__ wrow, int nch,
                          int lane) {
#pragma clang fp contract(off)
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

// One wave's copy of a weight row for a later pinned-order dot product:
// lane l requests chunks l, l + 64, ... (u < CPL) into registers.
template <int CPL>
SMOE_DEV void pinned_row(const uint16_t* __restrict__ row, int H, int lane, uint4 (&wv)[CPL]) {
    const uint4* r4 = reinterpret_cast<const uint4*>(row);
    const int nch = H >> 3;
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
        const int c = lane + 64 * u;
        if (c < nch) wv[u] = r4[c];
    }
}

// pinned_dot of the row x (in LDS or memory) with a row fetched by
// pinned_row (CPL * 64 * 8 >= H): the same chunks, added in the same order,
// so the value equals pinned_dot's and wave_logits'.
template <int CPL>
SMOE_DEV float pinned_dot_regs(const uint4* __restrict__ xr, const uint4 (&wv)[CPL], int H,
                               int lane) {
#pragma clang fp contract(off)
    const int nch = H >> 3;
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
        const int c = lane + 64 * u;
        if (c < nch) s = acc_chunk(s, xr[c], wv[u]);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) s = s + __shfl_xor(s, d);
    return s;
}

// Logits of the items i = first, first + stride, ... < n_items handled by one
// wave; item i is (token i / nvec, vector i % nvec), vector e < E being router
// row e and vector E the shared-gate row.  Up to D items of one token are
// evaluated together: the token's CPL chunks per lane are requested once and
// the D weight rows' chunks are all in flight before any sum starts.  Every
// sum is the pinned order of pinned_dot (a lane adds its chunks c = lane,
// lane + 64, ... in increasing order, then the same butterfly), so the values
// are identical.
template <int D, int CPL>
SMOE_DEV void wave_logits_batched(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                  const uint16_t* __restrict__ wsg, int H, int E, int nvec,
                                  int first, int n_items, int stride, float* out, int lane) {
#pragma clang fp contract(off)
    const int nch = H >> 3;
    for (int i = first; i < n_items;) {
        const int t = i / nvec;
        int nd = 0;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int ii = i + d * stride;
            if (ii < n_items && ii / nvec == t) nd = d + 1;  // a prefix: items increase
        }
        const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * H);
        uint4 xv[CPL];
        uint4 wv[D][CPL];
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            const int c = lane + 64 * u;
            if (c < nch) xv[u] = xr[c];
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d < nd) {
                const int e = (i + d * stride) - t * nvec;
                const uint4* row = reinterpret_cast<const uint4*>(e < E ? wr + (size_t)e * H : wsg);
#pragma unroll
                for (int u = 0; u < CPL; ++u) {
                    const int c = lane + 64 * u;
                    if (c < nch) wv[d][u] = row[c];
                }
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d < nd) {
                float s = 0.0f;
#pragma unroll
                for (int u = 0; u < CPL; ++u) {
                    const int c = lane + 64 * u;
                    if (c < nch) s = acc_chunk(s, xv[u], wv[d][u]);
                }
#pragma unroll
                for (int dd = 32; dd >= 1; dd >>= 1) s = s + __shfl_xor(s, dd);
                if (lane == 0) out[i + d * stride] = s;
            }
        }
        i += nd * stride;
    }
}

// wave_logits_batched for any H: batches sized so that at most 16 weight
// chunks per lane are in flight (H <= 4096); longer rows one item at a time.
SMOE_DEV void wave_logits(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                          const uint16_t* __restrict__ wsg, int H, int E, int nvec, int first,
                          int n_items, int stride, float* out, int lane) {
    const int cpl = ((H >> 3) + 63) / 64;
    if (cpl <= 1) {
        wave_logits_batched<4, 1>(x, wr, wsg, H, E, nvec, first, n_items, stride, out, lane);
    } else if (cpl <= 2) {
        wave_logits_batched<4, 2>(x, wr, wsg, H, E, nvec, first, n_items, stride, out, lane);
    } else if (cpl <= 4) {
        wave_logits_batched<4, 4>(x, wr, wsg, H, E, nvec, first, n_items, stride, out, lane);
    } else if (cpl <= 8) {
        wave_logits_batched<2, 8>(x, wr, wsg, H, E, nvec, first, n_items, stride, out, lane);
    } else {
        for (int i = first; i < n_items; i += stride) {
            const int t = i / nvec;
            const int e = i - t * nvec;
            const uint16_t* row = (e < E) ? wr + (size_t)e * H : wsg;
            const float s = pinned_dot(reinterpret_cast<const uint4*>(x + (size_t)t * H),
                                       reinterpret_cast<const uint4*>(row), H >> 3, lane);
            if (lane == 0) out[i] = s;
        }
    }
}

// Ranking of (logit, expert id) pairs: larger logit first, NaN below every
// number, equal logits (-0 equal to +0, or two NaNs) lower id first.  As a
// 64-bit key: the logit's bits mapped to an unsigned order (NaN lowest), then
// the complemented id; a pair ranks before another iff its key is larger.
SMOE_DEV uint64_t rank_key(float v, int e) {
    uint32_t u = __float_as_uint(v);
    uint32_t ord;
    if (v != v) {
        ord = 0u;
    } else {
        if ((u << 1) == 0u) u = 0u;  // -0 as +0
        ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// rank[i] += number of the E keys above key[i], for the NB key blocks held
// (lane l holds key[i] of expert l + 64 i); keys are broadcast by readlane.
template <int NB>
SMOE_DEV void count_ranks(const uint64_t (&key)[4], int E, int (&rank)[4]) {
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
        const int nj = min(64, E - 64 * ib);
        const uint32_t lo = (uint32_t)key[ib];
        const uint32_t hi = (uint32_t)(key[ib] >> 32);
#pragma unroll 4
        for (int j = 0; j < nj; ++j) {
            const uint64_t kj = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, j) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)lo, j);
#pragma unroll
            for (int i = 0; i < NB; ++i) rank[i] += (kj > key[i]) ? 1 : 0;
        }
    }
}

// The largest 64-bit value over the wave (every lane's v, all 64 lanes
// active; result uniform):
// DPP exchanges within each row of 16 lanes (quad xor 1, xor 2, then the
// half-row and row mirrors), then the four row maxima through readlane.
SMOE_DEV uint64_t wave_max_u64(uint64_t v) {
    auto step = [&](auto ctrl) {
        constexpr int C = decltype(ctrl)::value;
        const uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
        const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, C, 0xF, 0xF, false);
        const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, C, 0xF, 0xF, false);
        const uint64_t o = ((uint64_t)ohi << 32) | olo;
        v = o > v ? o : v;
    };
    step(std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    step(std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
    step(std::integral_constant<int, 0x141>{});  // row_half_mirror
    step(std::integral_constant<int, 0x140>{});  // row_mirror
    const uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
    uint64_t m = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint64_t c = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r);
        m = c > m ? c : m;
    }
    return m;
}

// rank[i] = r for the key selected in round r < k (the largest remaining key
// of the wave each round), k for every other key; the same ranks below k as
// count_ranks.  Dead slots hold key 0, below every live key (whose low word,
// the complemented id, is never 0).
template <int NB>
SMOE_DEV void select_ranks(const uint64_t (&key)[4], int k, int (&rank)[4]) {
    uint64_t kk[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        kk[i] = key[i];
        rank[i] = k;
    }
    for (int r = 0; r < k; ++r) {
        uint64_t best = kk[0];
#pragma unroll
        for (int i = 1; i < NB; ++i) best = kk[i] > best ? kk[i] : best;
        const uint64_t w = wave_max_u64(best);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (kk[i] == w) {
                rank[i] = r;
                kk[i] = 0;
            }
    }
}

// One wave selects the top k of a token's E logits (lg, in LDS; lg[E] is the
// shared-gate logit when has_gate) and writes ids, weights (softmax over all
// E at the chosen ids, optionally renormalised over the k) and the gate.
// ids_copy (nullable) receives the ids as well.  Lane l holds experts
// l + 64 i; each expert's rank is the number of keys above its own (every
// key taken from its lane by readlane), and the experts of rank < k are the
// selection, in rank order.
// Rank of every expert's logit (lane l holds experts l + 64 i): the number
// of keys above its own.
// Selections of up to kSelectMaxK experts take k rounds of a wave maximum;
// larger ones count, for every key, the keys above it.
#ifndef SMOE_SELECT_MAX_K
#define SMOE_SELECT_MAX_K 16
#endif
constexpr int kSelectMaxK = SMOE_SELECT_MAX_K;
SMOE_DEV void rank_experts(const float* lg, int E, int k, int lane, float (&v)[4],
                           int (&rank)[4]) {
    uint64_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        const bool live = e < E;
        v[i] = live ? lg[e] : 0.0f;
        key[i] = live ? rank_key(v[i], e) : 0ull;
        rank[i] = 0;
    }
    const int nblk = (E + 63) >> 6;  // key blocks actually held (uniform)
    if (k <= kSelectMaxK) {
        if (nblk == 1)
            select_ranks<1>(key, k, rank);
        else if (nblk == 2)
            select_ranks<2>(key, k, rank);
        else if (nblk == 3)
            select_ranks<3>(key, k, rank);
        else
            select_ranks<4>(key, k, rank);
        return;
    }
    if (nblk == 1)
        count_ranks<1>(key, E, rank);
    else if (nblk == 2)
        count_ranks<2>(key, E, rank);
    else if (nblk == 3)
        count_ranks<3>(key, E, rank);
    else
        count_ranks<4>(key, E, rank);
}

// The top-k ids alone (ids[r] = the expert of rank r < k), as
// topk_softmax_wave selects them.
SMOE_DEV void topk_ids_wave(const float* lg, int E, int k, int lane, int32_t* ids) {
    float v[4];
    int rank[4];
    rank_experts(lg, E, k, lane, v, rank);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < E && rank[i] < k) ids[rank[i]] = e;
    }
}

SMOE_DEV void topk_softmax_wave(const float* lg, int E, int k, int renorm, bool has_gate,
                                int lane, int32_t* ids, float* wout, float* gate,
                                int32_t* ids_copy) {
#pragma clang fp contract(off)
    float v[4];
    int rank[4];
    rank_experts(lg, E, k, lane, v, rank);
    // the largest logit: the value of the rank-0 expert, from its lane
    float v0 = 0.0f;
    bool has0 = false;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < E && rank[i] == 0) {
            v0 = v[i];
            has0 = true;
        }
    const uint64_t b0 = __ballot(has0);
    const float m = __shfl(v0, __ffsll((unsigned long long)b0) - 1);

    // softmax over all E at the chosen ids
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
        const bool sel = lane + 64 * i < E && rank[i] < k;
        p[i] = sel ? expf(v[i] - m) / ssum : 0.0f;
        part += p[i];
    }
    if (renorm) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) part = part + __shfl_xor(part, d);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < E && rank[i] < k) {
            ids[rank[i]] = e;
            if (ids_copy) ids_copy[rank[i]] = e;
            wout[rank[i]] = renorm ? p[i] / part : p[i];
        }
    }
    if (has_gate && lane == 0) *gate = 1.0f / (1.0f + expf(-lg[E]));
}

}  // namespace smoe_route
