// Device routines of the Expert Lookahead Buffer update and of the stable
// gather-by-expert maps, shared by their own kernels and by the fused
// route + ELB + gather kernel.
//
// Equal expert ids inside a wave are aggregated with ballots (one atomic or
// one LDS update per distinct id per wave), so the integer results do not
// depend on scheduling.
#pragma once

#include "common.h"

namespace smoe_maps {

constexpr int kGatherThreads = 1024;  // one workgroup, 16 waves
constexpr int kGatherWaves = kGatherThreads / 64;

SMOE_DEV uint64_t lanemask_lt(int lane) {
    return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// counters_row[e] += #{p in [p0, n) step stride : ids[p] == e}, with p the
// calling thread's pairs.  Invalid ids are skipped and flagged.
SMOE_DEV void elb_accumulate(const int32_t* ids, int n, int p_first, int stride, int E,
                             int32_t* __restrict__ row, int32_t* __restrict__ err) {
    const int lane = threadIdx.x & 63;
    // every lane of a wave runs the same number of iterations (ballots)
    const int wave_first = p_first - lane;
    for (int base = wave_first; base < n; base += stride) {
        const int p = base + lane;
        const int e = (p < n) ? ids[p] : -1;
        const bool valid = (p < n) && e >= 0 && e < E;
        if (p < n && !valid) flag_error(err, SMOE_DERR_BAD_ID);
        uint64_t todo = __ballot(valid);
        while (todo) {
            const int leader = __ffsll((unsigned long long)todo) - 1;
            const int v = __shfl(e, leader);
            const uint64_t same = __ballot(valid && e == v);
            if (lane == leader) atomicAdd(row + v, (int32_t)__popcll(same));
            todo &= ~same;
        }
    }
}

// Stable counting sort of the n = T*k pairs by expert, by one workgroup of
// kGatherThreads threads (all of which must call it).  ids may point to global
// memory or LDS.
SMOE_DEV void gather_block(const int32_t* ids, int n, int k, int E, int32_t* __restrict__ off,
                           int32_t* __restrict__ sorted_token, int32_t* __restrict__ sorted_pair,
                           int32_t* __restrict__ pair_pos, int32_t* __restrict__ active,
                           int32_t* __restrict__ n_active, int32_t* __restrict__ err) {
    __shared__ int cnt[256];
    __shared__ int base[256];
    __shared__ int wcnt[kGatherWaves][256];
    __shared__ int nvalid;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    for (int e = tid; e < 256; e += kGatherThreads) cnt[e] = 0;
    for (int i = tid; i < kGatherWaves * 256; i += kGatherThreads) (&wcnt[0][0])[i] = 0;
    __syncthreads();

    // 1. per-expert counts (ballot-aggregated LDS adds; order-free)
    for (int c0 = 0; c0 < n; c0 += kGatherThreads) {
        const int p = c0 + tid;
        const int e = (p < n) ? ids[p] : -1;
        const bool valid = (p < n) && e >= 0 && e < E;
        if (p < n && !valid) flag_error(err, SMOE_DERR_BAD_ID);
        uint64_t todo = __ballot(valid);
        while (todo) {
            const int leader = __ffsll((unsigned long long)todo) - 1;
            const int v = __shfl(e, leader);
            const uint64_t same = __ballot(valid && e == v);
            if (lane == leader) atomicAdd(&cnt[v], (int)__popcll(same));
            todo &= ~same;
        }
    }
    __syncthreads();

    // 2. exclusive scan of the counts and the active list (wave 0; E <= 256,
    //    4 consecutive experts per lane)
    if (wave == 0) {
        int c[4], a[4];
        int s = 0, na = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            c[i] = (e < E) ? cnt[e] : 0;
            a[i] = (c[i] > 0) ? 1 : 0;
            s += c[i];
            na += a[i];
        }
        int incl = s, inca = na;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d);
            const int oa = __shfl_up(inca, d);
            if (lane >= d) {
                incl += o;
                inca += oa;
            }
        }
        int run = incl - s, runa = inca - na;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            if (e < E) {
                base[e] = run;
                off[e] = run;
                if (a[i]) active[runa] = e;
            }
            run += c[i];
            runa += a[i];
        }
        const int total = __shfl(incl, 63);
        const int total_a = __shfl(inca, 63);
        if (lane == 0) {
            off[E] = total;
            *n_active = total_a;
            nvalid = total;
        }
        for (int e = total_a + lane; e < E; e += 64) active[e] = -1;
    }
    __syncthreads();

    // 3. stable placement, one chunk of kGatherThreads pairs at a time:
    //    position = base[e] + (same-expert pairs in earlier waves of the
    //    chunk) + (same-expert lanes below this one in the wave)
    for (int c0 = 0; c0 < n; c0 += kGatherThreads) {
        const int p = c0 + tid;
        const int e = (p < n) ? ids[p] : -1;
        const bool valid = (p < n) && e >= 0 && e < E;
        int rank = 0;
        uint64_t todo = __ballot(valid);
        while (todo) {
            const int leader = __ffsll((unsigned long long)todo) - 1;
            const int v = __shfl(e, leader);
            const uint64_t same = __ballot(valid && e == v);
            if (valid && e == v) rank = (int)__popcll(same & lanemask_lt(lane));
            if (lane == leader) wcnt[wave][v] = (int)__popcll(same);
            todo &= ~same;
        }
        __syncthreads();
        if (valid) {
            int pos = base[e] + rank;
            for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
            sorted_pair[pos] = p;
            sorted_token[pos] = p / k;
            pair_pos[p] = pos;
        } else if (p < n) {
            pair_pos[p] = -1;
        }
        __syncthreads();
        for (int ee = tid; ee < E; ee += kGatherThreads) {
            int add = 0;
            for (int w = 0; w < kGatherWaves; ++w) {
                add += wcnt[w][ee];
                wcnt[w][ee] = 0;
            }
            base[ee] += add;
        }
        __syncthreads();
    }
    // rows past the last valid one (dropped pairs) carry -1
    for (int r = nvalid + tid; r < n; r += kGatherThreads) {
        sorted_pair[r] = -1;
        sorted_token[r] = -1;
    }
}

// The ELB update and the maps of n <= kGatherThreads pairs whose ids are in
// LDS, by one workgroup of kGatherThreads threads (all of which must call
// it): thread e < E counts the pairs of expert e (and adds that count to the
// ELB row), thread p counts the earlier pairs with its id, so no loop runs
// over the distinct ids of a wave.  The same stable counting sort as
// gather_block, so the same maps.  kDistinct (the ids of a token are
// distinct, as a top-k's are) with at most 64 tokens: the counts come from
// LDS atomics and a pair's rank within its expert is the number of earlier
// tokens in the expert's token bitmask, with no loop over the pairs.
template <bool kDistinct = false>
SMOE_DEV void small_maps(const int32_t* ids_s, int n, int k, int E,
                         int32_t* __restrict__ counters_row, int32_t* __restrict__ off,
                         int32_t* __restrict__ sorted_token, int32_t* __restrict__ sorted_pair,
                         int32_t* __restrict__ pair_pos, int32_t* __restrict__ active,
                         int32_t* __restrict__ n_active, int32_t* __restrict__ err) {
    __shared__ int cnt_s[256];
    __shared__ int base_s[256];
    __shared__ int nvalid_s;
    __shared__ unsigned long long tmask_s[kDistinct ? 256 : 1];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool masks = kDistinct && n <= 64 * k;  // at most 64 tokens

    // 1. per-expert counts (and the ELB increments); invalid ids flagged
    if (masks) {
        if (tid < E) {
            cnt_s[tid] = 0;
            tmask_s[tid] = 0ull;
        }
        __syncthreads();
        if (tid < n) {
            const int e = ids_s[tid];
            if (e < 0 || e >= E) {
                flag_error(err, SMOE_DERR_BAD_ID);
            } else {
                atomicAdd(&cnt_s[e], 1);
                atomicOr(&tmask_s[e], 1ull << (tid / k));
            }
        }
        __syncthreads();
        if (tid < E && counters_row && cnt_s[tid]) atomicAdd(counters_row + tid, cnt_s[tid]);
    } else {
        if (tid < E) {
            int c = 0;
#pragma unroll 8
            for (int q = 0; q < n; ++q) c += (ids_s[q] == tid) ? 1 : 0;
            cnt_s[tid] = c;
            if (counters_row && c) atomicAdd(counters_row + tid, c);
        }
        if (tid < n) {
            const int e = ids_s[tid];
            if (e < 0 || e >= E) flag_error(err, SMOE_DERR_BAD_ID);
        }
    }
    __syncthreads();

    // 2. exclusive scan of the counts and the active list (wave 0; E <= 256,
    //    4 consecutive experts per lane)
    if (wave == 0) {
        int c[4], a[4];
        int sum = 0, na = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            c[i] = (e < E) ? cnt_s[e] : 0;
            a[i] = (c[i] > 0) ? 1 : 0;
            sum += c[i];
            na += a[i];
        }
        int incl = sum, inca = na;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d);
            const int oa = __shfl_up(inca, d);
            if (lane >= d) {
                incl += o;
                inca += oa;
            }
        }
        int run = incl - sum, runa = inca - na;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            if (e < E) {
                base_s[e] = run;
                off[e] = run;
                if (a[i]) active[runa] = e;
            }
            run += c[i];
            runa += a[i];
        }
        const int total = __shfl(incl, 63);
        const int total_a = __shfl(inca, 63);
        if (lane == 0) {
            off[E] = total;
            *n_active = total_a;
            nvalid_s = total;
        }
        for (int e = total_a + lane; e < E; e += 64) active[e] = -1;
    }
    __syncthreads();

    // 3. placement: sorted row = base of the expert + earlier pairs of it
    if (tid < n) {
        const int p = tid;
        const int e = ids_s[p];
        if (e >= 0 && e < E) {
            int r = 0;
            if (masks) {
                // earlier pairs of e: one per earlier token that chose e
                const int t = p / k;
                r = __popcll(tmask_s[e] & ((1ull << t) - 1ull));
            } else {
#pragma unroll 8
                for (int q = 0; q < p; ++q) r += (ids_s[q] == e) ? 1 : 0;
            }
            const int pos = base_s[e] + r;
            sorted_pair[pos] = p;
            sorted_token[pos] = p / k;
            pair_pos[p] = pos;
        } else {
            pair_pos[p] = -1;
        }
    }
    // rows past the last valid one (dropped pairs) carry -1
    for (int r = nvalid_s + tid; r < n; r += kGatherThreads) {
        sorted_pair[r] = -1;
        sorted_token[r] = -1;
    }
}

// The maps and ELB increments of one token's k distinct ids (ids in LDS), by
// any number of threads of a workgroup: the pair of rank j sits at sorted row
// #{i : ids[i] < ids[j]}, which is where the stable counting sort puts it
// (gather_block); the ELB row gets +1 per selected expert.
SMOE_DEV void one_token_maps(const int32_t* ids, int k, int E, int32_t* __restrict__ counters_row,
                             int32_t* __restrict__ off, int32_t* __restrict__ sorted_token,
                             int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
                             int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
    for (int j = threadIdx.x; j < k; j += blockDim.x) {
        const int id = ids[j];
        int pos = 0;
        for (int i = 0; i < k; ++i) pos += (ids[i] < id) ? 1 : 0;
        if (counters_row) atomicAdd(counters_row + id, 1);
        sorted_token[pos] = 0;
        sorted_pair[pos] = j;
        pair_pos[j] = pos;
        active[pos] = id;
    }
    for (int ee = threadIdx.x; ee <= E; ee += blockDim.x) {
        int c = 0;
        for (int i = 0; i < k; ++i) c += (ids[i] < ee) ? 1 : 0;
        off[ee] = c;
        if (ee >= k && ee < E) active[ee] = -1;
    }
    if (threadIdx.x == 0) *n_active = k;
}

}  // namespace smoe_maps
