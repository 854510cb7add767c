// Draft routed-expert SwiGLU FFN over GPTQ INT4 (group 128) weights, one
// launch per projection across every touched expert.
//
// "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step Speculative
// Offloading" (AI summary), Key Contributions 4: a fused multi-expert INT4
// draft kernel that gathers tokens by expert and runs all experts in one
// launch.  "Specter previews expert routing with an INT4 copy of the model
// itself", What shipped: W4A16, i.e. INT4 weight tiles are dequantised while
// the products are formed in higher precision; GPTQ, group size 128.
//
// At draft shapes (one to a few rows per expert) this is a weight-streaming
// GEMV: every packed byte is read from HBM once, so the design is about bytes
// in flight and VALU cost per weight, not matrix cores.
//
// Work decomposition.  A workgroup owns one (touched expert, block of NB
// weight columns) over the whole reduction, so no workgroup ever waits for
// another.  Inside a wave, LPR lanes share one packed row: lane q of the
// group reads 16 bytes = 4 adjacent columns, so a wave load is RPL = 64/LPR
// rows of 4*LPR columns (64- or 128-byte runs per row).  The RPL lane groups
// of every wave ("slots") each take whole 128-K quantisation groups, round
// robin, streaming a group's 16 packed rows with 16 loads in flight per lane
// (and, for one-row experts, the next group's rows requested before the
// current group is consumed); latency is hidden by the other waves resident on
// the SIMD.  With one activation row per expert (a one-token step) the row and
// the first weights are requested together before the row is staged.
// In the gate/up projection a block is NB/2 gate columns next to the matching
// NB/2 up columns, so SwiGLU is applied inside the workgroup.
//
// Dequantisation.  For a packed word w, (w & 0x000F000F) | 0x64006400 is the
// fp16 pair (1024 + q_i, 1024 + q_(i+4)) and (w & 0x00F000F0) | 0x64006400 is
// (1024 + 16 q_(i+1), 1024 + 16 q_(i+5)); a shift by 8 gives the other four
// codes.  These pairs go straight into v_dot2_f32_f16 against the matching
// activation pairs (fp32 accumulation; every product is exact).  The constant
// parts and the zero point are removed once per group and column with the
// group's activation sums over even and odd k, then the group sum is scaled by
// the fp16 scale.  Cost per packed word: 5 VALU ops (one shift, four
// and-or) plus 4 dot2 per activation row.  Activations are staged once per
// workgroup in LDS, already permuted into the pairs the dot2 needs, together
// with their per-group sums.
//
// The slots' partial sums are added in a fixed order through LDS: the output
// is deterministic and no floating-point atomics are used.
#include "common.h"

namespace {

constexpr uint32_t kMagic = 0x64006400u;
constexpr int kRowsPerGroup = 16;     // packed rows (8 K each) per 128-K group
#ifndef SMOE_W4_MAX_WAVES
#define SMOE_W4_MAX_WAVES 4
#endif
#ifndef SMOE_W4_MIN_WG
#define SMOE_W4_MIN_WG 128
#endif
#ifndef SMOE_W4_MAX_GROUPS_PER_SLOT
#define SMOE_W4_MAX_GROUPS_PER_SLOT 2
#endif
#ifndef SMOE_W4_ROWFENCE
#define SMOE_W4_ROWFENCE 1
#endif
#ifndef SMOE_W4_PREFETCH
#define SMOE_W4_PREFETCH 1
#endif
constexpr int kMaxWaves = SMOE_W4_MAX_WAVES;  // waves per workgroup (upper bound)
constexpr int kLdsBytes = 32 * 1024;  // activation staging budget per workgroup

struct W4Args {
    const uint16_t* xin;          // phase 1: x [T, H]; phase 2: h [rows, I]
    const int32_t* sorted_token;  // phase 1 only
    const int32_t* off;
    const int32_t* active;
    const int32_t* n_active;
    const smoe_w4_expert* experts;
    int K;      // reduction length: H (phase 1) or I (phase 2)
    int N;      // weight columns: 2I or H
    int I;
    int nCB;    // column blocks
    int MCH;    // rows per chunk (<= the kernel's row capacity)
    int XR;     // activation rows held in LDS
    int direct; // 1: all T token rows of x staged up front (gate/up projection)
    int T;      // token rows of x
    uint16_t* out;  // phase 1: h [rows, I]; phase 2: y [rows, H]
    int32_t* err;
};

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }
__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// Masks held in VGPRs: with a VGPR mask and the magic constant in an SGPR the
// compiler emits one v_and_or_b32 per code pair (a VOP3 op cannot take two
// scalar/literal operands on this target).
__device__ __forceinline__ uint32_t vgpr_const_lo() {
    uint32_t v;
    asm("v_mov_b32 %0, 0xf000f" : "=v"(v));
    return v;
}
__device__ __forceinline__ uint32_t vgpr_const_hi() {
    uint32_t v;
    asm("v_mov_b32 %0, 0xf000f0" : "=v"(v));
    return v;
}

// One 128-K group of M activation rows against this lane's 4 columns.
//   A_even = sum over even k of (1024 + q_k) x_k,
//   A_odd  = sum over odd  k of (1024 + 16 q_k) x_k,
//   sum_k (q_k - z) x_k = A_even + A_odd/16 - (1024 + z) S_even - (64 + z) S_odd
// with S_even, S_odd the group's activation sums (precomputed in LDS).
template <int M, int MAXM>
__device__ __forceinline__ void group_dot(const u4_t (&wv)[kRowsPerGroup],
                                          const uint4* __restrict__ xs,
                                          const float2* __restrict__ sums,
                                          const int (&xoff)[MAXM], const int (&soff)[MAXM],
                                          uint2 sv, uint32_t zw, uint32_t mlo, uint32_t mhi,
                                          float (&acc)[MAXM][4]) {
    float ae[M][4], ao[M][4];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) ae[m][c] = ao[m][c] = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowsPerGroup; ++i) {
        // one packed row at a time: keeps the activation reads from being
        // hoisted ahead of the whole group (register pressure)
        if (SMOE_W4_ROWFENCE) __builtin_amdgcn_sched_barrier(0);
        uint4 xp[M];
#pragma unroll
        for (int m = 0; m < M; ++m) xp[m] = xs[xoff[m] + i];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t w = wv[i][c];
            const uint32_t b = w >> 8;
            const h2_t e0 = as_h2((w & mlo) | kMagic);  // 1024+q0, 1024+q4
            const h2_t o0 = as_h2((w & mhi) | kMagic);  // 1024+16q1, 1024+16q5
            const h2_t e1 = as_h2((b & mlo) | kMagic);  // 1024+q2, 1024+q6
            const h2_t o1 = as_h2((b & mhi) | kMagic);  // 1024+16q3, 1024+16q7
#pragma unroll
            for (int m = 0; m < M; ++m) {
                ae[m][c] = __builtin_amdgcn_fdot2(e0, as_h2(xp[m].x), ae[m][c], false);
                ao[m][c] = __builtin_amdgcn_fdot2(o0, as_h2(xp[m].y), ao[m][c], false);
                ae[m][c] = __builtin_amdgcn_fdot2(e1, as_h2(xp[m].z), ae[m][c], false);
                ao[m][c] = __builtin_amdgcn_fdot2(o1, as_h2(xp[m].w), ao[m][c], false);
            }
        }
    }
    float2 se[M];
#pragma unroll
    for (int m = 0; m < M; ++m) se[m] = sums[soff[m]];
    const uint32_t sw[2] = {sv.x, sv.y};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float s = h2f((uint16_t)(sw[c >> 1] >> (16 * (c & 1))));
        const float z = (float)((zw >> (4 * c)) & 0xFu);
        const float ce = 1024.0f + z;
        const float co = 64.0f + z;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float t = ae[m][c] + 0.0625f * ao[m][c];
            t -= ce * se[m].x;
            t -= co * se[m].y;
            acc[m][c] += s * t;
        }
    }
}

struct GroupLoad {
    u4_t w[kRowsPerGroup];
    uint2 s;
    uint32_t z;
};

// Packed weights are read through a buffer resource: the lane's byte offset
// (column and group) is one VGPR and the packed-row stride a scalar offset,
// so a group's 16 row addresses cost no vector registers.
struct W4Src {
    __amdgpu_buffer_rsrc_t q;  // qweight [K/8, N] int32
    smoe_w4_mat m;
    int N;
};

constexpr int kBufWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family
constexpr int kAuxNT = 2;              // non-temporal (streamed once)

__device__ __forceinline__ W4Src make_src(const smoe_w4_mat& m, int K, int N) {
    W4Src s;
    s.q = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(m.qweight), (short)0,
                                            (K >> 3) * N * 4, kBufWord3);
    s.m = m;
    s.N = N;
    return s;
}

__device__ __forceinline__ void load_group(GroupLoad& L, const W4Src& src, int g, int col,
                                           bool colok) {
    const int N = src.N;
    const int voff = ((g * kRowsPerGroup) * N + col) * 4;
#pragma unroll
    for (int i = 0; i < kRowsPerGroup; ++i)
        L.w[i] = colok ? __builtin_amdgcn_raw_buffer_load_b128(src.q, voff, i * N * 4, kAuxNT)
                       : u4_t{0, 0, 0, 0};
    if (colok) {
        const uint64_t sv =
            *as_global(reinterpret_cast<const uint64_t*>(src.m.scales + (size_t)g * N + col));
        L.s = make_uint2((uint32_t)sv, (uint32_t)(sv >> 32));
        L.z = (uint32_t)*as_global(src.m.qzeros + (size_t)g * (N >> 3) + (col >> 3)) >> (4 * (col & 7));
    } else {
        L.s = make_uint2(0, 0);
        L.z = 0;
    }
}

template <int MAXM>
__device__ __forceinline__ void group_step(const GroupLoad& L, const uint4* xs, const float2* sums,
                                           const int (&xrow)[MAXM], int g, int K8, int G, int M,
                                           uint32_t mlo, uint32_t mhi, float (&acc)[MAXM][4]) {
    int xoff[MAXM], soff[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        xoff[m] = xrow[m] * K8 + g * kRowsPerGroup;
        soff[m] = xrow[m] * G + g;
    }
    if (MAXM == 1) {
        group_dot<1, MAXM>(L.w, xs, sums, xoff, soff, L.s, L.z, mlo, mhi, acc);
    } else {
        switch (M) {
            case 1: group_dot<1, MAXM>(L.w, xs, sums, xoff, soff, L.s, L.z, mlo, mhi, acc); break;
            case 2: group_dot<(MAXM >= 2 ? 2 : 1), MAXM>(L.w, xs, sums, xoff, soff, L.s, L.z, mlo, mhi, acc); break;
            case 3: group_dot<(MAXM >= 3 ? 3 : 1), MAXM>(L.w, xs, sums, xoff, soff, L.s, L.z, mlo, mhi, acc); break;
            default: group_dot<MAXM, MAXM>(L.w, xs, sums, xoff, soff, L.s, L.z, mlo, mhi, acc); break;
        }
    }
}

// Activations as the dot2 pairs the dequantised codes meet: (x0,x4), (x1,x5),
// (x2,x6), (x3,x7) of each 8-element chunk.
__device__ __forceinline__ uint4 pair_permute(uint4 d) {
    uint4 p;
    p.x = (d.x & 0xFFFFu) | (d.z << 16);      // (x0, x4)
    p.y = (d.x >> 16) | (d.z & 0xFFFF0000u);  // (x1, x5)
    p.z = (d.y & 0xFFFFu) | (d.w << 16);      // (x2, x6)
    p.w = (d.y >> 16) | (d.w & 0xFFFF0000u);  // (x3, x7)
    return p;
}

// Stage activation rows src_row(j), j < nrows, into LDS rows 0..nrows-1 as
// dot2 pairs, then their per-group sums over even and odd k.
template <typename RowPtr>
__device__ __forceinline__ void stage_rows(uint4* xs, float2* sums, int nrows, int K8, int G,
                                           RowPtr src_row) {
#pragma unroll 1
    for (int idx = threadIdx.x; idx < nrows * K8; idx += blockDim.x) {
        const int j = idx / K8;
        const int rr = idx - j * K8;
        xs[j * K8 + rr] = pair_permute(src_row(j)[rr]);
    }
    __syncthreads();
#pragma unroll 1
    for (int idx = threadIdx.x; idx < nrows * G; idx += blockDim.x) {
        const int j = idx / G;
        const int gg = idx - j * G;
        const uint4* xr = xs + j * K8 + gg * kRowsPerGroup;
        float se = 0.0f, so = 0.0f;
#pragma unroll 4
        for (int i = 0; i < kRowsPerGroup; ++i) {
            const uint4 p = xr[i];
            const h2_t x04 = as_h2(p.x), x15 = as_h2(p.y), x26 = as_h2(p.z), x37 = as_h2(p.w);
            se += ((float)x04.x + (float)x04.y) + ((float)x26.x + (float)x26.y);
            so += ((float)x15.x + (float)x15.y) + ((float)x37.x + (float)x37.y);
        }
        sums[j * G + gg] = make_float2(se, so);
    }
    __syncthreads();
}

// Add the slots' partial sums of rows [mc, mc+M) in a fixed order and write
// the epilogue: SwiGLU into h (gate/up projection) or y (down projection).
template <int PHASE, int MAXM, int NB>
__device__ __forceinline__ void reduce_store(const W4Args& a, float* red, const float (&acc)[MAXM][4],
                                             int myslot, int nslots, int q, int cb, int mc, int M) {
    const int tid = threadIdx.x;
    __syncthreads();  // every slot is done with the activations in LDS
#pragma unroll
    for (int m = 0; m < MAXM; ++m)
        if (m < M)
#pragma unroll
            for (int c = 0; c < 4; ++c) red[(myslot * MAXM + m) * NB + 4 * q + c] = acc[m][c];
    __syncthreads();
    if (PHASE == 1) {
        for (int idx = tid; idx < M * (NB / 2); idx += blockDim.x) {
            const int m = idx / (NB / 2);
            const int j = idx - m * (NB / 2);
            float gv = 0.0f, uv = 0.0f;
            for (int s = 0; s < nslots; ++s) {
                gv += red[(s * MAXM + m) * NB + j];
                uv += red[(s * MAXM + m) * NB + NB / 2 + j];
            }
            a.out[(size_t)(mc + m) * a.I + cb * (NB / 2) + j] = f2h(silu_f(gv) * uv);
        }
    } else {
        const int N = a.N;
        for (int idx = tid; idx < M * NB; idx += blockDim.x) {
            const int m = idx / NB;
            const int j = idx - m * NB;
            if (cb * NB + j < N) {
                float v = 0.0f;
                for (int s = 0; s < nslots; ++s) v += red[(s * MAXM + m) * NB + j];
                a.out[(size_t)(mc + m) * N + cb * NB + j] = f2h(v);
            }
        }
    }
    __syncthreads();  // red is rewritten by the next row chunk
}

// A slot's groups g, g + nslots, ... of the reduction.  With kPrefetch the
// next group's weights are requested before the current group is consumed.
template <bool kPrefetch, int MAXM>
__device__ __forceinline__ void run_groups(GroupLoad& cur, int g, int nslots, int G,
                                           const W4Src& src, int col, bool colok,
                                           const uint4* xs, const float2* sums,
                                           const int (&xrow)[MAXM], int K8, int M, uint32_t mlo,
                                           uint32_t mhi, float (&acc)[MAXM][4]) {
    if (g >= G) return;
    for (;;) {
        const int gn = g + nslots;
        GroupLoad nxt;
        if (kPrefetch && gn < G) load_group(nxt, src, gn, col, colok);
        group_step<MAXM>(cur, xs, sums, xrow, g, K8, G, M, mlo, mhi, acc);
        if (gn >= G) break;
        if (!kPrefetch) load_group(nxt, src, gn, col, colok);
        cur = nxt;
        g = gn;
    }
}

constexpr int kRowChunksPerThread = 8;  // activation chunks per thread requested early

template <int PHASE, int LPR, int MAXM>
__global__ __launch_bounds__(64 * kMaxWaves) void w4_kernel(W4Args a) {
    constexpr int RPL = 64 / LPR;  // lane groups (slots) per wave
    constexpr int NB = 4 * LPR;    // columns per block
    extern __shared__ uint4 smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int rho = lane / LPR;
    const int q = lane % LPR;
    const int cb = blockIdx.x % a.nCB;
    const int slot = blockIdx.x / a.nCB;
    const int K = a.K, N = a.N;
    const int G = K >> 7;
    const int K8 = K >> 3;
    uint4* xs = smem;                                                       // [XR][K8]
    float2* sums = reinterpret_cast<float2*>(smem + (size_t)a.XR * K8);     // [XR][G]
    float* red = reinterpret_cast<float*>(sums + (size_t)a.XR * G);  // [nslots][MAXM][NB]

    const int nslots = nwaves * RPL;
    const int myslot = wave * RPL + rho;
    int col;
    bool colok;
    if (PHASE == 1) {
        col = (q < LPR / 2) ? cb * (NB / 2) + 4 * q : a.I + cb * (NB / 2) + 4 * (q - LPR / 2);
        colok = true;
    } else {
        col = cb * NB + 4 * q;
        colok = col < N;
    }
    const uint32_t mlo = vgpr_const_lo();
    const uint32_t mhi = vgpr_const_hi();

    if constexpr (MAXM == 1) {
        // One token (T = 1): every pair's token is 0, and the touched experts
        // in increasing id (the active list) own sorted rows 0, 1, ... in
        // that order, so this slot's activation row is known before the maps
        // are read: x row 0 (gate/up) or h row `slot` (down).  It is
        // requested first, then the expert's first weights; the row is
        // permuted into LDS while both are in flight.
        const uint16_t* row = (PHASE == 1) ? a.xin : a.xin + (size_t)slot * K;
        const uint4* row4 = reinterpret_cast<const uint4*>(row);
        uint4 xv[kRowChunksPerThread];
#pragma unroll
        for (int u = 0; u < kRowChunksPerThread; ++u) {
            const int idx = tid + u * (int)blockDim.x;
            if (idx < K8) xv[u] = row4[idx];
        }
        const int e = a.active[slot];  // -1 past the touched experts
        if (e < 0) return;
        const smoe_w4_mat wm = (PHASE == 1) ? a.experts[e].w13 : a.experts[e].w2;
        if (!wm.qweight || !wm.scales || !wm.qzeros) {
            if (tid == 0 && cb == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
            return;
        }
        const W4Src src = make_src(wm, K, N);
        GroupLoad cur;
        const int g = myslot;
        if (g < G) load_group(cur, src, g, col, colok);
#pragma unroll
        for (int u = 0; u < kRowChunksPerThread; ++u) {
            const int idx = tid + u * (int)blockDim.x;
            if (idx < K8) xs[idx] = pair_permute(xv[u]);
        }
        // rows longer than the early requests cover (small workgroups)
        for (int idx = tid + kRowChunksPerThread * (int)blockDim.x; idx < K8; idx += blockDim.x)
            xs[idx] = pair_permute(row4[idx]);
        __syncthreads();
        for (int gg = tid; gg < G; gg += blockDim.x) {
            const uint4* xr = xs + gg * kRowsPerGroup;
            float se = 0.0f, so = 0.0f;
#pragma unroll 4
            for (int i = 0; i < kRowsPerGroup; ++i) {
                const uint4 p = xr[i];
                const h2_t x04 = as_h2(p.x), x15 = as_h2(p.y), x26 = as_h2(p.z), x37 = as_h2(p.w);
                se += ((float)x04.x + (float)x04.y) + ((float)x26.x + (float)x26.y);
                so += ((float)x15.x + (float)x15.y) + ((float)x37.x + (float)x37.y);
            }
            sums[gg] = make_float2(se, so);
        }
        __syncthreads();
        float acc[1][4] = {{0.0f, 0.0f, 0.0f, 0.0f}};
        const int xrow[1] = {0};
        run_groups<SMOE_W4_PREFETCH != 0, 1>(cur, g, nslots, G, src, col, colok, xs, sums, xrow,
                                             K8, 1, mlo, mhi, acc);
        reduce_store<PHASE, 1, NB>(a, red, acc, myslot, nslots, q, cb, slot, 1);
        return;
    } else {
        const int e = a.active[slot];  // -1 past the touched experts
        if (e < 0) return;
        const smoe_w4_mat wm = (PHASE == 1) ? a.experts[e].w13 : a.experts[e].w2;
        const int r0 = a.off[e];
        const int r1 = a.off[e + 1];
        if (!wm.qweight || !wm.scales || !wm.qzeros) {
            if (tid == 0 && cb == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
            return;
        }
        const W4Src src = make_src(wm, K, N);
        // The gate/up projection with every token fitting in LDS stages all
        // T activation rows once.
        const bool direct = (PHASE == 1) && a.direct;
        if (direct)
            stage_rows(xs, sums, a.T, K8, G, [&](int j) {
                return reinterpret_cast<const uint4*>(a.xin + (size_t)j * K);
            });
        for (int mc = r0; mc < r1; mc += a.MCH) {
            const int M = min(a.MCH, r1 - mc);
            int xrow[MAXM];
#pragma unroll
            for (int m = 0; m < MAXM; ++m)
                xrow[m] = direct ? a.sorted_token[mc + (m < M ? m : 0)] : m;
            if (!direct) {
                if (PHASE == 1)
                    stage_rows(xs, sums, M, K8, G, [&](int j) {
                        return reinterpret_cast<const uint4*>(a.xin +
                                                              (size_t)a.sorted_token[mc + j] * K);
                    });
                else
                    stage_rows(xs, sums, M, K8, G, [&](int j) {
                        return reinterpret_cast<const uint4*>(a.xin + (size_t)(mc + j) * K);
                    });
            }
            GroupLoad cur;
            const int g = myslot;
            if (g < G) load_group(cur, src, g, col, colok);
            float acc[MAXM][4];
#pragma unroll
            for (int m = 0; m < MAXM; ++m)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[m][c] = 0.0f;
            run_groups<false, MAXM>(cur, g, nslots, G, src, col, colok, xs, sums, xrow, K8, M, mlo,
                                    mhi, acc);
            reduce_store<PHASE, MAXM, NB>(a, red, acc, myslot, nslots, q, cb, mc, M);
        }
    }
}

// ---------------------------------------------------------------- launch ----

struct PhasePlan {
    int lpr, nCB, waves, mch, xr, direct;
    size_t lds;
};

PhasePlan plan_phase(int phase, int slots, int T, int K, int N, int I, int maxm) {
    // LPR 16 (64-column blocks, 256-byte row runs) when that still gives
    // SMOE_W4_MIN_WG workgroups and no slot walks more than
    // SMOE_W4_MAX_GROUPS_PER_SLOT groups in sequence; else LPR 8 (32 columns,
    // twice the workgroups and slots).  Measured on the decode shapes (H 2048
    // and 4096, I 1408 and 6400, one to sixteen rows per expert).
    PhasePlan p{};
    const int cols16 = (phase == 1) ? I / 32 : (N + 63) / 64;
    const int G16 = K / 128;
    const int serial16 = (G16 + 4 * kMaxWaves - 1) / (4 * kMaxWaves);
    p.lpr = ((long long)slots * cols16 >= SMOE_W4_MIN_WG &&
             serial16 <= SMOE_W4_MAX_GROUPS_PER_SLOT) ? 16 : 8;
    const int NB = 4 * p.lpr;
    p.nCB = (phase == 1) ? I / (NB / 2) : (N + NB - 1) / NB;
    const int rpl = 64 / p.lpr;
    const int G = K / 128;
    p.waves = (G + rpl - 1) / rpl;
    // the launch bound caps every kernel at kMaxWaves; the multi-row kernels'
    // register budget at 4
    const int wmax = (maxm == 1 || kMaxWaves < 4) ? kMaxWaves : 4;
    if (p.waves > wmax) p.waves = wmax;
    if (p.waves < 1) p.waves = 1;
    const size_t row_bytes = (size_t)K * 2 + (size_t)G * 8;  // pairs + group sums
    int cap = (int)(kLdsBytes / row_bytes);
    if (cap < 1) cap = 1;
    p.mch = cap < maxm ? cap : maxm;
    p.direct = (phase == 1 && T <= cap) ? 1 : 0;
    p.xr = p.direct ? T : p.mch;
    const size_t red_bytes = (size_t)p.waves * rpl * maxm * NB * 4;
    p.lds = (size_t)p.xr * row_bytes + red_bytes;
    return p;
}

template <int PHASE, int MAXM>
hipError_t launch_phase(const W4Args& a, int slots, const PhasePlan& p, hipStream_t s) {
    const dim3 grid(slots * p.nCB), block(64 * p.waves);
    if (p.lpr == 16)
        hipLaunchKernelGGL((w4_kernel<PHASE, 16, MAXM>), grid, block, p.lds, s, a);
    else
        hipLaunchKernelGGL((w4_kernel<PHASE, 8, MAXM>), grid, block, p.lds, s, a);
    return hipGetLastError();
}

template <int PHASE>
hipError_t launch_any(const W4Args& a, int slots, const PhasePlan& p, int maxm, hipStream_t s) {
    return (maxm == 1) ? launch_phase<PHASE, 1>(a, slots, p, s)
                       : launch_phase<PHASE, 4>(a, slots, p, s);
}

}  // namespace

namespace smoe {
size_t w4a16_workspace_bytes(int T, int k, int /*H*/, int I, int /*E*/) {
    return ((size_t)T * k * I * 2 + 255) & ~(size_t)255;  // h [T*k, I] fp16
}

bool w4a16_shape_supported(int H, int I) {
    return (size_t)H * 2 <= (size_t)kLdsBytes && (size_t)I * 2 <= (size_t)kLdsBytes;
}

hipError_t launch_w4a16_ffn(const uint16_t* x, const int32_t* sorted_token, const int32_t* off,
                            const int32_t* active, const int32_t* n_active,
                            const smoe_w4_expert* experts, int T, int k, int H, int I, int E,
                            uint16_t* y, void* ws, int32_t* err, hipStream_t s) {
    const int rows = T * k;
    const int slots = E < rows ? E : rows;
    const int maxm = (T == 1) ? 1 : 4;  // an expert holds at most T rows
    uint16_t* h = static_cast<uint16_t*>(ws);
    const PhasePlan p1 = plan_phase(1, slots, T, H, 2 * I, I, maxm);
    W4Args a1{};
    a1.xin = x;
    a1.sorted_token = sorted_token;
    a1.off = off;
    a1.active = active;
    a1.n_active = n_active;
    a1.experts = experts;
    a1.K = H;
    a1.N = 2 * I;
    a1.I = I;
    a1.nCB = p1.nCB;
    a1.MCH = p1.mch;
    a1.XR = p1.xr;
    a1.direct = p1.direct;
    a1.T = T;
    a1.out = h;
    a1.err = err;
    hipError_t st = launch_any<1>(a1, slots, p1, maxm, s);
    if (st != hipSuccess) return st;
    const PhasePlan p2 = plan_phase(2, slots, T, I, H, I, maxm);
    W4Args a2 = a1;
    a2.xin = h;
    a2.sorted_token = nullptr;
    a2.K = I;
    a2.N = H;
    a2.nCB = p2.nCB;
    a2.MCH = p2.mch;
    a2.XR = p2.xr;
    a2.direct = 0;
    a2.out = y;
    return launch_any<2>(a2, slots, p2, maxm, s);
}
}  // namespace smoe
