// Draft routed-expert SwiGLU FFN over GPTQ INT4 (group 128) weights, one
// launch per projection across every touched expert.
//
// Cited: "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step
// Speculative Offloading" (AI summary), Key Contributions 4, and "Specter
// previews expert routing with an INT4 copy of the model itself", What
// shipped.  The draft's routed experts hold 4-bit GPTQ codes (group 128, fp16
// scales); each projection of every touched expert runs in a single launch
// over rows already grouped by expert, the codes being expanded to fp16 inside
// the kernel and the products summed in fp32.
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
#include <algorithm>

#include "common.h"
#include "gemv_core.h"
#include "maps_core.h"
#include "route_core.h"
#include "combine_core.h"

namespace {

constexpr uint32_t kMagic = 0x64006400u;

// Geometry of a GPTQ-layout matrix with BITS-bit codes as a lane group walks
// it: a "pseudo-group" is the run of packed rows one lane group holds in
// registers at a time -- one 128-K quantisation group for 2 and 4 bits, half
// of one for 8 bits (its 32 packed rows would not fit).
template <int BITS>
struct QF {
    static_assert(BITS == 2 || BITS == 4 || BITS == 8, "code width");
    static constexpr int kCodes = 32 / BITS;            // codes per packed word
    static constexpr int kWords = (BITS == 2) ? 8 : 16;  // packed rows per pseudo-group
    static constexpr int kK = kWords * kCodes;          // K per pseudo-group: 128, 128, 64
    static constexpr int kChunks = kK / 8;              // 16-byte activation chunks per pseudo-group
    static constexpr int kPerQG = 128 / kK;             // pseudo-groups per quantisation group
};
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
#ifndef SMOE_W4_MFMA
#define SMOE_W4_MFMA 1  // multi-row 4-bit steps on the MFMA kernel
#endif
#ifndef SMOE_W4_T1_MAX_WAVES
#define SMOE_W4_T1_MAX_WAVES 4
#endif
#ifndef SMOE_W4_T1_MIN_WG
#define SMOE_W4_T1_MIN_WG 128
#endif
constexpr int kMaxWaves = SMOE_W4_MAX_WAVES;  // waves per workgroup (upper bound)
// one-token (T = 1) workgroups: up to kT1MaxWaves waves, 64-column blocks
// when they give at least kT1MinWG workgroups (measured on the decode shapes:
// wider row runs beat more workgroups down to about half a workgroup per CU)
constexpr int kT1MaxWaves = SMOE_W4_T1_MAX_WAVES;
constexpr int kT1MinWG = SMOE_W4_T1_MIN_WG;
constexpr int kLdsBytes = 32 * 1024;  // activation staging budget per workgroup

// Down-projection matrix of one slot's expert, written by the gate/up launch
// of a one-token step for the down launch (e = -1: the slot has no expert).
struct SlotDesc {
    int32_t e, pad;
    smoe_w4_mat w2;
};
static_assert(sizeof(SlotDesc) == 32, "SlotDesc layout");

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
    int E;      // experts in the table
    SlotDesc* desc;  // one-token steps: per-slot down-projection matrices
    uint16_t* out;  // phase 1: h [rows, I]; phase 2: y [rows, H]
    int32_t* err;
    // per-input-channel activation divisors (AWQ-style experts) or null:
    // ascale[2 e] is expert e's fp16 [H] for w13, ascale[2 e + 1] its [I] for w2
    const uint16_t* const* ascale;
};

// A read-only int32 through the scalar cache (constant address space: the
// address must be wave-uniform; the data was written by an earlier launch).
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
SMOE_DEV int32_t ld_const(const int32_t* p) { return *(const_i32_ptr)(p); }

SMOE_DEV const uint16_t* uniform_ptr_c(const uint16_t* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo);
}

// A chunk of 8 activations divided elementwise by the channels' divisors,
// each quotient rounded to fp16 (AWQ-style experts: the weights were
// quantised after scaling their input channels by these factors).
SMOE_DEV uint4 div_chunk(uint4 x, uint4 sv) {
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
    const uint32_t ss[4] = {sv.x, sv.y, sv.z, sv.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint16_t lo = f2h(h2f((uint16_t)(xs[i] & 0xFFFFu)) / h2f((uint16_t)(ss[i] & 0xFFFFu)));
        const uint16_t hi = f2h(h2f((uint16_t)(xs[i] >> 16)) / h2f((uint16_t)(ss[i] >> 16)));
        o[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// The activation divisors of expert e for projection PHASE (null without).
template <int PHASE>
SMOE_DEV const uint16_t* expert_ascale(const W4Args& a, int e) {
    return a.ascale ? uniform_ptr_c(a.ascale[2 * e + (PHASE - 1)]) : nullptr;
}

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }
__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// Masks held in VGPRs: with a VGPR mask and the magic constant in an SGPR the
// compiler emits one v_and_or_b32 per code pair (a VOP3 op cannot take two
// scalar/literal operands on this target).
template <uint32_t C>
__device__ __forceinline__ uint32_t vgpr_const() {
    uint32_t v;
    asm("v_mov_b32 %0, %1" : "=v"(v) : "i"(C));
    return v;
}
__device__ __forceinline__ uint32_t vgpr_const_lo() { return vgpr_const<0x000F000Fu>(); }
__device__ __forceinline__ uint32_t vgpr_const_hi() { return vgpr_const<0x00F000F0u>(); }

// The code masks of a BITS-bit word, held in VGPRs.  4 bits: (0x000F000F,
// 0x00F000F0); 8 bits: 0x00FF00FF; 2 bits: 0x00030003 << 2j, j < 4.
template <int BITS>
struct Masks {
    uint32_t m[4];
    __device__ __forceinline__ Masks() {
        if constexpr (BITS == 4) {
            m[0] = vgpr_const_lo();
            m[1] = vgpr_const_hi();
        } else if constexpr (BITS == 8) {
            m[0] = vgpr_const<0x00FF00FFu>();
        } else {
            m[0] = vgpr_const<0x00030003u>();
            m[1] = vgpr_const<0x000C000Cu>();
            m[2] = vgpr_const<0x00300030u>();
            m[3] = vgpr_const<0x00C000C0u>();
        }
    }
};

// One pseudo-group of M activation rows against this lane's 4 columns.  The
// codes of a word become fp16 pairs (1024 + 2^(BITS j) q) with one and-or
// each and meet activation pairs staged to match (see permute_chunk).  With
// A_j the dot over codes of class j (code index mod 2 for 4 bits, mod 4 for
// 2 bits, a single class for 8 bits) and S_j the matching activation sums:
//   4 bits: sum (q - z) x = A_0 + A_1/16 - (1024 + z) S_0 - (64 + z) S_1
//   2 bits: sum (q - z) x = A_0 + A_1/4 + A_2/16 + A_3/64
//                           - (1024 + z) S_0 - (256 + z) S_1 - (64 + z) S_2 - (16 + z) S_3
//   8 bits: sum (q - z) x = A_0 - (1024 + z) S_0
template <int BITS, int M, int MAXM>
__device__ __forceinline__ void group_dot(const u4_t (&wv)[QF<BITS>::kWords],
                                          const uint4* __restrict__ xs,
                                          const float4* __restrict__ sums,
                                          const int (&xoff)[MAXM], const int (&soff)[MAXM],
                                          uint2 sv, uint32_t zw, const Masks<BITS>& mk,
                                          float (&acc)[MAXM][4]) {
    constexpr int NCLS = (BITS == 2) ? 4 : (BITS == 4 ? 2 : 1);
    float a[NCLS][M][4];
#pragma unroll
    for (int j = 0; j < NCLS; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int c = 0; c < 4; ++c) a[j][m][c] = 0.0f;
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < QF<4>::kWords; ++i) {
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
                const h2_t e0 = as_h2((w & mk.m[0]) | kMagic);  // 1024+q0, 1024+q4
                const h2_t o0 = as_h2((w & mk.m[1]) | kMagic);  // 1024+16q1, 1024+16q5
                const h2_t e1 = as_h2((b & mk.m[0]) | kMagic);  // 1024+q2, 1024+q6
                const h2_t o1 = as_h2((b & mk.m[1]) | kMagic);  // 1024+16q3, 1024+16q7
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    a[0][m][c] = __builtin_amdgcn_fdot2(e0, as_h2(xp[m].x), a[0][m][c], false);
                    a[1][m][c] = __builtin_amdgcn_fdot2(o0, as_h2(xp[m].y), a[1][m][c], false);
                    a[0][m][c] = __builtin_amdgcn_fdot2(e1, as_h2(xp[m].z), a[0][m][c], false);
                    a[1][m][c] = __builtin_amdgcn_fdot2(o1, as_h2(xp[m].w), a[1][m][c], false);
                }
            }
        }
    } else if constexpr (BITS == 8) {
        // two packed rows (8 K) per activation chunk
#pragma unroll
        for (int u = 0; u < QF<8>::kChunks; ++u) {
            if (SMOE_W4_ROWFENCE) __builtin_amdgcn_sched_barrier(0);
            uint4 xp[M];
#pragma unroll
            for (int m = 0; m < M; ++m) xp[m] = xs[xoff[m] + u];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t w0 = wv[2 * u][c];
                const uint32_t w1 = wv[2 * u + 1][c];
                const h2_t p0 = as_h2((w0 & mk.m[0]) | kMagic);         // 1024+q0, 1024+q2
                const h2_t p1 = as_h2(((w0 >> 8) & mk.m[0]) | kMagic);  // 1024+q1, 1024+q3
                const h2_t p2 = as_h2((w1 & mk.m[0]) | kMagic);         // 1024+q4, 1024+q6
                const h2_t p3 = as_h2(((w1 >> 8) & mk.m[0]) | kMagic);  // 1024+q5, 1024+q7
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    a[0][m][c] = __builtin_amdgcn_fdot2(p0, as_h2(xp[m].x), a[0][m][c], false);
                    a[0][m][c] = __builtin_amdgcn_fdot2(p1, as_h2(xp[m].y), a[0][m][c], false);
                    a[0][m][c] = __builtin_amdgcn_fdot2(p2, as_h2(xp[m].z), a[0][m][c], false);
                    a[0][m][c] = __builtin_amdgcn_fdot2(p3, as_h2(xp[m].w), a[0][m][c], false);
                }
            }
        }
    } else {
        // one packed row (16 K) per two activation chunks
#pragma unroll
        for (int i = 0; i < QF<2>::kWords; ++i) {
            if (SMOE_W4_ROWFENCE) __builtin_amdgcn_sched_barrier(0);
            uint4 xa[M], xb[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                xa[m] = xs[xoff[m] + 2 * i];
                xb[m] = xs[xoff[m] + 2 * i + 1];
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t w = wv[i][c];
                const uint32_t b = w >> 8;
                h2_t pw[4], pb[4];  // class j: 1024 + 4^j q (codes j, j+8 and j+4, j+12)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pw[j] = as_h2((w & mk.m[j]) | kMagic);
                    pb[j] = as_h2((b & mk.m[j]) | kMagic);
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const uint32_t xav[4] = {xa[m].x, xa[m].y, xa[m].z, xa[m].w};
                    const uint32_t xbv[4] = {xb[m].x, xb[m].y, xb[m].z, xb[m].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        a[j][m][c] = __builtin_amdgcn_fdot2(pw[j], as_h2(xav[j]), a[j][m][c], false);
                        a[j][m][c] = __builtin_amdgcn_fdot2(pb[j], as_h2(xbv[j]), a[j][m][c], false);
                    }
                }
            }
        }
    }
    float4 se[M];
#pragma unroll
    for (int m = 0; m < M; ++m) se[m] = sums[soff[m]];
    const uint32_t sw[2] = {sv.x, sv.y};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float s = h2f((uint16_t)(sw[c >> 1] >> (16 * (c & 1))));
        const float z = (float)((zw >> (BITS * c)) & ((1u << BITS) - 1u));
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float t;
            if constexpr (BITS == 4) {
                t = a[0][m][c] + 0.0625f * a[1][m][c];
                t -= (1024.0f + z) * se[m].x;
                t -= (64.0f + z) * se[m].y;
            } else if constexpr (BITS == 8) {
                t = a[0][m][c];
                t -= (1024.0f + z) * se[m].x;
            } else {
                t = a[0][m][c] + 0.25f * a[1][m][c] + 0.0625f * a[2][m][c] +
                    0.015625f * a[3][m][c];
                t -= (1024.0f + z) * se[m].x;
                t -= (256.0f + z) * se[m].y;
                t -= (64.0f + z) * se[m].z;
                t -= (16.0f + z) * se[m].w;
            }
            acc[m][c] += s * t;
        }
    }
}

template <int BITS>
struct GroupLoad {
    u4_t w[QF<BITS>::kWords];
    uint2 s;
    uint32_t z;
};

// Packed weights are read through a buffer resource: the lane's byte offset
// (column and group) is one VGPR and the packed-row stride a scalar offset,
// so a group's 16 row addresses cost no vector registers.
struct W4Src {
    __amdgpu_buffer_rsrc_t q;  // qweight [K*BITS/32, N] int32
    smoe_w4_mat m;
    int N;
};

constexpr int kBufWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family
constexpr int kAuxNT = 2;              // non-temporal (streamed once)

// A workgroup-uniform pointer as scalar registers (the matrix of one expert
// is the same for every lane), so its buffer resource needs no per-lane
// handling.
template <typename T>
SMOE_DEV T* uniform_ptr(T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

template <int BITS>
__device__ __forceinline__ W4Src make_src(const smoe_w4_mat& mm, int K, int N) {
    smoe_w4_mat m;
    m.qweight = uniform_ptr(mm.qweight);
    m.scales = uniform_ptr(mm.scales);
    m.qzeros = uniform_ptr(mm.qzeros);
    W4Src s;
    s.q = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(m.qweight), (short)0,
                                            (K / QF<BITS>::kCodes) * N * 4, kBufWord3);
    s.m = m;
    s.N = N;
    return s;
}

// Every load is unconditional (a column past N reads column 0; its sums are
// never stored), so the loads in flight are a static count and the waits the
// compiler places for older loads (the activation row) leave them in flight.
template <int BITS>
__device__ __forceinline__ void load_group(GroupLoad<BITS>& L, const W4Src& src, int g, int col,
                                           bool colok) {
    using F = QF<BITS>;
    const int N = src.N;
    const int c = colok ? col : 0;
    const int qg = g / F::kPerQG;  // quantisation group
    const int voff = ((g * F::kWords) * N + c) * 4;
#pragma unroll
    for (int i = 0; i < F::kWords; ++i)
        L.w[i] = __builtin_amdgcn_raw_buffer_load_b128(src.q, voff, i * N * 4, kAuxNT);
    const uint64_t sv =
        *as_global(reinterpret_cast<const uint64_t*>(src.m.scales + (size_t)qg * N + c));
    L.s = make_uint2((uint32_t)sv, (uint32_t)(sv >> 32));
    // the word holding this lane's 4 zeros (shifted when the group is
    // consumed, so that issuing the loads waits for none of them)
    L.z = (uint32_t)*as_global(src.m.qzeros + (size_t)qg * (N / F::kCodes) + (c / F::kCodes));
}

// Shift of a lane's first zero inside its zero word (columns are 4-aligned).
template <int BITS>
SMOE_DEV int zero_shift(int col) { return BITS * (col & (QF<BITS>::kCodes - 1)); }

template <int BITS, int MAXM>
__device__ __forceinline__ void group_step(const GroupLoad<BITS>& L, const uint4* xs,
                                           const float4* sums, const int (&xrow)[MAXM], int g,
                                           int K8, int G, int M, int zsh, const Masks<BITS>& mk,
                                           float (&acc)[MAXM][4]) {
    const uint32_t zw = L.z >> zsh;
    int xoff[MAXM], soff[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        xoff[m] = xrow[m] * K8 + g * QF<BITS>::kChunks;
        soff[m] = xrow[m] * G + g;
    }
    if (MAXM == 1) {
        group_dot<BITS, 1, MAXM>(L.w, xs, sums, xoff, soff, L.s, zw, mk, acc);
    } else {
        switch (M) {
            case 1: group_dot<BITS, 1, MAXM>(L.w, xs, sums, xoff, soff, L.s, zw, mk, acc); break;
            case 2: group_dot<BITS, (MAXM >= 2 ? 2 : 1), MAXM>(L.w, xs, sums, xoff, soff, L.s, zw, mk, acc); break;
            case 3: group_dot<BITS, (MAXM >= 3 ? 3 : 1), MAXM>(L.w, xs, sums, xoff, soff, L.s, zw, mk, acc); break;
            default: group_dot<BITS, MAXM, MAXM>(L.w, xs, sums, xoff, soff, L.s, zw, mk, acc); break;
        }
    }
}

// Activations as the dot2 pairs the dequantised codes meet.  4 bits: (x0,x4),
// (x1,x5), (x2,x6), (x3,x7) of each 8-element chunk; 8 bits: (x0,x2),
// (x1,x3), (x4,x6), (x5,x7).  2 bits pair elements 8 apart, so a pair of
// chunks is permuted together (permute_chunk_pair).
template <int BITS>
__device__ __forceinline__ uint4 permute_chunk(uint4 d) {
    uint4 p;
    if constexpr (BITS == 4) {
        p.x = (d.x & 0xFFFFu) | (d.z << 16);      // (x0, x4)
        p.y = (d.x >> 16) | (d.z & 0xFFFF0000u);  // (x1, x5)
        p.z = (d.y & 0xFFFFu) | (d.w << 16);      // (x2, x6)
        p.w = (d.y >> 16) | (d.w & 0xFFFF0000u);  // (x3, x7)
    } else if constexpr (BITS == 8) {
        p.x = (d.x & 0xFFFFu) | (d.y << 16);      // (x0, x2)
        p.y = (d.x >> 16) | (d.y & 0xFFFF0000u);  // (x1, x3)
        p.z = (d.z & 0xFFFFu) | (d.w << 16);      // (x4, x6)
        p.w = (d.z >> 16) | (d.w & 0xFFFF0000u);  // (x5, x7)
    } else {
        p = d;  // 2 bits: natural order here, paired by permute_chunk_pair
    }
    return p;
}

// 2 bits: chunks d0 = x0..x7, d1 = x8..x15 of one packed row become
// (x0,x8), (x1,x9), (x2,x10), (x3,x11) and (x4,x12), ..., (x7,x15).
__device__ __forceinline__ void permute_chunk_pair(uint4 d0, uint4 d1, uint4& pa, uint4& pb) {
    pa.x = (d0.x & 0xFFFFu) | (d1.x << 16);
    pa.y = (d0.x >> 16) | (d1.x & 0xFFFF0000u);
    pa.z = (d0.y & 0xFFFFu) | (d1.y << 16);
    pa.w = (d0.y >> 16) | (d1.y & 0xFFFF0000u);
    pb.x = (d0.z & 0xFFFFu) | (d1.z << 16);
    pb.y = (d0.z >> 16) | (d1.z & 0xFFFF0000u);
    pb.z = (d0.w & 0xFFFFu) | (d1.w << 16);
    pb.w = (d0.w >> 16) | (d1.w & 0xFFFF0000u);
}

// After the chunks of `nrows` rows are in LDS (permuted for 4 and 8 bits,
// natural for 2 bits): pair the 2-bit chunks in place, then the per-class
// activation sums of every (row, pseudo-group).  Ends with a barrier.
template <int BITS>
__device__ __forceinline__ void finish_rows(uint4* xs, float4* sums, int nrows, int K8, int G) {
    using F = QF<BITS>;
    if constexpr (BITS == 2) {
        __syncthreads();
#pragma unroll 1
        for (int idx = threadIdx.x; idx < nrows * (K8 / 2); idx += blockDim.x) {
            uint4* c = xs + 2 * idx;  // rows hold K8 chunks, K8 even
            uint4 pa, pb;
            permute_chunk_pair(c[0], c[1], pa, pb);
            c[0] = pa;
            c[1] = pb;
        }
    }
    __syncthreads();
#pragma unroll 1
    for (int idx = threadIdx.x; idx < nrows * G; idx += blockDim.x) {
        const int j = idx / G;
        const int gg = idx - j * G;
        const uint4* xr = xs + j * K8 + gg * F::kChunks;
        float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
        for (int i = 0; i < F::kChunks; ++i) {
            const uint4 p = xr[i];
            const h2_t x0 = as_h2(p.x), x1 = as_h2(p.y), x2 = as_h2(p.z), x3 = as_h2(p.w);
            if constexpr (BITS == 4) {
                s4[0] += ((float)x0.x + (float)x0.y) + ((float)x2.x + (float)x2.y);
                s4[1] += ((float)x1.x + (float)x1.y) + ((float)x3.x + (float)x3.y);
            } else if constexpr (BITS == 8) {
                s4[0] += (((float)x0.x + (float)x0.y) + ((float)x1.x + (float)x1.y)) +
                         (((float)x2.x + (float)x2.y) + ((float)x3.x + (float)x3.y));
            } else {
                s4[0] += (float)x0.x + (float)x0.y;
                s4[1] += (float)x1.x + (float)x1.y;
                s4[2] += (float)x2.x + (float)x2.y;
                s4[3] += (float)x3.x + (float)x3.y;
            }
        }
        sums[j * G + gg] = make_float4(s4[0], s4[1], s4[2], s4[3]);
    }
    __syncthreads();
}

// finish_rows<4> for chunks staged in natural order: each (row, group)'s
// chunks are read, permuted in place and summed as finish_rows<4> sums the
// permuted chunks (the same values in the same order).  The caller has made
// every chunk visible (waits and a barrier); ends with a barrier.
__device__ __forceinline__ void finish_rows_natural4(uint4* xs, float4* sums, int nrows, int K8,
                                                     int G) {
#pragma unroll 1
    for (int idx = threadIdx.x; idx < nrows * G; idx += blockDim.x) {
        const int j = idx / G;
        const int gg = idx - j * G;
        uint4* xr = xs + j * K8 + gg * 16;
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll 4
        for (int i = 0; i < 16; ++i) {
            const uint4 p = permute_chunk<4>(xr[i]);
            xr[i] = p;
            const h2_t x0 = as_h2(p.x), x1 = as_h2(p.y), x2 = as_h2(p.z), x3 = as_h2(p.w);
            s0 += ((float)x0.x + (float)x0.y) + ((float)x2.x + (float)x2.y);
            s1 += ((float)x1.x + (float)x1.y) + ((float)x3.x + (float)x3.y);
        }
        sums[j * G + gg] = make_float4(s0, s1, 0.0f, 0.0f);
    }
    __syncthreads();
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Stage activation rows src_row(j), j < nrows, into LDS rows 0..nrows-1 as
// dot2 pairs, then their per-class sums.
template <int BITS, typename RowPtr>
__device__ __forceinline__ void stage_rows(uint4* xs, float4* sums, int nrows, int K8, int G,
                                           RowPtr src_row, const uint16_t* as = nullptr) {
    const uint4* as4 = reinterpret_cast<const uint4*>(as);
#pragma unroll 1
    for (int idx = threadIdx.x; idx < nrows * K8; idx += blockDim.x) {
        const int j = idx / K8;
        const int rr = idx - j * K8;
        uint4 v = src_row(j)[rr];
        if (as4) v = div_chunk(v, as4[rr]);
        xs[j * K8 + rr] = permute_chunk<BITS>(v);
    }
    finish_rows<BITS>(xs, sums, nrows, K8, G);
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
template <int BITS, bool kPrefetch, int MAXM>
__device__ __forceinline__ void run_groups(GroupLoad<BITS>& cur, int g, int nslots, int G,
                                           const W4Src& src, int col, bool colok,
                                           const uint4* xs, const float4* sums,
                                           const int (&xrow)[MAXM], int K8, int M,
                                           const Masks<BITS>& mk, float (&acc)[MAXM][4]) {
    if (g >= G) return;
    for (;;) {
        const int gn = g + nslots;
        GroupLoad<BITS> nxt;
        if (kPrefetch && gn < G) load_group<BITS>(nxt, src, gn, col, colok);
        group_step<BITS, MAXM>(cur, xs, sums, xrow, g, K8, G, M, zero_shift<BITS>(col), mk, acc);
        if (gn >= G) break;
        if (!kPrefetch) load_group<BITS>(nxt, src, gn, col, colok);
        cur = nxt;
        g = gn;
    }
}

constexpr int kRowChunksPerThread = 8;  // activation chunks per thread requested early
constexpr int kSpecTable = 64;          // experts whose descriptors are read speculatively

// Request the first kRowChunksPerThread chunks of an activation row per
// thread.  The requests are unconditional (indexes past the row repeat its
// last chunk) so that the number of loads in flight is static and a later
// wait for older loads does not also wait for the row.
SMOE_DEV void request_row(const uint4* row4, int K8, uint4 (&xv)[kRowChunksPerThread]) {
#pragma unroll
    for (int u = 0; u < kRowChunksPerThread; ++u) {
        const int idx = threadIdx.x + u * (int)blockDim.x;
        xv[u] = row4[idx < K8 ? idx : K8 - 1];
    }
}

SMOE_DEV const void* bcast_ptr(const void* p, int src_lane) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src_lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src_lane);
    return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// The projection's matrix descriptor of every expert, one per lane, requested
// before the active list is read (tables of at most kSpecTable experts), so
// that the expert's weights are requested one memory round trip after the
// launch instead of two.
SMOE_DEV smoe_w4_expert spec_table(const W4Args& a, int lane) {
    smoe_w4_expert m{{nullptr, nullptr, nullptr}, {nullptr, nullptr, nullptr}};
    if (a.E <= kSpecTable && lane < a.E) m = a.experts[lane];
    return m;
}

template <int PHASE>
SMOE_DEV smoe_w4_mat pick_mat(const W4Args& a, const smoe_w4_expert& spec, int e) {
    if (a.E > kSpecTable) {
        // larger tables: the entry itself, through the scalar cache (the
        // table is read-only here), so no vector-load wait is involved
        using cptr = const __attribute__((address_space(4))) uint64_t*;
        static_assert(sizeof(smoe_w4_expert) == 6 * sizeof(uint64_t), "expert table layout");
        const cptr t = (cptr)a.experts;
        const int b = 6 * e + (PHASE == 1 ? 0 : 3);
        smoe_w4_mat m;
        m.qweight = reinterpret_cast<const int32_t*>(t[b]);
        m.scales = reinterpret_cast<const uint16_t*>(t[b + 1]);
        m.qzeros = reinterpret_cast<const int32_t*>(t[b + 2]);
        return m;
    }
    const smoe_w4_mat& sm = (PHASE == 1) ? spec.w13 : spec.w2;
    smoe_w4_mat m;
    m.qweight = static_cast<const int32_t*>(bcast_ptr(sm.qweight, e));
    m.scales = static_cast<const uint16_t*>(bcast_ptr(sm.scales, e));
    m.qzeros = static_cast<const int32_t*>(bcast_ptr(sm.qzeros, e));
    return m;
}

// The gate/up launch of a one-token step hands each slot's expert and its
// down-projection matrix to the down launch, which thus reads them from a
// recently written line instead of the expert table.
SMOE_DEV void write_slot_desc(const W4Args& a, const smoe_w4_expert& spec, int slot, int e) {
    smoe_w4_mat w2{nullptr, nullptr, nullptr};
    if (e >= 0) w2 = pick_mat<2>(a, spec, e);
    if (threadIdx.x == 0) {
        SlotDesc d;
        d.e = e;
        d.pad = 0;
        d.w2 = w2;
        a.desc[slot] = d;
    }
}

// LDS layout of a workgroup: the activation rows as dot2 pairs, their group
// sums, then the slots' partial sums.
struct W4Lds {
    uint4* xs;     // [XR][K8]
    float4* sums;  // [XR][G] per-class activation sums of each pseudo-group
    float* red;    // [nslots][MAXM][NB]
};

template <int BITS>
SMOE_DEV W4Lds carve_lds(uint4* smem, const W4Args& a) {
    const int K8 = a.K >> 3, G = a.K / QF<BITS>::kK;
    W4Lds l;
    l.xs = smem;
    l.sums = reinterpret_cast<float4*>(smem + (size_t)a.XR * K8);
    l.red = reinterpret_cast<float*>(l.sums + (size_t)a.XR * G);
    return l;
}

// First weight column of a lane: in the gate/up projection lanes q < LPR/2
// take gate columns and the others the matching up columns.
template <int PHASE, int LPR>
SMOE_DEV int lane_column(const W4Args& a, int cb, int q) {
    constexpr int NB = 4 * LPR;
    if (PHASE == 1)
        return (q < LPR / 2) ? cb * (NB / 2) + 4 * q : a.I + cb * (NB / 2) + 4 * (q - LPR / 2);
    return cb * NB + 4 * q;
}

// Group g of a one-token slot (g >= G: a slot past the reduction, whose loads
// read group G - 1 and whose contribution is dropped).
SMOE_DEV int clamp_group(int g, int G) { return g < G ? g : G - 1; }

template <int BITS>
SMOE_DEV void step_if(const GroupLoad<BITS>& L, const W4Lds& l, int g, int G, int K8, int zsh,
                      const Masks<BITS>& mk, float (&acc)[1][4]) {
    float t[1][4] = {{0.0f, 0.0f, 0.0f, 0.0f}};
    const int xrow[1] = {0};
    group_step<BITS, 1>(L, l.xs, l.sums, xrow, clamp_group(g, G), K8, G, 1, zsh, mk, t);
    const bool valid = g < G;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[0][c] += valid ? t[0][c] : 0.0f;
}

// Epilogue of a one-token block: the lane groups' partial sums of the column
// block added in a fixed order -- inside each wave across its 64 / LPR lane
// groups by a butterfly over lane distances LPR, 2 LPR, ..., then the waves'
// sums in increasing wave order through LDS -- and SwiGLU (gate/up projection,
// into h) or the plain sum (down projection, into y) stored.  One barrier; no
// thread adds more than one partial per wave.
template <int PHASE, int LPR>
SMOE_DEV void reduce_store_t1(const W4Args& a, float* red, float (&acc)[1][4], int q, int cb,
                              int slot) {
    constexpr int NB = 4 * LPR;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nw = (int)(blockDim.x >> 6);
#pragma unroll
    for (int d = LPR; d < 64; d *= 2)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[0][c] += __shfl_xor(acc[0][c], d);
    if (lane < LPR)
#pragma unroll
        for (int c = 0; c < 4; ++c) red[wave * NB + 4 * q + c] = acc[0][c];
    __syncthreads();
    if (PHASE == 1) {
        // red[w][j] is gate column j, red[w][NB/2 + j] the matching up column
        if (tid < NB / 2) {
            float gv = 0.0f, uv = 0.0f;
            for (int w = 0; w < nw; ++w) {
                gv += red[w * NB + tid];
                uv += red[w * NB + NB / 2 + tid];
            }
            a.out[(size_t)slot * a.I + cb * (NB / 2) + tid] = f2h(silu_f(gv) * uv);
        }
    } else if (tid < NB && cb * NB + tid < a.N) {
        float v = 0.0f;
        for (int w = 0; w < nw; ++w) v += red[w * NB + tid];
        a.out[(size_t)slot * a.N + cb * NB + tid] = f2h(v);
    }
}

// One activation row (T = 1) against the column block cb of matrix wm; each
// slot takes groups myslot + j * nslots, j < NG.  xv holds the row's chunks,
// requested by the caller.  The slot's groups go through two register
// buffers in straight-line code.  The first group is requested before the
// row is permuted into LDS; the second only after the first has been
// consumed when NG == 2 (a wave whose requests stall for the memory pipeline
// to drain would otherwise reach its arithmetic only once every group of it
// is in flight, late in the launch); with three or four groups the second is
// requested up front and a buffer is refilled as soon as it has been
// consumed, so every wait is for one group while the next is in flight.
template <int BITS, int PHASE, int LPR, int NG>
SMOE_DEV void one_token_block(const W4Args& a, const W4Lds& l, const smoe_w4_mat& wm,
                              uint4 (&xv)[kRowChunksPerThread], int slot, int cb,
                              const uint16_t* as = nullptr) {
    static_assert(NG >= 1 && NG <= 4, "groups per slot");
    constexpr int RPL = 64 / LPR;
    constexpr int NB = 4 * LPR;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int nslots = (int)(blockDim.x >> 6) * RPL;
    const int myslot = (tid >> 6) * RPL + lane / LPR;
    const int q = lane % LPR;
    const int K = a.K, N = a.N;
    const int G = K / QF<BITS>::kK;
    const int K8 = K >> 3;
    const int col = lane_column<PHASE, LPR>(a, cb, q);
    const bool colok = col < N;
    const int zsh = zero_shift<BITS>(col);
    const Masks<BITS> mk;
    if (!wm.qweight || !wm.scales || !wm.qzeros || (a.ascale && !as)) {
        if (tid == 0 && cb == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
        return;
    }
    if (as) {
        // AWQ-style divisors: requested with the row, before any weight
        uint4 sv[kRowChunksPerThread];
        request_row(reinterpret_cast<const uint4*>(as), K8, sv);
#pragma unroll
        for (int u = 0; u < kRowChunksPerThread; ++u) xv[u] = div_chunk(xv[u], sv[u]);
    }
    const W4Src src = make_src<BITS>(wm, K, N);
    const int g0 = myslot;
    GroupLoad<BITS> A, B;
    load_group<BITS>(A, src, clamp_group(g0, G), col, colok);
    if (NG >= 3) load_group<BITS>(B, src, clamp_group(g0 + nslots, G), col, colok);
    __builtin_amdgcn_sched_barrier(0);  // every request above is issued before the row is staged
    // straight-line stores (indexes past the row rewrite its last chunk with
    // the same value), so the wait for the row leaves the weights in flight;
    // the launch guarantees kRowChunksPerThread * blockDim >= K8
#pragma unroll
    for (int u = 0; u < kRowChunksPerThread; ++u) {
        const int idx = tid + u * (int)blockDim.x;
        l.xs[idx < K8 ? idx : K8 - 1] = permute_chunk<BITS>(xv[u]);
    }
    finish_rows<BITS>(l.xs, l.sums, 1, K8, G);
    float acc[1][4] = {{0.0f, 0.0f, 0.0f, 0.0f}};
    step_if<BITS>(A, l, g0, G, K8, zsh, mk, acc);
    if (NG == 2) {
        load_group<BITS>(B, src, clamp_group(g0 + nslots, G), col, colok);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (NG >= 3) load_group<BITS>(A, src, clamp_group(g0 + 2 * nslots, G), col, colok);
    if (NG >= 2) step_if<BITS>(B, l, g0 + nslots, G, K8, zsh, mk, acc);
    if (NG >= 4) load_group<BITS>(B, src, clamp_group(g0 + 3 * nslots, G), col, colok);
    if (NG >= 3) step_if<BITS>(A, l, g0 + 2 * nslots, G, K8, zsh, mk, acc);
    if (NG >= 4) step_if<BITS>(B, l, g0 + 3 * nslots, G, K8, zsh, mk, acc);
    reduce_store_t1<PHASE, LPR>(a, l.red, acc, q, cb, slot);
}

// Occupancy of the one-token kernels: four waves per SIMD with one group per
// slot (at most 128 registers), two with two or more.
template <int MAXM, int NG>
constexpr int w4_waves_per_eu() { return (MAXM == 1 && NG == 1) ? 4 : 2; }

template <int BITS, int PHASE, int LPR, int MAXM, int NG>
__global__ __launch_bounds__(64 * (MAXM == 1 ? kT1MaxWaves : kMaxWaves))
__attribute__((amdgpu_waves_per_eu(w4_waves_per_eu<MAXM, NG>()))) void w4_kernel(W4Args a) {
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
    const int G = K / QF<BITS>::kK;
    const int K8 = K >> 3;
    const W4Lds l = carve_lds<BITS>(smem, a);
    uint4* xs = l.xs;
    float4* sums = l.sums;
    float* red = l.red;

    const int nslots = nwaves * RPL;
    const int myslot = wave * RPL + rho;
    const int col = lane_column<PHASE, LPR>(a, cb, q);
    const bool colok = col < N;

    if constexpr (MAXM == 1) {
        // One token (T = 1): every pair's token is 0, and the touched experts
        // in increasing id (the active list) own sorted rows 0, 1, ... in
        // that order, so this slot's activation row is known before the maps
        // are read: x row 0 (gate/up) or h row `slot` (down).  It is
        // requested first, then the expert's first weights; the row is
        // permuted into LDS while both are in flight.
        const uint4* row4 =
            reinterpret_cast<const uint4*>((PHASE == 1) ? a.xin : a.xin + (size_t)slot * K);
        uint4 xv[kRowChunksPerThread];
        if (PHASE == 1) {
            const smoe_w4_expert spec = spec_table(a, lane);
            int e = a.active[slot];  // -1 past the touched experts
            request_row(row4, K8, xv);
            if (e >= a.E) {
                if (tid == 0 && cb == 0) flag_error(a.err, SMOE_DERR_BAD_ID);
                e = -1;
            }
            if (cb == 0) write_slot_desc(a, spec, slot, e);
            if (e < 0) return;
            one_token_block<BITS, 1, LPR, NG>(a, l, pick_mat<1>(a, spec, e), xv, slot, cb,
                                              expert_ascale<1>(a, e));
        } else {
            const SlotDesc d = a.desc[slot];
            request_row(row4, K8, xv);
            if (d.e < 0) return;
            one_token_block<BITS, 2, LPR, NG>(a, l, d.w2, xv, slot, cb, expert_ascale<2>(a, d.e));
        }
        return;
    } else {
        const int e = a.active[slot];  // -1 past the touched experts
        if (e < 0) return;
        const smoe_w4_mat wm = (PHASE == 1) ? a.experts[e].w13 : a.experts[e].w2;
        const uint16_t* as = expert_ascale<PHASE>(a, e);
        const int r0 = a.off[e];
        const int r1 = a.off[e + 1];
        if (!wm.qweight || !wm.scales || !wm.qzeros || (a.ascale && !as)) {
            if (tid == 0 && cb == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
            return;
        }
        const W4Src src = make_src<BITS>(wm, K, N);
        const Masks<BITS> mk;
        // The gate/up projection with every token fitting in LDS stages all
        // T activation rows once.
        const bool direct = (PHASE == 1) && a.direct;
        if (direct)
            stage_rows<BITS>(xs, sums, a.T, K8, G, [&](int j) {
                return reinterpret_cast<const uint4*>(a.xin + (size_t)j * K);
            }, as);
        for (int mc = r0; mc < r1; mc += a.MCH) {
            const int M = min(a.MCH, r1 - mc);
            int xrow[MAXM];
#pragma unroll
            for (int m = 0; m < MAXM; ++m)
                xrow[m] = direct ? a.sorted_token[mc + (m < M ? m : 0)] : m;
            if (!direct) {
                if (PHASE == 1)
                    stage_rows<BITS>(xs, sums, M, K8, G, [&](int j) {
                        return reinterpret_cast<const uint4*>(a.xin +
                                                              (size_t)a.sorted_token[mc + j] * K);
                    }, as);
                else
                    stage_rows<BITS>(xs, sums, M, K8, G, [&](int j) {
                        return reinterpret_cast<const uint4*>(a.xin + (size_t)(mc + j) * K);
                    }, as);
            }
            GroupLoad<BITS> cur;
            const int g = myslot;
            if (g < G) load_group<BITS>(cur, src, g, col, colok);
            float acc[MAXM][4];
#pragma unroll
            for (int m = 0; m < MAXM; ++m)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[m][c] = 0.0f;
            run_groups<BITS, false, MAXM>(cur, g, nslots, G, src, col, colok, xs, sums, xrow, K8,
                                          M, mk, acc);
            reduce_store<PHASE, MAXM, NB>(a, red, acc, myslot, nslots, q, cb, mc, M);
        }
    }
}

// ------------------------------------------ multi-row 4-bit path on MFMA ----
//
// With several rows per expert the dot products dominate the VALU path (four
// dot2 per packed word and row).  Here the dequantised codes are the B
// operand of v_mfma_f32_16x16x32_f16 and up to 16 activation rows its A
// operand, so a word costs its 5 dequantisation ops whatever the row count.
// Lane l holds columns 4(l%16)..+3 (one 16-byte load per packed row) at
// packed row 4j + l/16 of each 32-K step j: word c of the load is exactly
// the B fragment (8 K of one column) of the c-th MFMA, whose 16 columns are
// 4(l%16) + c.  The fp16 pairs (1024+q, 1024+16q) meet activation pairs
// staged as for the VALU path, with the (1024+16q) halves' activations
// scaled by 1/16 in registers, so one accumulator per column set sums
//   sum_even (1024+q) x + sum_odd (64+q) x;
// the constant parts and the zero come off per 128-K group with the group's
// activation sums, then the fp16 scale.  The 4 waves take groups g = wave,
// wave + 4, ... through two register buffers (loads of the next two groups
// in flight while one is multiplied) and add their tiles through LDS.
// Gathered activation rows take their token indices through scalar loads
// issued together, so staging a chunk costs one dependent round trip (with
// vector loads each row's index load waited for the row loads before it).
// Measured against the form with vector index loads, on the DeepSeek-V2-Lite
// draft layer step: T = 16 104.0 -> 99.4 us, T = 4 65.5 -> 64.0 us; the down
// projection at four waves per SIMD (127 VGPRs) a further 2.6 us at T = 16.
// Four buffers (every group of a wave requested up front; 201 VGPRs, two
// waves per SIMD) were slower: 72.2 and 119.7 us.  Staging the rows with
// global->LDS loads instead of through registers frees 32 VGPRs (153 -> 122
// for the gate/up projection: four waves per SIMD, four workgroups per CU):
// layer step T = 4 52.2 -> 49.1 us, T = 16 90.4 -> 85.1 us.
#ifndef SMOE_W4_MFMA_WAVES
#define SMOE_W4_MFMA_WAVES 4
#endif
#ifndef SMOE_W4_MFMA_WPE
#define SMOE_W4_MFMA_WPE 2
#endif
#ifndef SMOE_W4_MFMA_WPE2
#define SMOE_W4_MFMA_WPE2 4  // down projection (127 VGPRs)
#endif
#ifndef SMOE_W4_MFMA_BUFS
#define SMOE_W4_MFMA_BUFS 2
#endif
#ifndef SMOE_W4_MFMA_DMA
#define SMOE_W4_MFMA_DMA 1  // activation rows staged by global->LDS loads
#endif
constexpr int kMfmaWaves = SMOE_W4_MFMA_WAVES;
#ifndef SMOE_W4_MFMA_WAVES2
#define SMOE_W4_MFMA_WAVES2 SMOE_W4_MFMA_WAVES  // down projection
#endif
template <int PHASE>
constexpr int mfma_waves() { return PHASE == 1 ? SMOE_W4_MFMA_WAVES : SMOE_W4_MFMA_WAVES2; }
// the reduction area (>= waves * 256 bytes) absorbs a row load's overrun
static_assert(mfma_waves<1>() >= 4 && mfma_waves<2>() >= 4, "at least 4 waves per workgroup");
constexpr int kMfmaBufs = SMOE_W4_MFMA_BUFS;  // groups of a wave in flight
constexpr int kMfmaRows = 16;
constexpr int kMfmaLdsBytes = 32 * 1024;  // activation staging budget

struct MfmaLoad {
    u4_t w[4];  // packed rows 4j + l/16 of the group, 4 columns each
    uint2 s;
    uint32_t z;
};

// Group g of this lane's columns; a group past the reduction (g >= G) reads
// nothing: its packed words come from an offset past the buffer's records,
// which returns zeros without a memory access (they are never multiplied),
// and its scale and zero words from group G - 1.  The request count is the
// same either way, so the compiler's waits stay exact.
__device__ __forceinline__ void mfma_load(MfmaLoad& L, const W4Src& src, int g, int G, int col,
                                          int kq) {
    const int N = src.N;
    const bool live = g < G;
    const int gc = live ? g : G - 1;
    const int voff = live ? ((gc * 16 + kq) * N + col) * 4 : 0x7FFFFFF0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        L.w[j] = __builtin_amdgcn_raw_buffer_load_b128(src.q, voff, 4 * j * N * 4, kAuxNT);
    const uint64_t sv =
        *as_global(reinterpret_cast<const uint64_t*>(src.m.scales + (size_t)gc * N + col));
    L.s = make_uint2((uint32_t)sv, (uint32_t)(sv >> 32));
    L.z = (uint32_t)*as_global(src.m.qzeros + (size_t)gc * (N >> 3) + (col >> 3));
}

// One 128-K group into acc (acc[c][i]: row 4(l/16)+i, column 4(l%16)+c).
__device__ __forceinline__ void mfma_group(const MfmaLoad& L, const uint4* __restrict__ xs,
                                           const float4* __restrict__ sums, int arow, bool aok,
                                           const int (&drow)[4], int g, int K8, int G, int kq,
                                           int zsh, const Masks<4>& mk, f4_t (&acc)[4]) {
    f4_t d[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) d[c] = f4_t{0.f, 0.f, 0.f, 0.f};
    const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint4 xp = aok ? xs[arow * K8 + g * 16 + 4 * j + kq] : make_uint4(0, 0, 0, 0);
        xp.y = __builtin_bit_cast(uint32_t, as_h2(xp.y) * sixteenth);
        xp.w = __builtin_bit_cast(uint32_t, as_h2(xp.w) * sixteenth);
        const h8_t av = __builtin_bit_cast(h8_t, xp);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t w = L.w[j][c];
            const uint32_t b = w >> 8;
            const u4_t bw = {(w & mk.m[0]) | kMagic, (w & mk.m[1]) | kMagic,
                             (b & mk.m[0]) | kMagic, (b & mk.m[1]) | kMagic};
            d[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(h8_t, bw), d[c],
                                                          0, 0, 0);
        }
    }
    float4 se[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) se[i] = sums[drow[i] * G + g];
    const uint32_t zw = L.z >> zsh;
    const uint32_t sw[2] = {L.s.x, L.s.y};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float s = h2f((uint16_t)(sw[c >> 1] >> (16 * (c & 1))));
        const float z = (float)((zw >> (4 * c)) & 0xFu);
        const float ce = 1024.0f + z, co = 64.0f + z;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float t = d[c][i];
            t -= ce * se[i].x;
            t -= co * se[i].y;
            acc[c][i] += s * t;
        }
    }
}

// A dense shared expert (FP16 w13 [2 Is, H], w2 [H, Is], the nn.Linear
// layout of the verify path) over the T rows of a multi-row step, as extra
// workgroups of the multi-row launches (from workgroup wg0 on) or as launches
// of its own.
struct RowsShared {
    const uint16_t* w;    // phase 1: w13; phase 2: w2
    const uint16_t* xin;  // phase 1: x [T, H]; phase 2: the shared h [T, Is]
    uint16_t* out;        // phase 1: h [T, Is]; phase 2: the shared output [T, H]
    int K, Ncol, Is;      // reduction length, output columns, shared intermediate
    int rows;             // T
    int wg0;              // first shared workgroup of the launch (nfront == 0)
    int nfront;           // > 0: the launch's first nfront workgroups are the shared ones
};

// Column b * waves + wave of the shared projection, one column per wave,
// through verify_grouped_gemm's matrix-vector routine (every weight chunk of
// the column requested at once, then the rows one at a time; gemv_core.h), so
// the values are bit-identical to that call's over the same rows.
template <int PHASE, int CPL>
SMOE_DEV void shared_rows_item(const RowsShared& sh, int b) {
    constexpr int NM = (PHASE == 1) ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int n = b * (int)(blockDim.x >> 6) + (int)(threadIdx.x >> 6);
    const int nc = n < sh.Ncol ? n : sh.Ncol - 1;  // loads stay in the matrix
    u4_t wv[NM][CPL];
    smoe_gemv::gemv_load_w<NM, CPL>(sh.w, sh.K, sh.Is, nc, lane, wv);
    uint4 xr[CPL];
    smoe_gemv::gemv_load_x<CPL>(sh.xin, sh.K, lane, xr);
    __builtin_amdgcn_sched_barrier(0);  // every request above before the first use
    auto one_row = [&](int r) {
        const uint16_t v = smoe_gemv::gemv_dot<NM, CPL>(wv, xr, sh.K, lane);
        if (lane == 0 && n < sh.Ncol) sh.out[(size_t)r * sh.Ncol + n] = v;
    };
    one_row(0);
    for (int r = 1; r < sh.rows; ++r) {
        smoe_gemv::gemv_load_x<CPL>(sh.xin + (size_t)r * sh.K, sh.K, lane, xr);
        one_row(r);
    }
}

template <int PHASE, int CPL>
__global__ __launch_bounds__(256) void shared_rows_kernel(RowsShared sh) {
    shared_rows_item<PHASE, CPL>(sh, (int)blockIdx.x);
}

// The shared projection's 16-column items over 5-16 rows on MFMA, the
// arithmetic of verify_grouped_gemm's one-group ring launches item for item
// (waves per item and their contiguous step ranges, the order of the MFMAs,
// the partial tiles added in wave order), so the values are bit-identical to
// them; the operands come straight from memory in the MFMA layout (lane l:
// row l%16, 8 K at 8(l/16) + 32u of each 128-K step u-th quarter) through
// two register buffers, a step ahead, instead of an LDS ring.  Rows past
// the T feed output rows that are not stored.  Loads past a wave's range
// read past the buffers' records (zeros, no memory access).  red: LDS of
// 4 waves x NM x 64 x 16 bytes.
template <int PHASE>
SMOE_DEV void shared_mfma_item(const RowsShared& sh, int b, f4_t* red) {
    constexpr int NM = (PHASE == 1) ? 2 : 1;
    constexpr int WPI = (PHASE == 1) ? SMOE_SH_GU_WAVES : SMOE_SH_DN_WAVES;  // waves per item
    constexpr int W = mfma_waves<PHASE>();
    static_assert(WPI >= 1 && W % WPI == 0, "items per workgroup");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = wave % WPI;
    const int item = b * (W / WPI) + wave / WPI;
    const bool live = item * 16 < sh.Ncol;
    const int n0 = live ? item * 16 : 0;
    const int K = sh.K;
    const int nsteps = K / 128;
    const int s0 = (nsteps * sub) / WPI, s1 = (nsteps * (sub + 1)) / WPI;
    const int q = lane & 15, kq = lane >> 4;
    const int arow = q < sh.rows ? q : 0;
    const __amdgpu_buffer_rsrc_t ax = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(sh.xin), (short)0, sh.rows * K * 2, kBufWord3);
    const __amdgpu_buffer_rsrc_t wx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(sh.w), (short)0,
        (PHASE == 1 ? 2 * sh.Is : sh.Ncol) * K * 2, kBufWord3);
    const int aoff = (arow * K + 8 * kq) * 2;
    const int boff0 = ((n0 + q) * K + 8 * kq) * 2;
    const int boff1 = ((sh.Is + n0 + q) * K + 8 * kq) * 2;  // up rows (gate/up)
    struct Buf {
        h8_t a[4];
        h8_t w[NM][4];
    };
    auto load = [&](Buf& B, int st) {
        const bool in = st < s1;
        const int k2 = st * 256;  // byte offset of the step
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int o = k2 + 64 * u;
            B.a[u] = __builtin_bit_cast(h8_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                  ax, in ? aoff + o : 0x7FFFFFF0, 0, 0));
            B.w[0][u] = __builtin_bit_cast(h8_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                     wx, in ? boff0 + o : 0x7FFFFFF0, 0, kAuxNT));
            if constexpr (NM == 2)
                B.w[1][u] = __builtin_bit_cast(h8_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                         wx, in ? boff1 + o : 0x7FFFFFF0, 0,
                                                         kAuxNT));
        }
    };
    f4_t accg = f4_t{0.f, 0.f, 0.f, 0.f}, accu = f4_t{0.f, 0.f, 0.f, 0.f};
    auto mul = [&](const Buf& B) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            accg = __builtin_amdgcn_mfma_f32_16x16x32_f16(B.a[u], B.w[0][u], accg, 0, 0, 0);
            if constexpr (NM == 2)
                accu = __builtin_amdgcn_mfma_f32_16x16x32_f16(B.a[u], B.w[1][u], accu, 0, 0, 0);
        }
    };
    Buf P, Q;
    load(P, s0);
    load(Q, s0 + 1);
    for (int st = s0; st < s1; st += 2) {
        mul(P);
        load(P, st + 2);
        if (st + 1 < s1) mul(Q);
        load(Q, st + 3);
    }
    // the item's partial tiles, added in wave order
    red[(wave * NM) * 64 + lane] = accg;
    if constexpr (NM == 2) red[(wave * NM + 1) * 64 + lane] = accu;
    __syncthreads();
    if (sub == 0 && live) {
        const int w0 = wave;
        f4_t g = red[(w0 * NM) * 64 + lane];
        f4_t uu = (NM == 2) ? red[(w0 * NM + NM - 1) * 64 + lane] : g;
#pragma unroll
        for (int w = 1; w < WPI; ++w) {
            g += red[((w0 + w) * NM) * 64 + lane];
            if constexpr (NM == 2) uu += red[((w0 + w) * NM + 1) * 64 + lane];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * kq + i;
            if (r < sh.rows) {
                const float v = (PHASE == 1) ? silu_f(g[i]) * uu[i] : g[i];
                sh.out[(size_t)r * sh.Ncol + n0 + q] = f2h(v);
            }
        }
    }
}

// CPLS > 0: the workgroups from sh.wg0 on are the shared expert's columns
// (4 per workgroup, the matrix-vector routine with CPLS chunks per lane);
// CPLS < 0: its 16-column MFMA items (shared_mfma_item).
template <int PHASE, int CPLS = 0>
__global__ __launch_bounds__(64 * mfma_waves<PHASE>())
__attribute__((amdgpu_waves_per_eu(PHASE == 1 ? SMOE_W4_MFMA_WPE : SMOE_W4_MFMA_WPE2))) void
w4_mfma_kernel(W4Args a, RowsShared sh) {
    extern __shared__ uint4 smem[];
    int bid = (int)blockIdx.x;
    if constexpr (CPLS != 0) {
        const bool shw = sh.nfront ? bid < sh.nfront : bid >= sh.wg0;
        if (shw) {
            const int b = sh.nfront ? bid : bid - sh.wg0;
            if constexpr (CPLS > 0)
                shared_rows_item<PHASE, CPLS>(sh, b);
            else
                shared_mfma_item<PHASE>(sh, b, reinterpret_cast<f4_t*>(smem));
            return;
        }
        bid -= sh.nfront;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int q = lane & 15;
    const int kq = lane >> 4;
    const int cb = bid % a.nCB;
    const int slot = bid / a.nCB;
    const int K = a.K, N = a.N;
    const int G = K >> 7;
    const int K8 = K >> 3;
    const W4Lds l = carve_lds<4>(smem, a);
    const int e = a.active[slot];  // -1 past the touched experts
    if (e < 0) return;
    if (e >= a.E) {
        if (tid == 0 && cb == 0) flag_error(a.err, SMOE_DERR_BAD_ID);
        return;
    }
    const smoe_w4_mat wm = (PHASE == 1) ? a.experts[e].w13 : a.experts[e].w2;
    const int r0 = a.off[e];
    const int r1 = a.off[e + 1];
    if (!wm.qweight || !wm.scales || !wm.qzeros) {
        if (tid == 0 && cb == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
        return;
    }
    // 64 columns per block: gate cb*32.. and up I + cb*32.. (gate/up), or cb*64..
    const int col = (PHASE == 1) ? ((q < 8) ? cb * 32 + 4 * q : a.I + cb * 32 + 4 * (q - 8))
                                 : cb * 64 + 4 * q;
    const int colc = col < N ? col : 0;  // columns past N read column 0 (never stored)
    const int zsh = zero_shift<4>(colc);
    const W4Src src = make_src<4>(wm, K, N);
    const Masks<4> mk;
    constexpr int W = mfma_waves<PHASE>();
    float* red = l.red;  // [W][MCH][64]
    const bool direct = (PHASE == 1) && a.direct;
    const int g0 = wave;
    MfmaLoad L[kMfmaBufs];
    for (int mc = r0; mc < r1; mc += a.MCH) {
        const int M = min(a.MCH, r1 - mc);
        const bool stage = !direct || mc == r0;
        // rows of this chunk (all T tokens in the direct mode): source row j
        const int nrows = direct ? a.T : M;
        auto src_row = [&](int j) -> const uint4* {
            size_t r;
            if (direct) r = j;
            else r = (PHASE == 1) ? (size_t)a.sorted_token[mc + j] : (size_t)(mc + j);
            return reinterpret_cast<const uint4*>(a.xin + r * K);
        };
        // the rows' first chunks are requested, then this wave's first two
        // groups, and the rows are written to LDS while the weights are in
        // flight (requests are unconditional, so the wait for the rows is an
        // exact count that leaves the weights outstanding)
        const int nch = nrows * K8;
        // A operand row (MFMA row l%16) and the LDS rows of this lane's D rows
        // (requested before the rows, so one wait covers both)
        const bool aok = q < M;
        const int ar = direct ? a.sorted_token[mc + (aok ? q : 0)] : (aok ? q : 0);
        int drow[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * kq + i;
            const int rr = r < M ? r : 0;
            drow[i] = direct ? a.sorted_token[mc + rr] : rr;
        }
#if SMOE_W4_MFMA_DMA
        // The rows go straight to LDS in natural order (global->LDS loads:
        // a wave's instruction fills 64 consecutive 16-byte chunks, and no
        // register holds them), requested before the weights; once they have
        // landed their pairs are permuted in place and the sums taken.
        if (stage) {
            const bool gath = PHASE == 1 && !direct;
#pragma unroll
            for (int u = 0; u < kRowChunksPerThread; ++u) {
                const int b0 = wave_u * 64 + u * (int)blockDim.x;  // the wave's first chunk
                if (b0 < nch) {
                    // gathered rows: the (at most two, K8 >= 64) rows of the
                    // wave's chunks take their tokens through scalar loads
                    const int jlo = b0 / K8;
                    const int jhi = jlo + 1 < nrows ? jlo + 1 : nrows - 1;
                    const int tlo = gath ? ld_const(a.sorted_token + mc + jlo) : 0;
                    const int thi = gath ? ld_const(a.sorted_token + mc + jhi) : 0;
                    int idx = b0 + lane;
                    idx = idx < nch ? idx : nch - 1;  // (its LDS slot lies past the rows,
                                                      // in the sums or the reduction area)
                    const int j = idx / K8;
                    size_t r;
                    if (gath) r = (size_t)((j == jlo) ? tlo : thi);
                    else r = direct ? (size_t)j : (size_t)(mc + j);
                    __builtin_amdgcn_global_load_lds(
                        (const void*)(a.xin + r * K + 8 * (idx - j * K8)),
                        (__attribute__((address_space(3))) void*)(l.xs + b0), 16, 0, 0);
                }
            }
        }
#pragma unroll
        for (int b = 0; b < kMfmaBufs; ++b) mfma_load(L[b], src, g0 + b * W, G, colc, kq);
        __builtin_amdgcn_sched_barrier(0);
        if (stage) {
            // this wave's chunks have landed (the weight requests after them
            // stay in flight), then every wave's: a plain barrier (a fenced
            // one would also wait for the weights)
            wait_vm<6 * kMfmaBufs>();
            __builtin_amdgcn_s_barrier();
            finish_rows_natural4(l.xs, l.sums, nrows, K8, G);
        }
#else
        uint4 xv[kRowChunksPerThread];
        if (stage && PHASE == 1 && !direct && K8 >= 64) {
            // gathered rows: a wave's 64 consecutive chunks span at most two
            // rows, whose tokens come through scalar loads issued together
            // (one wait for all of them, none for the vector loads)
            int jlo[kRowChunksPerThread], tlo[kRowChunksPerThread], thi[kRowChunksPerThread];
#pragma unroll
            for (int u = 0; u < kRowChunksPerThread; ++u) {
                int b0 = wave_u * 64 + u * (int)blockDim.x;
                b0 = b0 < nch ? b0 : nch - 1;
                jlo[u] = b0 / K8;
                const int jhi = jlo[u] + 1 < nrows ? jlo[u] + 1 : nrows - 1;
                tlo[u] = ld_const(a.sorted_token + mc + jlo[u]);
                thi[u] = ld_const(a.sorted_token + mc + jhi);
            }
#pragma unroll
            for (int u = 0; u < kRowChunksPerThread; ++u) {
                int idx = tid + u * (int)blockDim.x;
                idx = idx < nch ? idx : nch - 1;
                const int j = idx / K8;
                const int t = (j == jlo[u]) ? tlo[u] : thi[u];
                xv[u] = reinterpret_cast<const uint4*>(a.xin + (size_t)t * K)[idx - j * K8];
            }
        } else if (stage) {
#pragma unroll
            for (int u = 0; u < kRowChunksPerThread; ++u) {
                int idx = tid + u * (int)blockDim.x;
                idx = idx < nch ? idx : nch - 1;
                const int j = idx / K8;
                xv[u] = src_row(j)[idx - j * K8];
            }
        }
        // (unconditional: groups past G read nothing and are not multiplied)
#pragma unroll
        for (int b = 0; b < kMfmaBufs; ++b) mfma_load(L[b], src, g0 + b * W, G, colc, kq);
        __builtin_amdgcn_sched_barrier(0);
        if (stage) {
#pragma unroll
            for (int u = 0; u < kRowChunksPerThread; ++u) {
                int idx = tid + u * (int)blockDim.x;
                idx = idx < nch ? idx : nch - 1;
                l.xs[idx] = permute_chunk<4>(xv[u]);
            }
            // rows longer than the early requests cover
            for (int idx = tid + kRowChunksPerThread * (int)blockDim.x; idx < nch;
                 idx += blockDim.x) {
                const int j = idx / K8;
                l.xs[idx] = permute_chunk<4>(src_row(j)[idx - j * K8]);
            }
            finish_rows<4>(l.xs, l.sums, nrows, K8, G);
        }
#endif
        f4_t acc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = f4_t{0.f, 0.f, 0.f, 0.f};
        // groups wave, wave + 4, ... through the buffers, each refilled with
        // the group kMfmaBufs further on as soon as it has been multiplied
        // (branches on the group index are wave-uniform)
        for (int g = g0; g < G; g += kMfmaBufs * W) {
#pragma unroll
            for (int b = 0; b < kMfmaBufs; ++b) {
                const int gb = g + b * W;
                if (b == 0 || gb < G)
                    mfma_group(L[b], l.xs, l.sums, ar, aok, drow, gb, K8, G, kq, zsh, mk, acc);
                mfma_load(L[b], src, gb + kMfmaBufs * W, G, colc, kq);
            }
        }
        // the waves' tiles, added in a fixed order
        __syncthreads();  // every wave is done with the staged rows
        const int MCH = a.MCH;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * kq + i < M) red[(wave * MCH + 4 * kq + i) * 64 + 4 * q + c] = acc[c][i];
        __syncthreads();
        if (PHASE == 1) {
            for (int idx = tid; idx < M * 32; idx += blockDim.x) {
                const int m = idx >> 5, j = idx & 31;
                float gv = 0.0f, uv = 0.0f;
                for (int w = 0; w < W; ++w) {
                    gv += red[(w * MCH + m) * 64 + j];
                    uv += red[(w * MCH + m) * 64 + 32 + j];
                }
                a.out[(size_t)(mc + m) * a.I + cb * 32 + j] = f2h(silu_f(gv) * uv);
            }
        } else {
            for (int idx = tid; idx < M * 64; idx += blockDim.x) {
                const int m = idx >> 6, j = idx & 63;
                if (cb * 64 + j < N) {
                    float v = 0.0f;
                    for (int w = 0; w < W; ++w) v += red[(w * MCH + m) * 64 + j];
                    a.out[(size_t)(mc + m) * N + cb * 64 + j] = f2h(v);
                }
            }
        }
        __syncthreads();  // red and the staged rows are rewritten by the next chunk
    }
}

// --------------------------------------------- routing + gate/up, T = 1 ----
//
// The one-token draft step's routing, ELB update and gather maps folded into
// the gate/up launch (Specter, Key Contributions 4: routing, gathering and the
// experts' FFN of a draft step in one fused launch).  Every workgroup reads
// the token's E (+1 shared-gate) router logits, computed just before by
// route_logits_kernel with the pinned routine of the routing kernels, and
// takes the top k itself, so every workgroup reaches the same selection,
// bit-identical to moe_route_topk / moe_route_plan; slot s then takes the
// s-th smallest selected id, which is the expert moe_gather places at sorted
// row s.  One extra workgroup writes the routing outputs, the ELB increments
// and the maps, which the down projection and the combine read after this
// launch.
// A dense shared expert folded into the one-token draft launches (FP16 w13
// [2 Is, H], w2 [H, Is], the nn.Linear layout of the verify path): the
// workgroups from wg0 on compute its columns with the matrix-vector routine
// of gemv_core.h, so its output is bit-identical to verify_grouped_gemm's on
// the same row.  They read only the token row (gate/up) or the shared h
// written by the gate/up launch (down), so they need nothing from the routed
// workgroups beside them.
struct SharedArgs {
    const uint16_t* w13;
    const uint16_t* w2;
    int Is;         // shared intermediate
    int wg0;        // first shared workgroup of the launch
    uint16_t* h;    // [Is] fp16
    uint16_t* out;  // [H] fp16
};

// Columns (b * waves + wave) * CPW + c, c < CPW, of the shared expert's
// projection: all their weight chunks are requested, then the row, then each
// column is reduced.  Phase 1: K = H, Ncol = Is, gate row n and up row Is + n
// of w13, output h; phase 2: K = Is, Ncol = H, row n of w2, output y.
template <int PHASE, int CPL, int CPW>
SMOE_DEV void shared_gemv_block(const uint16_t* xrow, const uint16_t* W, int K, int I, int Ncol,
                                int b, uint16_t* out) {
    constexpr int NM = (PHASE == 1) ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    int n[CPW];
    u4_t wv[CPW][NM][CPL];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        n[c] = (b * nw + wave) * CPW + c;
        const int nc = (n[c] < Ncol) ? n[c] : Ncol - 1;  // loads stay in the matrix
        smoe_gemv::gemv_load_w<NM, CPL>(W, K, I, nc, lane, wv[c]);
    }
    uint4 xr[CPL];
    smoe_gemv::gemv_load_x<CPL>(xrow, K, lane, xr);
    __builtin_amdgcn_sched_barrier(0);  // every request above before the first use
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const uint16_t v = smoe_gemv::gemv_dot<NM, CPL>(wv[c], xr, K, lane);
        if (lane == 0 && n[c] < Ncol) out[n[c]] = v;
    }
}

// The shared expert's projection as a launch of its own (shapes without a
// fused instantiation): 4 waves per workgroup, one column per wave.
template <int PHASE, int CPL>
__global__ __launch_bounds__(256) void shared_gemv_kernel(SharedArgs sh, const uint16_t* x, int H) {
    if (PHASE == 1)
        shared_gemv_block<1, CPL, 1>(x, sh.w13, H, sh.Is, sh.Is, blockIdx.x, sh.h);
    else
        shared_gemv_block<2, CPL, 1>(sh.h, sh.w2, sh.Is, 0, H, blockIdx.x, sh.out);
}

struct RouteArgs {
    const uint16_t* wr;   // router [E, H]
    const uint16_t* wsg;  // shared-expert gate row [H] or null
    const float* logits;  // the E (+1) logits from route_logits_kernel
    int k, renorm;
    int32_t* counters_row;  // ELB row of the layer or null
    int32_t* ids;
    float* w;
    float* gate;
    int32_t* off;
    int32_t* sorted_token;
    int32_t* sorted_pair;
    int32_t* pair_pos;
    int32_t* active;
    int32_t* n_active;
};

constexpr int kFusedMaxK = 32;

// The token's router logits, one per wave, for route_w4_kernel (every one of
// its workgroups needs all of them; reading the whole router in each, from
// L2, measured slower than this extra launch at every decode shape, by 1-3
// us for a 131 KB router and more for larger ones).  Same routine and order
// as the routing kernels, so the logits are bit-identical.
__global__ __launch_bounds__(256) void route_logits_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           const uint16_t* __restrict__ wsg,
                                                           int H, int E, int nvec,
                                                           float* __restrict__ lg) {
    const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * (blockDim.x >> 6);
    smoe_route::wave_logits(x, wr, wsg, H, E, nvec, wave, nvec, nwaves, lg, threadIdx.x & 63);
}

template <int LPR, int NG, int CPLS>
__global__ __launch_bounds__(64 * kT1MaxWaves)
__attribute__((amdgpu_waves_per_eu(2))) void route_w4_kernel(W4Args a, RouteArgs r, SharedArgs sh) {
    __shared__ float lg_s[257];
    __shared__ int32_t ids_s[kFusedMaxK];
    extern __shared__ uint4 smem[];
    if constexpr (CPLS > 0) {
        // the shared expert's gate/up columns, two per wave
        if ((int)blockIdx.x >= sh.wg0) {
            shared_gemv_block<1, CPLS, 2>(a.xin, sh.w13, a.K, sh.Is, sh.Is,
                                          (int)blockIdx.x - sh.wg0, sh.h);
            return;
        }
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cb = blockIdx.x % a.nCB;
    const int slot = blockIdx.x / a.nCB;
    const int E = a.E, k = r.k;

    const smoe_w4_expert spec = spec_table(a, lane);
    // the token row, requested with the logits (its latency overlaps the
    // routing below)
    uint4 xv[kRowChunksPerThread];
    request_row(reinterpret_cast<const uint4*>(a.xin), a.K >> 3, xv);

    // 1. the router logits of the launch before
    const int nvec = E + (r.wsg ? 1 : 0);
    for (int i = tid; i < nvec; i += blockDim.x) lg_s[i] = r.logits[i];
    __syncthreads();
    // 2. the last workgroup (beyond the projection's): routing outputs (the
    //    routing kernels' own routine), the ELB increments and the maps,
    //    beside the projection rather than after a share of it
    if (blockIdx.x == (unsigned)(k * a.nCB)) {
        if (wave == 0)
            smoe_route::topk_softmax_wave(lg_s, E, k, r.renorm, r.wsg != nullptr, lane, r.ids,
                                          r.w, r.gate, ids_s);
        __syncthreads();
        smoe_maps::one_token_maps(ids_s, k, E, r.counters_row, r.off, r.sorted_token,
                                  r.sorted_pair, r.pair_pos, r.active, r.n_active);
        return;
    }
    // 3. the selected ids (wave 0)
    if (wave == 0) smoe_route::topk_ids_wave(lg_s, E, k, lane, ids_s);
    __syncthreads();
    // 4. this slot's expert: the slot-th smallest selected id (the ids of one
    //    token are distinct), i.e. the expert moe_gather places at row slot
    int e = -1;
    for (int j = 0; j < k; ++j) {
        int less = 0;
        for (int i = 0; i < k; ++i) less += (ids_s[i] < ids_s[j]) ? 1 : 0;
        if (less == slot) e = ids_s[j];
    }
    // 5. this slot's block of the gate/up projection
    if (cb == 0) write_slot_desc(a, spec, slot, e);
    if (e >= 0) {
        one_token_block<4, 1, LPR, NG>(a, carve_lds<4>(smem, a), pick_mat<1>(a, spec, e), xv,
                                       slot, cb);
    }
}

// The down projection of a one-token step (as w4_kernel's) with the shared
// expert's down columns in the workgroups from sh.wg0 on, one per wave.
template <int LPR, int NG, int CPLS>
__global__ __launch_bounds__(64 * kT1MaxWaves)
__attribute__((amdgpu_waves_per_eu(w4_waves_per_eu<1, NG>()))) void w4_down_shared_kernel(
    W4Args a, SharedArgs sh) {
    extern __shared__ uint4 smem[];
    if ((int)blockIdx.x >= sh.wg0) {
        shared_gemv_block<2, CPLS, 1>(sh.h, sh.w2, sh.Is, 0, a.N, (int)blockIdx.x - sh.wg0,
                                      sh.out);
        return;
    }
    const int cb = blockIdx.x % a.nCB;
    const int slot = blockIdx.x / a.nCB;
    const uint4* row4 = reinterpret_cast<const uint4*>(a.xin + (size_t)slot * a.K);
    uint4 xv[kRowChunksPerThread];
    const SlotDesc d = a.desc[slot];
    request_row(row4, a.K >> 3, xv);
    if (d.e < 0) return;
    one_token_block<4, 2, LPR, NG>(a, carve_lds<4>(smem, a), d.w2, xv, slot, cb);
}

// ---------------------------------------------------------------- launch ----

// ============================================= one-launch draft layer (T = 1) ===
//
// [S1] Key Contributions 4 and Methodology in Plain English: the draft's
// routing, expert FFN and combine of a decode step are dispatched inside a
// single GPU launch.  moe_draft_layer does a whole one-token MoE layer in one
// persistent launch of one 8-wave workgroup per CU, every workgroup resident:
//
//   0 (no logits given): the router logits of x, one per wave across the
//     chip, into the workspace; grid barrier.
//   A every workgroup takes the top k of the logits itself (the routing
//     kernels' routine) and keeps its slots' matrices in LDS; the last
//     workgroup also writes the routing outputs, the ELB increments and the
//     maps.
//   B gate/up items -- routed INT4 blocks and the FP16 shared expert's
//     columns -- against x staged once per workgroup; h stored; grid barrier.
//   D down items: each requests its block's first weights, then stages the h
//     row it needs; y stored; grid barrier.
//   F combine (+ residual, + the norm epilogue, + the next layer's router
//     logits) by the first workgroups, as moe_combine_route_logits.
//
// Each item runs on a sub-group of 4 waves with the same geometry, loads and
// reduction order as the two one-token launches of moe_draft_route_ffn, so
// y_sorted, h and every later value are bit-identical to those launches.
// Values one workgroup writes for another (logits, h, y, the shared
// expert's h and output) are stored and loaded with device-scope accesses,
// which are coherent across the XCDs' separate L2 caches; a grid barrier is
// an atomic counter that each workgroup increments after its stores have
// completed and then polls.  Every poll is bounded in time: on expiry the
// workgroup flags SMOE_DERR_SYNC and skips to the end, so no wave can wait
// forever.  The last workgroup to finish resets the counters.
//
// Measured on MI355X this one launch is slower than the three launches plus
// combine it replaces (each grid barrier costs about 3.5 us, about two memory
// round trips between XCDs, more than a kernel boundary on one stream); it
// is kept as the single-launch form of the layer, bit-identical to the split
// form.  Staging the down weights in LDS during B measured slower still:
// the extra stream competes with gate/up, and the compiler orders every LDS
// access after outstanding LDS-DMA loads.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

SMOE_DEV smoe_w4_expert spec_table_e(const smoe_w4_expert* experts, int E, int lane) {
    W4Args t{};
    t.experts = experts;
    t.E = E;
    return spec_table(t, lane);
}
template <int PHASE>
SMOE_DEV smoe_w4_mat pick_mat_e(const smoe_w4_expert* experts, int E, const smoe_w4_expert& spec,
                                int e) {
    W4Args t{};
    t.experts = experts;
    t.E = E;
    return pick_mat<PHASE>(t, spec, e);
}

constexpr int kLayerWaves = 8;  // two sub-groups of four
constexpr int kSubWaves = 4;
constexpr int kLayerRed = kSubWaves * 64;           // floats per sub-group (waves x NB <= 64)
constexpr uint64_t kSyncSpinTicks = 10000000ull;    // 100 ms of the 100 MHz real-time clock

struct LayerArgs {
    const uint16_t* x;      // [H] the layer's (normalised) input row
    const uint16_t* wr;     // router [E, H] (phase 0 only)
    const uint16_t* wsg;    // shared-expert gate row [H] or null
    const float* logits;    // [nvec] logits of x, or null: phase 0
    float* lg_ws;           // [nvec] workspace (phase 0)
    int H, I, E, k, renorm, nvec;
    const smoe_w4_expert* experts;
    int32_t* counters_row;
    int32_t* ids;
    float* w;
    float* gate;
    int32_t* off;
    int32_t* sorted_token;
    int32_t* sorted_pair;
    int32_t* pair_pos;
    int32_t* active;
    int32_t* n_active;
    const uint16_t* sw13;   // shared expert [2 Is, H] or null
    const uint16_t* sw2;    // [H, Is]
    int Is;
    uint16_t* h;            // [k, I] workspace
    uint16_t* sh_h;         // [Is]
    uint16_t* y;            // [k, H] y_sorted
    uint16_t* sh_out;       // [H]
    uint32_t* sync;         // [2] zero between calls
    const uint16_t* resid;
    uint16_t* out;
    uint16_t* norm_out;     // or null
    float eps;
    const uint16_t* wr_next;   // next layer's router [E_next, H] or null
    const uint16_t* wsg_next;
    int E_next, nvec_next;
    float* lg_next;
    int32_t* err;
    // plan
    int P;                   // workgroups (one per CU)
    int nCB1, na1;           // gate/up: column blocks per slot, active waves per item
    int nCB2, na2, G2;       // down: column blocks per slot, active waves, groups
    int n_gu, n_dn;          // gate/up items (routed, then shared), down items
    int R1, R2;              // rounds of gate/up and down items
    int nF;                  // workgroups of phase F
    int row_bytes;           // dynamic LDS: staged rows
};

struct DevRows {
    SMOE_DEV uint4 operator()(const uint16_t* p) const { return ld_dev4(p); }
};

// vmcnt(0): this wave's loads, stores and LDS-DMA loads have completed.
SMOE_DEV void wait_vm0() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); }

// Grid barrier number `nb` (1, 2, ...) of the launch: returns false when the
// wait expired (flagged), after which the workgroup only runs layer_exit.
SMOE_DEV bool layer_sync(const LayerArgs& a, int nb, int* flag_s) {
    wait_vm0();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t target = (uint32_t)nb * (uint32_t)a.P;
        const uint32_t old = __hip_atomic_fetch_add(a.sync, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        int ok = 1;
        if (old + 1 < target) {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (ld_dev(a.sync) < target) {
                __builtin_amdgcn_s_sleep(1);
                if (__builtin_amdgcn_s_memrealtime() - t0 > kSyncSpinTicks) {
                    ok = 0;
                    flag_error(a.err, SMOE_DERR_SYNC);
                    break;
                }
            }
        }
        *flag_s = ok;
    }
    __syncthreads();
    return *flag_s != 0;
}

// Every workgroup ends here: the last one to arrive (all others have left
// every barrier) returns both counters to zero for the next call.
SMOE_DEV void layer_exit(const LayerArgs& a) {
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(a.sync + 1, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1 == (uint32_t)a.P) {
            st_dev(a.sync, 0u);
            st_dev(a.sync + 1, 0u);
        }
    }
}

// One item's place: workgroup i mod P, sub-group (i / P) mod 2, round i / 2P.
SMOE_DEV int layer_item(int P, int b, int sub, int r) { return (2 * r + sub) * P + b; }

// A source whose loads fetch nothing: an empty buffer (loads return zero)
// and scale / zero reads of `safe` (N = 0 keeps every offset at 0).
SMOE_DEV W4Src empty_src(const void* safe) {
    W4Src s;
    s.q = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(safe), (short)0, 0, kBufWord3);
    s.m.qweight = static_cast<const int32_t*>(safe);
    s.m.scales = static_cast<const uint16_t*>(safe);
    s.m.qzeros = static_cast<const int32_t*>(safe);
    s.N = 0;
    return s;
}

constexpr int kAuxDev = 16;  // sc1: device-scope (coherent across the XCDs)

// The matrices of expert slot `slot` kept in LDS after routing (w13 in words
// 0-2, w2 in 3-5), as workgroup-uniform pointers.
template <int PHASE>
SMOE_DEV smoe_w4_mat slot_mat(const uint64_t (*mat)[6], int slot) {
    const uint64_t* m = mat[slot] + (PHASE == 1 ? 0 : 3);
    smoe_w4_mat r;
    r.qweight = uniform_ptr(reinterpret_cast<const int32_t*>(m[0]));
    r.scales = uniform_ptr(reinterpret_cast<const uint16_t*>(m[1]));
    r.qzeros = uniform_ptr(reinterpret_cast<const int32_t*>(m[2]));
    return r;
}

// Sums of a sub-group item's slots for its four columns (as one_token_block):
// groups myslot, myslot + nslots, ... through two register buffers.
template <int NG, typename Load>
SMOE_DEV void item_groups(Load load, const uint4* xs, const float4* sums, int myslot, int nslots,
                          int G, int K8, int zsh, float (&acc)[1][4], GroupLoad<4>& A) {
    const Masks<4> mk;
    const W4Lds l{const_cast<uint4*>(xs), const_cast<float4*>(sums), nullptr};
    GroupLoad<4> B;
    const int g0 = myslot;
    if (NG >= 3) load(B, clamp_group(g0 + nslots, G));
    step_if<4>(A, l, g0, G, K8, zsh, mk, acc);
    if (NG == 2) {
        load(B, clamp_group(g0 + nslots, G));
        __builtin_amdgcn_sched_barrier(0);
    }
    if (NG >= 3) load(A, clamp_group(g0 + 2 * nslots, G));
    if (NG >= 2) step_if<4>(B, l, g0 + nslots, G, K8, zsh, mk, acc);
    if (NG >= 4) load(B, clamp_group(g0 + 3 * nslots, G));
    if (NG >= 3) step_if<4>(A, l, g0 + 2 * nslots, G, K8, zsh, mk, acc);
    if (NG >= 4) step_if<4>(B, l, g0 + 3 * nslots, G, K8, zsh, mk, acc);
}

// Butterfly of a wave's slot partials (lane distances LPR, 2 LPR, ...) into
// the sub-group's LDS row; wave ws of the sub-group writes red[ws * NB + .].
template <int LPR>
SMOE_DEV void item_partials(float (&acc)[1][4], float* red, int ws, int lane) {
    constexpr int NB = 4 * LPR;
#pragma unroll
    for (int d = LPR; d < 64; d *= 2)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[0][c] += __shfl_xor(acc[0][c], d);
    if (lane < LPR)
#pragma unroll
        for (int c = 0; c < 4; ++c) red[ws * NB + 4 * lane + c] = acc[0][c];
}

// The shared expert's projection columns of one sub-group item (one or two
// per wave, shared_gemv_block's arithmetic), the row read device-coherently
// when it was written in this launch.
template <int PHASE, int CPL, int CPW, bool kDevRow>
SMOE_DEV void shared_item(const uint16_t* xrow, const uint16_t* W, int K, int I, int Ncol, int b,
                          int ws, int lane, uint16_t* out) {
    constexpr int NM = (PHASE == 1) ? 2 : 1;
    int n[CPW];
    u4_t wv[CPW][NM][CPL];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        n[c] = (b * kSubWaves + ws) * CPW + c;
        const int nc = (n[c] < Ncol) ? n[c] : Ncol - 1;
        smoe_gemv::gemv_load_w<NM, CPL>(W, K, I, nc, lane, wv[c]);
    }
    uint4 xr[CPL];
    if constexpr (kDevRow) {
        const int kc = K >> 3;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lane + 64 * j;
            xr[j] = ld_dev4(xrow + 8 * (c < kc ? c : kc - 1));
        }
    } else {
        smoe_gemv::gemv_load_x<CPL>(xrow, K, lane, xr);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const uint16_t v = smoe_gemv::gemv_dot<NM, CPL>(wv[c], xr, K, lane);
        if (lane == 0 && n[c] < Ncol) st_dev(out + n[c], v);
    }
}

template <int LPR1, int NG1, int LPR2, int NG2, int CPLS1, int CPLS2>
__global__ __launch_bounds__(64 * kLayerWaves) void draft_layer_kernel(LayerArgs a) {
    constexpr int RPL1 = 64 / LPR1, NB1 = 4 * LPR1;
    constexpr int RPL2 = 64 / LPR2, NB2 = 4 * LPR2;
    __shared__ float lg_s[257];
    __shared__ int32_t ids_s[kFusedMaxK];   // top-k ids by rank
    __shared__ int32_t e_s[kFusedMaxK];     // expert of each slot (increasing id)
    __shared__ uint64_t mat_s[kFusedMaxK][6];  // each slot's w13 and w2 matrices
    __shared__ int32_t ids_w[kFusedMaxK];
    __shared__ int32_t pp_s[kFusedMaxK];
    __shared__ float w_s[kFusedMaxK];
    __shared__ float gate_s;
    __shared__ float redf[kLayerWaves];
    __shared__ int flag_s;
    extern __shared__ uint4 smem[];
    char* dyn = reinterpret_cast<char*>(smem);
    float* red = reinterpret_cast<float*>(dyn + a.row_bytes);  // [2][kLayerRed]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sub = wave / kSubWaves;
    const int ws = wave % kSubWaves;
    const int b = blockIdx.x;
    const int P = a.P;
    const int H = a.H, I = a.I, E = a.E, k = a.k;
    const int K8_1 = H >> 3, G1 = H / 128;
    const int K8_2 = I >> 3;
    const int n_rt1 = k * a.nCB1, n_rt2 = k * a.nCB2;
    int nbar = 0;
    bool ok = true;

    const smoe_w4_expert spec = spec_table_e(a.experts, E, lane);

    // ---- 0: router logits of x, one per wave across the chip ----
    if (!a.logits) {
        const int item = b * kLayerWaves + wave;
        if (item < a.nvec)
            smoe_route::wave_logits(a.x, a.wr, a.wsg, H, E, a.nvec, item, a.nvec,
                                    P * kLayerWaves, lg_s, lane);
        __syncthreads();
        if (tid < kLayerWaves && b * kLayerWaves + tid < a.nvec)
            st_dev(reinterpret_cast<uint32_t*>(a.lg_ws) + b * kLayerWaves + tid,
                   __float_as_uint(lg_s[b * kLayerWaves + tid]));
        ok = layer_sync(a, ++nbar, &flag_s);
        if (ok)
            for (int i = tid; i < a.nvec; i += blockDim.x)
                lg_s[i] = __uint_as_float(ld_dev(reinterpret_cast<const uint32_t*>(a.lg_ws) + i));
    } else {
        for (int i = tid; i < a.nvec; i += blockDim.x) lg_s[i] = a.logits[i];
    }
    if (!ok) {
        layer_exit(a);
        return;
    }
    __syncthreads();

    // ---- A: routing ----
    if (wave == 0) smoe_route::topk_ids_wave(lg_s, E, k, lane, ids_s);
    __syncthreads();
    if (tid < k) {
        const int id = ids_s[tid];
        int pos = 0;
        for (int i = 0; i < k; ++i) pos += (ids_s[i] < id) ? 1 : 0;
        e_s[pos] = id;
        pp_s[tid] = pos;
    }
    if (b == P - 1) {
        if (wave == 0)
            smoe_route::topk_softmax_wave(lg_s, E, k, a.renorm, a.wsg != nullptr, lane, a.ids,
                                          a.w, a.gate, ids_w);
        __syncthreads();
        smoe_maps::one_token_maps(ids_w, k, E, a.counters_row, a.off, a.sorted_token,
                                  a.sorted_pair, a.pair_pos, a.active, a.n_active);
    }
    __syncthreads();
    if (wave == 0)
        for (int j = 0; j < k; ++j) {
            const int e = __builtin_amdgcn_readfirstlane(e_s[j]);
            const smoe_w4_mat m1 = pick_mat_e<1>(a.experts, E, spec, e);
            const smoe_w4_mat m2 = pick_mat_e<2>(a.experts, E, spec, e);
            if (lane == 0) {
                mat_s[j][0] = reinterpret_cast<uint64_t>(m1.qweight);
                mat_s[j][1] = reinterpret_cast<uint64_t>(m1.scales);
                mat_s[j][2] = reinterpret_cast<uint64_t>(m1.qzeros);
                mat_s[j][3] = reinterpret_cast<uint64_t>(m2.qweight);
                mat_s[j][4] = reinterpret_cast<uint64_t>(m2.scales);
                mat_s[j][5] = reinterpret_cast<uint64_t>(m2.qzeros);
            }
        }
    __syncthreads();

    // ---- B: gate/up items (routed INT4 blocks, then shared FP16 columns) ----
    uint4* xs = reinterpret_cast<uint4*>(dyn);
    float4* sums = reinterpret_cast<float4*>(dyn + (size_t)K8_1 * 16);
    auto gu_src = [&](int i, int& cb, int& slot) {
        slot = i / a.nCB1;
        cb = i - slot * a.nCB1;
        return slot_mat<1>(mat_s, slot);
    };
    const int q1 = lane % LPR1;
    const int myslot1 = ws * RPL1 + lane / LPR1;
    const int nslots1 = a.na1 * RPL1;
    // the token row, then round 0's first group (an empty source where the
    // wave has no routed item: a fixed load count), then x is staged
    uint4 xv[kRowChunksPerThread];
    {
        const uint4* x4 = reinterpret_cast<const uint4*>(a.x);
#pragma unroll
        for (int u = 0; u < kRowChunksPerThread; ++u) {
            const int idx = tid + u * 64 * kLayerWaves;
            xv[u] = x4[idx < K8_1 ? idx : K8_1 - 1];
        }
    }
    GroupLoad<4> A1;
    {
        const int i0 = layer_item(P, b, sub, 0);
        const bool rt0 = i0 < n_rt1;
        const int slot0 = rt0 ? i0 / a.nCB1 : 0;
        const int cb0 = i0 - slot0 * a.nCB1;
        const smoe_w4_mat wm0 = slot_mat<1>(mat_s, slot0);
        const bool v0 = rt0 && ws < a.na1 && wm0.qweight && wm0.scales && wm0.qzeros;
        const int col0 = !v0 ? 0
                         : (q1 < LPR1 / 2) ? cb0 * (NB1 / 2) + 4 * q1
                                           : I + cb0 * (NB1 / 2) + 4 * (q1 - LPR1 / 2);
        const W4Src src0 = v0 ? make_src<4>(wm0, H, 2 * I) : empty_src(a.x);
        load_group<4>(A1, src0, clamp_group(myslot1, G1), col0, true);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kRowChunksPerThread; ++u) {
        const int idx = tid + u * 64 * kLayerWaves;
        if (idx < K8_1) xs[idx] = permute_chunk<4>(xv[u]);
    }
    // the group sums of x (finish_rows' arithmetic)
    __syncthreads();
    for (int gg = tid; gg < G1; gg += 64 * kLayerWaves) {
        const uint4* xr = xs + gg * QF<4>::kChunks;
        float s4[2] = {0.0f, 0.0f};
#pragma unroll 4
        for (int c = 0; c < QF<4>::kChunks; ++c) {
            const uint4 p = xr[c];
            const h2_t x0 = as_h2(p.x), x1 = as_h2(p.y), x2 = as_h2(p.z), x3 = as_h2(p.w);
            s4[0] += ((float)x0.x + (float)x0.y) + ((float)x2.x + (float)x2.y);
            s4[1] += ((float)x1.x + (float)x1.y) + ((float)x3.x + (float)x3.y);
        }
        sums[gg] = make_float4(s4[0], s4[1], 0.0f, 0.0f);
    }
    __syncthreads();
    for (int r = 0; r < a.R1; ++r) {
        const int i = layer_item(P, b, sub, r);
        float* rd = red + sub * kLayerRed;
        if (i < n_rt1) {
            int cb, slot;
            const smoe_w4_mat wm = gu_src(i, cb, slot);
            const bool good = wm.qweight && wm.scales && wm.qzeros;
            if (!good && tid % (64 * kSubWaves) == 0 && cb == 0)
                flag_error(a.err, SMOE_DERR_NULL_EXPERT);
            if (ws < a.na1 && good) {
                const int col = (q1 < LPR1 / 2) ? cb * (NB1 / 2) + 4 * q1
                                                : I + cb * (NB1 / 2) + 4 * (q1 - LPR1 / 2);
                const W4Src src = make_src<4>(wm, H, 2 * I);
                if (r > 0) load_group<4>(A1, src, clamp_group(myslot1, G1), col, true);
                float acc[1][4] = {{0.0f, 0.0f, 0.0f, 0.0f}};
                auto ld = [&](GroupLoad<4>& L, int g) { load_group<4>(L, src, g, col, true); };
                item_groups<NG1>(ld, xs, sums, myslot1, nslots1, G1, K8_1, zero_shift<4>(col),
                                 acc, A1);
                item_partials<LPR1>(acc, rd, ws, lane);
            }
        } else {
            if constexpr (CPLS1 > 0) {
                if (i < a.n_gu)
                    shared_item<1, CPLS1, 2, false>(a.x, a.sw13, H, a.Is, a.Is, i - n_rt1, ws,
                                                    lane, a.sh_h);
            }
        }
        __syncthreads();
        if (i < n_rt1) {
            const int slot = i / a.nCB1;
            const int cb = i - slot * a.nCB1;
            const smoe_w4_mat wm = slot_mat<1>(mat_s, slot);
            const int ts = tid % (64 * kSubWaves);
            if (wm.qweight && wm.scales && wm.qzeros && ts < NB1 / 2) {
                float gv = 0.0f, uv = 0.0f;
                for (int w = 0; w < a.na1; ++w) {
                    gv += rd[w * NB1 + ts];
                    uv += rd[w * NB1 + NB1 / 2 + ts];
                }
                st_dev(a.h + (size_t)slot * I + cb * (NB1 / 2) + ts, f2h(silu_f(gv) * uv));
            }
        }
        __syncthreads();
    }
    ok = layer_sync(a, ++nbar, &flag_s);

    // ---- D: down items (routed blocks from LDS, shared columns) ----
    if (ok) {
        const int q2 = lane % LPR2;
        const int myslot2 = ws * RPL2 + lane / LPR2;
        const int nslots2 = a.na2 * RPL2;
        const int G2 = a.G2;
        for (int r = 0; r < a.R2; ++r) {
            const int i = layer_item(P, b, sub, r);
            float* rd = red + sub * kLayerRed;
            uint4* hs = reinterpret_cast<uint4*>(dyn) + (size_t)sub * K8_2;
            float4* hsum = reinterpret_cast<float4*>(dyn + (size_t)2 * K8_2 * 16) + sub * G2;
            // the h rows of both sub-groups' routed items, staged together
            const bool rt = i < n_rt2;
            const int slot = rt ? i / a.nCB2 : 0;
            const int cb2 = rt ? i - slot * a.nCB2 : 0;
            const int col2 = cb2 * NB2 + 4 * q2;
            const smoe_w4_mat wm2 = slot_mat<2>(mat_s, slot);
            const bool good2 = rt && wm2.qweight && wm2.scales && wm2.qzeros;
            // the block's first group, requested before h is staged (an empty
            // source where the wave has nothing to compute)
            const bool v2 = good2 && ws < a.na2;
            const W4Src src2 = v2 ? make_src<4>(wm2, I, H) : empty_src(a.x);
            GroupLoad<4> A2;
            load_group<4>(A2, src2, clamp_group(myslot2, G2), v2 ? col2 : 0, true);
            __builtin_amdgcn_sched_barrier(0);
            if (rt) {
                // the whole row requested at once (16-byte device-scope loads)
                const int srow = __builtin_amdgcn_readfirstlane(slot);
                const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
                    a.h + (size_t)srow * I, (short)0, I * 2, kBufWord3);
                const int ts = tid % (64 * kSubWaves);
                u4_t hv[kRowChunksPerThread];
#pragma unroll
                for (int u = 0; u < kRowChunksPerThread; ++u)
                    hv[u] = __builtin_amdgcn_raw_buffer_load_b128(
                        hr, (ts + u * 64 * kSubWaves) * 16, 0, kAuxDev);
#pragma unroll
                for (int u = 0; u < kRowChunksPerThread; ++u) {
                    const int c = ts + u * 64 * kSubWaves;
                    if (c < K8_2) hs[c] = permute_chunk<4>(__builtin_bit_cast(uint4, hv[u]));
                }
            }
            __syncthreads();
            if (rt) {
                for (int gg = tid % (64 * kSubWaves); gg < G2; gg += 64 * kSubWaves) {
                    const uint4* xr = hs + gg * QF<4>::kChunks;
                    float s4[2] = {0.0f, 0.0f};
#pragma unroll 4
                    for (int c = 0; c < QF<4>::kChunks; ++c) {
                        const uint4 p = xr[c];
                        const h2_t x0 = as_h2(p.x), x1 = as_h2(p.y), x2 = as_h2(p.z), x3 = as_h2(p.w);
                        s4[0] += ((float)x0.x + (float)x0.y) + ((float)x2.x + (float)x2.y);
                        s4[1] += ((float)x1.x + (float)x1.y) + ((float)x3.x + (float)x3.y);
                    }
                    hsum[gg] = make_float4(s4[0], s4[1], 0.0f, 0.0f);
                }
            }
            __syncthreads();
            if (rt) {
                if (!good2 && tid % (64 * kSubWaves) == 0 && cb2 == 0)
                    flag_error(a.err, SMOE_DERR_NULL_EXPERT);
                if (v2) {
                    float acc[1][4] = {{0.0f, 0.0f, 0.0f, 0.0f}};
                    auto ld = [&](GroupLoad<4>& L, int g) { load_group<4>(L, src2, g, col2, true); };
                    item_groups<NG2>(ld, hs, hsum, myslot2, nslots2, G2, K8_2, zero_shift<4>(col2),
                                     acc, A2);
                    item_partials<LPR2>(acc, rd, ws, lane);
                }
            } else {
                if constexpr (CPLS2 > 0) {
                    if (i < a.n_dn)
                        shared_item<2, CPLS2, 1, true>(a.sh_h, a.sw2, a.Is, 0, H, i - n_rt2, ws,
                                                       lane, a.sh_out);
                }
            }
            __syncthreads();
            if (rt) {
                const int cb = i - slot * a.nCB2;
                const smoe_w4_mat wm = slot_mat<2>(mat_s, slot);
                const int ts = tid % (64 * kSubWaves);
                if (wm.qweight && wm.scales && wm.qzeros && ts < NB2 && cb * NB2 + ts < H) {
                    float v = 0.0f;
                    for (int w = 0; w < a.na2; ++w) v += rd[w * NB2 + ts];
                    st_dev(a.y + (size_t)slot * H + cb * NB2 + ts, f2h(v));
                }
            }
            __syncthreads();
        }
        ok = layer_sync(a, ++nbar, &flag_s);
    }

    // ---- F: combine (+ norm, + the next layer's router logits) ----
    if (ok && b < a.nF) {
        if (wave == 0)
            smoe_route::topk_softmax_wave(lg_s, E, k, a.renorm, a.wsg != nullptr, lane, ids_w,
                                          w_s, &gate_s, nullptr);
        __syncthreads();
        const int nch = H / 8;
        uint4* row = reinterpret_cast<uint4*>(dyn);
        const bool writer = b == 0;
        float sq = 0.0f;
        if (tid < smoe_comb::kCombThreads)
            for (int c8 = tid; c8 < nch; c8 += smoe_comb::kCombThreads) {
                float acc[8];
                smoe_comb::combine_chunk(a.y, pp_s, w_s, a.sw13 ? a.sh_out : nullptr,
                                         a.wsg ? &gate_s : nullptr, a.resid, 0, k, H, c8, acc,
                                         DevRows());
                const uint4 ov = smoe_comb::round_chunk(acc, sq);
                row[c8] = ov;
                if (writer) reinterpret_cast<uint4*>(a.out)[c8] = ov;
            }
        if (a.norm_out) {
            const float inv = smoe_comb::row_inv_rms(sq, H, a.eps, redf);
            if (tid < smoe_comb::kCombThreads)
                for (int c8 = tid; c8 < nch; c8 += smoe_comb::kCombThreads) {
                    const uint4 qv = smoe_comb::norm_chunk(row[c8], inv);
                    row[c8] = qv;
                    if (writer) reinterpret_cast<uint4*>(a.norm_out)[c8] = qv;
                }
            __syncthreads();
            if (a.wr_next)
                smoe_route::wave_logits(reinterpret_cast<const uint16_t*>(row), a.wr_next,
                                        a.wsg_next, H, a.E_next, a.nvec_next,
                                        b * kLayerWaves + wave, a.nvec_next, a.nF * kLayerWaves,
                                        a.lg_next, lane);
        }
    }
    layer_exit(a);
}

struct PhasePlan {
    int lpr, nCB, waves, mch, xr, direct;
    int ng;  // one-token workgroups: groups per slot (ceil(G / slots per workgroup))
    size_t lds;
};

// K per pseudo-group of a code width (QF<BITS>::kK).
int pseudo_group_k(int bits) { return bits == 8 ? 64 : 128; }

PhasePlan plan_phase(int phase, int slots, int T, int K, int N, int I, int maxm, int bits) {
    // LPR 16 (64-column blocks, 256-byte row runs) when that still gives
    // SMOE_W4_MIN_WG workgroups and no slot walks more than
    // SMOE_W4_MAX_GROUPS_PER_SLOT groups in sequence; else LPR 8 (32 columns,
    // twice the workgroups and slots).  Measured on the decode shapes (H 2048
    // and 4096, I 1408 and 6400, one to sixteen rows per expert).
    PhasePlan p{};
    const int cols16 = (phase == 1) ? I / 32 : (N + 63) / 64;
    const int G16 = K / pseudo_group_k(bits);
    const int maxw = (maxm == 1) ? kT1MaxWaves : kMaxWaves;
    const int min_wg = (maxm == 1) ? kT1MinWG : SMOE_W4_MIN_WG;
    const int serial16 = (G16 + 4 * maxw - 1) / (4 * maxw);
    p.lpr = ((long long)slots * cols16 >= min_wg &&
             serial16 <= SMOE_W4_MAX_GROUPS_PER_SLOT) ? 16 : 8;
    const int NB = 4 * p.lpr;
    p.nCB = (phase == 1) ? I / (NB / 2) : (N + NB - 1) / NB;
    const int rpl = 64 / p.lpr;
    const int G = K / pseudo_group_k(bits);
    p.waves = (G + rpl - 1) / rpl;
    // the launch bound caps every kernel at kMaxWaves; the multi-row kernels'
    // register budget at 4
    const int wmax = (maxm == 1) ? kT1MaxWaves : (kMaxWaves < 4 ? kMaxWaves : 4);
    if (p.waves > wmax) p.waves = wmax;
    // one-token workgroups request the whole activation row up front
    if (maxm == 1) {
        const int need = (K / 8 + 64 * kRowChunksPerThread - 1) / (64 * kRowChunksPerThread);
        if (p.waves < need) p.waves = need;
    }
    if (p.waves < 1) p.waves = 1;
    const size_t row_bytes = (size_t)K * 2 + (size_t)G * 16;  // pairs + per-class sums
    int cap = (int)(kLdsBytes / row_bytes);
    if (cap < 1) cap = 1;
    p.mch = cap < maxm ? cap : maxm;
    p.direct = (phase == 1 && T <= cap) ? 1 : 0;
    p.xr = p.direct ? T : p.mch;
    const size_t red_bytes = (size_t)p.waves * rpl * maxm * NB * 4;
    p.lds = (size_t)p.xr * row_bytes + red_bytes;
    p.ng = (G + p.waves * rpl - 1) / (p.waves * rpl);
    return p;
}

// The MFMA multi-row kernel: 64-column blocks, chunks of up to 16 rows within
// the staging budget (all T rows at once for the gate/up projection when they
// fit).
PhasePlan plan_mfma(int phase, int T, int K, int N, int I) {
    PhasePlan p{};
    p.lpr = 16;
    p.nCB = (phase == 1) ? I / 32 : (N + 63) / 64;
    const int W = (phase == 1) ? mfma_waves<1>() : mfma_waves<2>();
    p.waves = W;
    const int G = K / 128;
    const size_t row_bytes = (size_t)K * 2 + (size_t)G * 16;
    int cap = (int)(kMfmaLdsBytes / row_bytes);
    if (cap < 1) cap = 1;
    p.mch = cap < kMfmaRows ? cap : kMfmaRows;
    p.direct = (phase == 1 && T <= cap) ? 1 : 0;
    p.xr = p.direct ? T : p.mch;
    // (a wave's last global->LDS row load may fill up to 63 chunks, 1008
    // bytes, past the rows: into the sums and the reduction area, at least
    // W * 256 bytes together and both unused while rows are staged)
    p.lds = (size_t)p.xr * row_bytes + (size_t)W * p.mch * 64 * 4;
    p.ng = 1;
    return p;
}

template <int BITS, int PHASE, int LPR, int NG>
hipError_t launch_one_token(const W4Args& a, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
    hipLaunchKernelGGL((w4_kernel<BITS, PHASE, LPR, 1, NG>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int BITS, int PHASE, int LPR>
hipError_t launch_one_token_ng(const W4Args& a, dim3 grid, dim3 block, const PhasePlan& p,
                               hipStream_t s) {
    switch (p.ng) {
        case 1: return launch_one_token<BITS, PHASE, LPR, 1>(a, grid, block, p.lds, s);
        case 2: return launch_one_token<BITS, PHASE, LPR, 2>(a, grid, block, p.lds, s);
        case 3: return launch_one_token<BITS, PHASE, LPR, 3>(a, grid, block, p.lds, s);
        case 4: return launch_one_token<BITS, PHASE, LPR, 4>(a, grid, block, p.lds, s);
        default: return hipErrorInvalidValue;  // the caller falls back to the multi-row kernel
    }
}

template <int BITS, int PHASE, int MAXM>
hipError_t launch_phase(const W4Args& a, int slots, const PhasePlan& p, hipStream_t s) {
    const dim3 grid(slots * p.nCB), block(64 * p.waves);
    if (MAXM == 1)
        return (p.lpr == 16) ? launch_one_token_ng<BITS, PHASE, 16>(a, grid, block, p, s)
                             : launch_one_token_ng<BITS, PHASE, 8>(a, grid, block, p, s);
    if (p.lpr == 16)
        hipLaunchKernelGGL((w4_kernel<BITS, PHASE, 16, MAXM, 1>), grid, block, p.lds, s, a);
    else
        hipLaunchKernelGGL((w4_kernel<BITS, PHASE, 8, MAXM, 1>), grid, block, p.lds, s, a);
    return hipGetLastError();
}

template <int PHASE>
hipError_t launch_any(const W4Args& a, int slots, const PhasePlan& p, int maxm, int bits,
                      hipStream_t s) {
    if (bits == 2)
        return (maxm == 1) ? launch_phase<2, PHASE, 1>(a, slots, p, s)
                           : launch_phase<2, PHASE, 4>(a, slots, p, s);
    if (bits == 8)
        return (maxm == 1) ? launch_phase<8, PHASE, 1>(a, slots, p, s)
                           : launch_phase<8, PHASE, 4>(a, slots, p, s);
    return (maxm == 1) ? launch_phase<4, PHASE, 1>(a, slots, p, s)
                       : launch_phase<4, PHASE, 4>(a, slots, p, s);
}

}  // namespace

namespace smoe {
// h [T*k, I] fp16, then (one-token steps) a SlotDesc per slot
static size_t h_bytes(int T, int k, int I) { return ((size_t)T * k * I * 2 + 255) & ~(size_t)255; }

static size_t desc_bytes(int T, int k, int E) {
    const int slots = E < T * k ? E : T * k;
    return ((size_t)slots * sizeof(SlotDesc) + 255) & ~(size_t)255;
}

// h, the slot descriptors, then the router logits of a one-token step
size_t w4a16_workspace_bytes(int T, int k, int /*H*/, int I, int E) {
    return h_bytes(T, k, I) + desc_bytes(T, k, E) + (((size_t)(E + 1) * 4 + 255) & ~(size_t)255);
}

bool w4a16_shape_supported(int H, int I) {
    // activation rows staged in LDS; one-token workgroups request a whole row
    // with kRowChunksPerThread chunks per thread
    const int row_cap = 8 * 64 * kRowChunksPerThread * kT1MaxWaves;
    return (size_t)H * 2 <= (size_t)kLdsBytes && (size_t)I * 2 <= (size_t)kLdsBytes &&
           H <= row_cap && I <= row_cap;
}

namespace {
W4Args phase_args(const PhasePlan& p, const uint16_t* xin, const int32_t* sorted_token,
                  const int32_t* off, const int32_t* active, const int32_t* n_active,
                  const smoe_w4_expert* experts, int K, int N, int I, int T, int E,
                  uint16_t* out, int32_t* err, SlotDesc* desc) {
    W4Args a{};
    a.desc = desc;
    a.xin = xin;
    a.sorted_token = sorted_token;
    a.off = off;
    a.active = active;
    a.n_active = n_active;
    a.experts = experts;
    a.K = K;
    a.N = N;
    a.I = I;
    a.nCB = p.nCB;
    a.MCH = p.mch;
    a.XR = p.xr;
    a.direct = p.direct;
    a.T = T;
    a.E = E;
    a.out = out;
    a.err = err;
    return a;
}
}  // namespace

hipError_t launch_w4a16_ffn(const uint16_t* x, const int32_t* sorted_token, const int32_t* off,
                            const int32_t* active, const int32_t* n_active,
                            const smoe_w4_expert* experts, int T, int k, int H, int I, int E,
                            int bits, uint16_t* y, void* ws, int32_t* err, hipStream_t s,
                            const uint16_t* const* ascale) {
    const int rows = T * k;
    const int slots = E < rows ? E : rows;
    // an expert holds at most T rows; one-token kernels unless a slot would
    // walk more than four pseudo-groups (long 8-bit reductions)
    int maxm = (T == 1) ? 1 : 4;
    PhasePlan p1 = plan_phase(1, slots, T, H, 2 * I, I, maxm, bits);
    PhasePlan p2 = plan_phase(2, slots, T, I, H, I, maxm, bits);
    if (maxm == 1 && (p1.ng > 4 || p2.ng > 4)) {
        maxm = 4;
        p1 = plan_phase(1, slots, T, H, 2 * I, I, maxm, bits);
        p2 = plan_phase(2, slots, T, I, H, I, maxm, bits);
    }
    uint16_t* h = static_cast<uint16_t*>(ws);
    SlotDesc* desc = reinterpret_cast<SlotDesc*>(static_cast<char*>(ws) + h_bytes(T, k, I));
    // multi-row 4-bit steps take the MFMA kernel, except with AWQ-style
    // divisors (applied where the VALU kernels stage their rows)
    if (maxm > 1 && bits == 4 && SMOE_W4_MFMA && !ascale) {
        const PhasePlan m1 = plan_mfma(1, T, H, 2 * I, I);
        const W4Args b1 = phase_args(m1, x, sorted_token, off, active, n_active, experts, H,
                                     2 * I, I, T, E, h, err, desc);
        hipLaunchKernelGGL((w4_mfma_kernel<1>), dim3(slots * m1.nCB), dim3(64 * m1.waves),
                           m1.lds, s, b1, RowsShared{});
        hipError_t e1 = hipGetLastError();
        if (e1 != hipSuccess) return e1;
        const PhasePlan m2 = plan_mfma(2, T, I, H, I);
        const W4Args b2 =
            phase_args(m2, h, nullptr, off, active, n_active, experts, I, H, I, T, E, y, err, desc);
        hipLaunchKernelGGL((w4_mfma_kernel<2>), dim3(slots * m2.nCB), dim3(64 * m2.waves),
                           m2.lds, s, b2, RowsShared{});
        return hipGetLastError();
    }
    W4Args a1 = phase_args(p1, x, sorted_token, off, active, n_active, experts, H, 2 * I, I, T, E,
                           h, err, desc);
    a1.ascale = ascale;
    hipError_t st = launch_any<1>(a1, slots, p1, maxm, bits, s);
    if (st != hipSuccess) return st;
    W4Args a2 =
        phase_args(p2, h, nullptr, off, active, n_active, experts, I, H, I, T, E, y, err, desc);
    a2.ascale = ascale;
    return launch_any<2>(a2, slots, p2, maxm, bits, s);
}

#ifndef SMOE_SH_FRONT_ROWS
#define SMOE_SH_FRONT_ROWS 0  // matrix-vector shared items first in the multi-row launches
#endif
#ifndef SMOE_SH_FRONT_MFMA
#define SMOE_SH_FRONT_MFMA 1  // MFMA shared items first
#endif

// The shared expert's projection as launches of its own (4 columns per
// workgroup), any chunk count of the matrix-vector routine.
// (chunk counts rounded up as verify_grouped_gemm's matrix-vector launches
// round them)
template <int PHASE>
static hipError_t launch_shared_rows(const RowsShared& sh, int cpl, hipStream_t s) {
    const dim3 grid((sh.Ncol + 3) / 4), block(256);
    if (cpl <= 2) shared_rows_kernel<PHASE, 2><<<grid, block, 0, s>>>(sh);
    else if (cpl <= 4) shared_rows_kernel<PHASE, 4><<<grid, block, 0, s>>>(sh);
    else if (cpl <= 6) shared_rows_kernel<PHASE, 6><<<grid, block, 0, s>>>(sh);
    else if (cpl <= 8) shared_rows_kernel<PHASE, 8><<<grid, block, 0, s>>>(sh);
    else if (cpl <= 12) shared_rows_kernel<PHASE, 12><<<grid, block, 0, s>>>(sh);
    else shared_rows_kernel<PHASE, 16><<<grid, block, 0, s>>>(sh);
    return hipGetLastError();
}

hipError_t launch_w4a16_ffn_shared(const uint16_t* x, const int32_t* sorted_token,
                                   const int32_t* off, const int32_t* active,
                                   const int32_t* n_active, const smoe_w4_expert* experts, int T,
                                   int k, int H, int I, int E, uint16_t* y, void* ws,
                                   const uint16_t* sw13, const uint16_t* sw2, int Is,
                                   uint16_t* sh_h, uint16_t* sh_out, int32_t* err,
                                   hipStream_t s) {
    // the shared expert as verify_grouped_gemm computes one group of all T
    // rows: the matrix-vector routine up to 4 rows, else the one-group ring
    const bool gemv = T <= 4 && H <= 512 * smoe_gemv::kMaxChunks &&
                      Is <= 512 * smoe_gemv::kMaxChunks;
    const RowsShared g1{sw13, x, sh_h, H, Is, Is, T, 0};
    const RowsShared g2{sw2, sh_h, sh_out, Is, H, Is, T, 0};
    const int c1 = smoe_gemv::chunks_for(H), c2 = smoe_gemv::chunks_for(Is);
    const bool mfma = T > 1 && SMOE_W4_MFMA;  // launch_w4a16_ffn's multi-row 4-bit path
    // (fused chunk counts: those whose item fits the launches' register
    // budget; 12 for the down projection spilled)
    if (gemv && mfma && (c1 == 4 || c1 == 8) && (c2 == 6 || c2 == 8)) {
        // its columns as the last workgroups of the two multi-row launches
        const int rows = T * k;
        const int slots = E < rows ? E : rows;
        uint16_t* h = static_cast<uint16_t*>(ws);
        SlotDesc* desc =
            reinterpret_cast<SlotDesc*>(static_cast<char*>(ws) + h_bytes(T, k, I));
        const PhasePlan m1 = plan_mfma(1, T, H, 2 * I, I);
        const W4Args b1 = phase_args(m1, x, sorted_token, off, active, n_active, experts, H,
                                     2 * I, I, T, E, h, err, desc);
        RowsShared s1 = g1;
        s1.wg0 = slots * m1.nCB;
        const int nsh1 = (Is + m1.waves - 1) / m1.waves;  // one column per wave
        if (SMOE_SH_FRONT_ROWS) s1.nfront = nsh1;
        const dim3 grid1(slots * m1.nCB + nsh1), block(64 * m1.waves);
        if (c1 == 4) hipLaunchKernelGGL((w4_mfma_kernel<1, 4>), grid1, block, m1.lds, s, b1, s1);
        else hipLaunchKernelGGL((w4_mfma_kernel<1, 8>), grid1, block, m1.lds, s, b1, s1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const PhasePlan m2 = plan_mfma(2, T, I, H, I);
        const W4Args b2 =
            phase_args(m2, h, nullptr, off, active, n_active, experts, I, H, I, T, E, y, err, desc);
        RowsShared s2 = g2;
        s2.wg0 = slots * m2.nCB;
        const int nsh2 = (H + m2.waves - 1) / m2.waves;
        if (SMOE_SH_FRONT_ROWS) s2.nfront = nsh2;
        const dim3 grid2(slots * m2.nCB + nsh2), block2(64 * m2.waves);
        if (c2 == 6) hipLaunchKernelGGL((w4_mfma_kernel<2, 6>), grid2, block2, m2.lds, s, b2, s2);
        else hipLaunchKernelGGL((w4_mfma_kernel<2, 8>), grid2, block2, m2.lds, s, b2, s2);
        return hipGetLastError();
    }
    // 5-16 rows: 16-column MFMA items with the one-group ring launches'
    // arithmetic (those launches' geometry needs at least 8 steps of 128 K;
    // the items' buffer offsets are 32-bit)
    if (!gemv && mfma && T <= 16 && H / 128 >= 8 && Is / 128 >= 8 &&
        4LL * Is * H < 0x7FFFFFFFLL) {
        const int rows = T * k;
        const int slots = E < rows ? E : rows;
        uint16_t* h = static_cast<uint16_t*>(ws);
        SlotDesc* desc =
            reinterpret_cast<SlotDesc*>(static_cast<char*>(ws) + h_bytes(T, k, I));
        constexpr int ipw1 = mfma_waves<1>() / SMOE_SH_GU_WAVES;  // items per workgroup
        constexpr int ipw2 = mfma_waves<2>() / SMOE_SH_DN_WAVES;
        const size_t red1 = (size_t)mfma_waves<1>() * 2 * 64 * 16;
        const size_t red2 = (size_t)mfma_waves<2>() * 64 * 16;
        PhasePlan m1 = plan_mfma(1, T, H, 2 * I, I);
        if (m1.lds < red1) m1.lds = red1;
        const W4Args b1 = phase_args(m1, x, sorted_token, off, active, n_active, experts, H,
                                     2 * I, I, T, E, h, err, desc);
        RowsShared s1 = g1;
        s1.wg0 = slots * m1.nCB;
        if (SMOE_SH_FRONT_MFMA) s1.nfront = (Is / 16 + ipw1 - 1) / ipw1;
        hipLaunchKernelGGL((w4_mfma_kernel<1, -1>), dim3(s1.wg0 + (Is / 16 + ipw1 - 1) / ipw1),
                           dim3(64 * m1.waves), m1.lds, s, b1, s1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        PhasePlan m2 = plan_mfma(2, T, I, H, I);
        if (m2.lds < red2) m2.lds = red2;
        const W4Args b2 =
            phase_args(m2, h, nullptr, off, active, n_active, experts, I, H, I, T, E, y, err, desc);
        RowsShared s2 = g2;
        s2.wg0 = slots * m2.nCB;
        if (SMOE_SH_FRONT_MFMA) s2.nfront = (H / 16 + ipw2 - 1) / ipw2;
        hipLaunchKernelGGL((w4_mfma_kernel<2, -1>), dim3(s2.wg0 + (H / 16 + ipw2 - 1) / ipw2),
                           dim3(64 * m2.waves), m2.lds, s, b2, s2);
        return hipGetLastError();
    }
    hipError_t e = launch_w4a16_ffn(x, sorted_token, off, active, n_active, experts, T, k, H, I,
                                    E, 4, y, ws, err, s);
    if (e != hipSuccess) return e;
    if (!gemv) return launch_dense_group(x, T, H, sw13, sw2, Is, sh_h, sh_out, err, s);
    e = launch_shared_rows<1>(g1, c1, s);
    if (e != hipSuccess) return e;
    return launch_shared_rows<2>(g2, c2, s);
}

bool draft_route_ffn_supported(int E, int k) { return E <= 256 && k <= kFusedMaxK; }

// The shared expert's projection as its own launch (no fused instantiation
// for its chunk count).
template <int PHASE>
hipError_t launch_shared_gemv(const SharedArgs& sh, const uint16_t* x, int H, int cpl,
                              hipStream_t s) {
    const int ncol = (PHASE == 1) ? sh.Is : H;
    const dim3 grid((ncol + 3) / 4), block(256);
    switch (cpl) {
        case 2: shared_gemv_kernel<PHASE, 2><<<grid, block, 0, s>>>(sh, x, H); break;
        case 4: shared_gemv_kernel<PHASE, 4><<<grid, block, 0, s>>>(sh, x, H); break;
        case 6: shared_gemv_kernel<PHASE, 6><<<grid, block, 0, s>>>(sh, x, H); break;
        case 8: shared_gemv_kernel<PHASE, 8><<<grid, block, 0, s>>>(sh, x, H); break;
        case 12: shared_gemv_kernel<PHASE, 12><<<grid, block, 0, s>>>(sh, x, H); break;
        default: shared_gemv_kernel<PHASE, 16><<<grid, block, 0, s>>>(sh, x, H); break;
    }
    return hipGetLastError();
}

hipError_t launch_draft_route_ffn(const uint16_t* x, const uint16_t* wr, const uint16_t* wsg,
                                  int H, int E, int k, int renorm, int32_t* counters_row,
                                  int32_t* ids, float* w, float* gate, int32_t* off, int32_t* st,
                                  int32_t* sp, int32_t* pp, int32_t* active, int32_t* n_active,
                                  const smoe_w4_expert* experts, int I, uint16_t* y, void* ws,
                                  const uint16_t* sw13, const uint16_t* sw2, int Is,
                                  uint16_t* sh_h, uint16_t* sh_out, const float* logits_in,
                                  int32_t* err, hipStream_t s) {
    const int nvec = E + (wsg ? 1 : 0);
    uint16_t* h = static_cast<uint16_t*>(ws);
    SlotDesc* desc = reinterpret_cast<SlotDesc*>(static_cast<char*>(ws) + h_bytes(1, k, I));
    const float* logits = logits_in;
    if (!logits) {
        // the token's router logits, one wave per router row (the caller
        // passes them when an earlier launch computed them)
        float* lg = reinterpret_cast<float*>(static_cast<char*>(ws) + h_bytes(1, k, I) +
                                             desc_bytes(1, k, E));
        constexpr int kLogitWaves = 4;
        route_logits_kernel<<<dim3((nvec + kLogitWaves - 1) / kLogitWaves),
                              dim3(64 * kLogitWaves), 0, s>>>(x, wr, wsg, H, E, nvec, lg);
        hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return e0;
        logits = lg;
    }
    const PhasePlan p1 = plan_phase(1, k, 1, H, 2 * I, I, 1, 4);
    const W4Args a1 = phase_args(p1, x, st, off, active, n_active, experts, H, 2 * I, I, 1, E, h,
                                 err, desc);
    RouteArgs r{wr,  wsg, logits, k,  renorm, counters_row, ids,    w,
                gate, off, st,     sp, pp,     active,       n_active};
    if (p1.ng < 1 || p1.ng > 4) return hipErrorInvalidValue;  // excluded by the shape checks
    // The shared expert (if any): its gate/up columns ride in the gate/up
    // launch when H takes 4 or 8 chunks per lane (two columns per wave), its
    // down columns in the down launch when Is takes 6, 8 or 12; other shapes
    // run the same routine as launches of their own.
    SharedArgs sh{sw13, sw2, Is, k * p1.nCB + 1, sh_h, sh_out};
    const int c1 = sw13 ? smoe_gemv::chunks_for(H) : 0;
    const int cs1 = (c1 == 4 || c1 == 8) ? c1 : 0;
    const int nsh1 = cs1 ? (Is + 2 * p1.waves - 1) / (2 * p1.waves) : 0;
    const dim3 grid(k * p1.nCB + 1 + nsh1), block(64 * p1.waves);  // + the routing workgroup
#define SMOE_ROUTE_W4(L, NG)                                                                     \
    do {                                                                                         \
        if (cs1 == 4) hipLaunchKernelGGL((route_w4_kernel<L, NG, 4>), grid, block, p1.lds, s, a1, r, sh); \
        else if (cs1 == 8) hipLaunchKernelGGL((route_w4_kernel<L, NG, 8>), grid, block, p1.lds, s, a1, r, sh); \
        else hipLaunchKernelGGL((route_w4_kernel<L, NG, 0>), grid, block, p1.lds, s, a1, r, sh); \
    } while (0)
    if (p1.lpr == 16) {
        if (p1.ng == 1) SMOE_ROUTE_W4(16, 1);
        else if (p1.ng == 2) SMOE_ROUTE_W4(16, 2);
        else if (p1.ng == 3) SMOE_ROUTE_W4(16, 3);
        else SMOE_ROUTE_W4(16, 4);
    } else {
        if (p1.ng == 1) SMOE_ROUTE_W4(8, 1);
        else if (p1.ng == 2) SMOE_ROUTE_W4(8, 2);
        else if (p1.ng == 3) SMOE_ROUTE_W4(8, 3);
        else SMOE_ROUTE_W4(8, 4);
    }
#undef SMOE_ROUTE_W4
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (sw13 && !cs1) {
        e = launch_shared_gemv<1>(sh, x, H, c1, s);
        if (e != hipSuccess) return e;
    }
    const PhasePlan p2 = plan_phase(2, k, 1, I, H, I, 1, 4);
    const W4Args a2 = phase_args(p2, h, nullptr, off, active, n_active, experts, I, H, I, 1, E, y,
                                 err, desc);
    const int c2 = sw13 ? smoe_gemv::chunks_for(Is) : 0;
    const bool fuse2 = (c2 == 6 || c2 == 8 || c2 == 12) && p2.ng <= 2;
    if (!fuse2) {
        e = launch_any<2>(a2, k, p2, 1, 4, s);
        if (e != hipSuccess || !sw13) return e;
        return launch_shared_gemv<2>(sh, x, H, c2, s);
    }
    sh.wg0 = k * p2.nCB;
    const dim3 grid2(k * p2.nCB + (H + p2.waves - 1) / p2.waves), block2(64 * p2.waves);
#define SMOE_DOWN_SH(L, NG)                                                                      \
    do {                                                                                         \
        if (c2 == 6) hipLaunchKernelGGL((w4_down_shared_kernel<L, NG, 6>), grid2, block2, p2.lds, s, a2, sh); \
        else if (c2 == 8) hipLaunchKernelGGL((w4_down_shared_kernel<L, NG, 8>), grid2, block2, p2.lds, s, a2, sh); \
        else hipLaunchKernelGGL((w4_down_shared_kernel<L, NG, 12>), grid2, block2, p2.lds, s, a2, sh); \
    } while (0)
    if (p2.lpr == 16) {
        if (p2.ng == 1) SMOE_DOWN_SH(16, 1);
        else SMOE_DOWN_SH(16, 2);
    } else {
        if (p2.ng == 1) SMOE_DOWN_SH(8, 1);
        else SMOE_DOWN_SH(8, 2);
    }
#undef SMOE_DOWN_SH
    return hipGetLastError();
}
}  // namespace smoe

// ------------------------------------------------ one-launch draft layer ----
namespace {

struct LayerPlan {
    PhasePlan p1, p2;
    int P, row_bytes, lds, cs1, cs2, nsh1, nsh2, variant;
};

// Instantiated geometries (gate/up LPR and groups per slot, down LPR and
// groups per slot, shared-expert chunks per lane of gate/up and down):
//   0: 16/2, 8/2, none       (H 4096, I 6400: the Phi-3.5-MoE layer)
//   1: 16/1, 16/1, none      (H 2048, I 1408)
//   2: 16/1, 16/1, 4 / 6     (H 2048, I 1408, shared I 2816: DeepSeek-V2-Lite)
//   3: 16/1, 16/1, 4 / 12    (H 2048, I 1408, shared I 5632: Qwen1.5-MoE)
constexpr int kLayerStatic = 4096;            // the kernel's static arrays (< 4 KB)
constexpr int kLayerLdsMax = 160 * 1024;
constexpr int kLayerLdsOnePerCU = 84 * 1024;  // more than half a CU's LDS

bool plan_layer(int H, int I, int E, int k, int Is, LayerPlan& L) {
    if (E < 1 || E > kSpecTable || k < 1 || k > kFusedMaxK || k > E) return false;
    if (H % 128 || I % 128 || H > 8192 || I > 16384 || H <= 0 || I <= 0) return false;
    L.p1 = plan_phase(1, k, 1, H, 2 * I, I, 1, 4);
    L.p2 = plan_phase(2, k, 1, I, H, I, 1, 4);
    if (L.p1.waves > kSubWaves || L.p2.waves > kSubWaves) return false;
    L.cs1 = Is ? smoe_gemv::chunks_for(H) : 0;
    L.cs2 = Is ? smoe_gemv::chunks_for(Is) : 0;
    const int g1 = L.p1.lpr * 10 + L.p1.ng, g2 = L.p2.lpr * 10 + L.p2.ng;
    L.variant = -1;
    if (g1 == 162 && g2 == 82 && !Is) L.variant = 0;
    if (g1 == 161 && g2 == 161) {
        if (!Is) L.variant = 1;
        else if (L.cs1 == 4 && L.cs2 == 6) L.variant = 2;
        else if (L.cs1 == 4 && L.cs2 == 12) L.variant = 3;
    }
    if (L.variant < 0) return false;
    const int NB2 = 4 * L.p2.lpr;
    if (H % NB2) return false;
    L.P = smoe::device_cu_count();
    if (L.P <= 0) return false;
    const int G2 = I / 128, G1 = H / 128;
    int rb = H / 8 * 16 + G1 * 16;
    rb = std::max(rb, 2 * (I / 8) * 16 + 2 * G2 * 16);
    rb = std::max(rb, 2 * H);
    L.row_bytes = (rb + 255) & ~255;
    L.lds = L.row_bytes + 2 * kLayerRed * 4;  // dynamic part
    if (kLayerStatic + L.lds > kLayerLdsMax) return false;
    // one workgroup per CU: every CU streams its share
    L.lds = std::max(L.lds, kLayerLdsOnePerCU - kLayerStatic);
    L.nsh1 = Is ? (Is + 2 * kSubWaves - 1) / (2 * kSubWaves) : 0;
    L.nsh2 = Is ? (H + kSubWaves - 1) / kSubWaves : 0;
    return true;
}

template <int LPR1, int NG1, int LPR2, int NG2, int CPLS1, int CPLS2>
hipError_t launch_layer_variant(const LayerArgs& a, int lds, hipStream_t s) {
    static int lds_set = 0;  // the dynamic LDS limit raised for this instantiation
    auto fn = draft_layer_kernel<LPR1, NG1, LPR2, NG2, CPLS1, CPLS2>;
    if (lds > lds_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        lds_set = lds;
    }
    hipLaunchKernelGGL(fn, dim3(a.P), dim3(64 * kLayerWaves), lds, s, a);
    return hipGetLastError();
}

}  // namespace

namespace smoe {
bool draft_layer_supported(int H, int I, int E, int k, int Is) {
    LayerPlan L;
    return plan_layer(H, I, E, k, Is, L);
}

size_t draft_layer_workspace_bytes(int k, int I, int E) {
    const size_t lg = ((size_t)4 * (E + 1) + 255) & ~(size_t)255;
    return 256 + lg + h_bytes(1, k, I);
}

hipError_t launch_draft_layer(const DraftLayerCall& c, hipStream_t s) {
    LayerPlan L;
    if (!plan_layer(c.H, c.I, c.E, c.k, c.sw13 ? c.Is : 0, L)) return hipErrorNotSupported;
    LayerArgs a{};
    char* ws = static_cast<char*>(c.ws);
    a.sync = reinterpret_cast<uint32_t*>(ws);
    a.lg_ws = reinterpret_cast<float*>(ws + 256);
    a.h = reinterpret_cast<uint16_t*>(ws + 256 + (((size_t)4 * (c.E + 1) + 255) & ~(size_t)255));
    a.x = c.x;
    a.wr = c.wr;
    a.wsg = c.wsg;
    a.logits = c.logits;
    a.H = c.H;
    a.I = c.I;
    a.E = c.E;
    a.k = c.k;
    a.renorm = c.renorm;
    a.nvec = c.E + (c.wsg ? 1 : 0);
    a.experts = c.experts;
    a.counters_row = c.counters_row;
    a.ids = c.ids;
    a.w = c.w;
    a.gate = c.gate;
    a.off = c.off;
    a.sorted_token = c.st;
    a.sorted_pair = c.sp;
    a.pair_pos = c.pp;
    a.active = c.active;
    a.n_active = c.n_active;
    a.sw13 = c.sw13;
    a.sw2 = c.sw13 ? c.sw2 : nullptr;
    a.Is = c.sw13 ? c.Is : 0;
    a.sh_h = c.sh_h;
    a.y = c.y;
    a.sh_out = c.sh_out;
    a.resid = c.resid;
    a.out = c.out;
    a.norm_out = c.norm_out;
    a.eps = c.eps;
    a.wr_next = c.norm_out ? c.wr_next : nullptr;
    a.wsg_next = a.wr_next ? c.wsg_next : nullptr;
    a.E_next = c.E_next;
    a.nvec_next = a.wr_next ? c.E_next + (c.wsg_next ? 1 : 0) : 0;
    a.lg_next = c.lg_next;
    a.err = c.err;
    a.P = L.P;
    a.nCB1 = L.p1.nCB;
    a.na1 = L.p1.waves;
    a.nCB2 = L.p2.nCB;
    a.na2 = L.p2.waves;
    a.G2 = c.I / 128;
    a.n_gu = c.k * L.p1.nCB + L.nsh1;
    a.n_dn = c.k * L.p2.nCB + L.nsh2;
    a.R1 = (a.n_gu + 2 * L.P - 1) / (2 * L.P);
    a.R2 = (a.n_dn + 2 * L.P - 1) / (2 * L.P);
    a.nF = a.wr_next ? (a.nvec_next + kLayerWaves - 1) / kLayerWaves : 1;
    if (a.nF > L.P) return hipErrorNotSupported;
    a.row_bytes = L.row_bytes;
    switch (L.variant) {
        case 0: return launch_layer_variant<16, 2, 8, 2, 0, 0>(a, L.lds, s);
        case 1: return launch_layer_variant<16, 1, 16, 1, 0, 0>(a, L.lds, s);
        case 2: return launch_layer_variant<16, 1, 16, 1, 4, 6>(a, L.lds, s);
        case 3: return launch_layer_variant<16, 1, 16, 1, 4, 12>(a, L.lds, s);
        default: return hipErrorNotSupported;
    }
}
}  // namespace smoe
