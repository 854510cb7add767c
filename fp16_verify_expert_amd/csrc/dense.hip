// Dense-regime FP16 verify FFN: many rows per expert (a batched or long
// verification), a tiled grouped GEMM on MFMA.
//
// "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step Speculative
// Offloading" (AI summary), Key Contributions 4 and Methodology: packing the
// tokens routed to one expert turns per-token matrix-vector products into one
// matrix-matrix product per expert.  At K+1 <= 33 rows the product stays a
// weight stream (the kernels of verify.hip); once an expert holds a few
// hundred rows it is a real contraction, and this kernel is the one that
// keeps the matrix cores busy.
//
// Work decomposition.  A small planning kernel lists the touched experts
// with their row-tile counts; the GEMM grid covers every (expert, column
// block, 128-row tile) item, expert-major with an expert's row tiles
// innermost, so a weight tile is read from HBM once and re-read from L2 by
// the expert's other row tiles.  Workgroup b takes item (b mod 8) * W/8 +
// b / 8: blocks on one XCD (b mod 8) walk a contiguous run of items, which
// keeps an expert's activation rows and weight tiles in that XCD's L2.
//
// Tile.  128 rows x BN columns x 64 K per step, 4 waves in a 2 x 2 layout,
// each wave 64 x BN/2 = 4 x BN/32 MFMA 16x16x32 f16 blocks with fp32
// accumulators.  The gate/up projection takes BN = 256 (a wave reads 12
// fragments from LDS per 32 MFMAs instead of 8 per 16: 916 -> 815 us at the
// Phi-3.5-MoE shape, T = 2048), the down projection BN = 128.
// Operands are staged global -> registers -> LDS (rows padded to 144 bytes so
// the fragment reads of 16 rows hit 16 different bank groups); the next step's
// loads are in flight while the current step is multiplied.  In the gate/up
// projection the tile columns are pairs of (16 gate, 16 up) columns of
// the same h columns, so every lane holds the gate and up value of its
// outputs and applies SwiGLU in registers.  In the down projection a last,
// partial column block (H not a multiple of BN) re-reads the last weight
// row for the missing columns and does not store them.  With at least a full
// row tile per expert on average the same tile runs from a global->LDS ring
// instead (dense_ring_kernel below).
#include "common.h"

#ifndef SMOE_DENSE_STAGES
#define SMOE_DENSE_STAGES 3
#endif

namespace {

constexpr int kBM = 128;             // rows per tile
// tile columns BN: 256 in the gate/up projection, 128 in the down projection
constexpr int kBK = 64;              // K per step
constexpr int kLdsRow = kBK + 8;     // halves per LDS row (144 bytes)
constexpr int kThreads = 256;
constexpr int kChunksA = kBM * kBK / 8 / kThreads;  // 16-byte chunks per thread: activations

struct DenseArgs {
    const uint16_t* xin;          // phase 1: x [T, H]; phase 2: h [rows, I]
    const int32_t* sorted_token;  // phase 1
    const int32_t* off;
    const smoe_f16_expert* experts;
    const int32_t* plan;          // [0] = items, [1] = experts listed, then 4 ints per expert
    int K;
    int Ncol;   // output columns: I (phase 1, h) or H (phase 2, y)
    int I;
    int nNT;    // column blocks: I/(BN/2) (phase 1) or ceil(H/BN) (phase 2)
    int Wpad;   // grid size (a multiple of 8)
    uint16_t* out;
    int32_t* err;
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// One workgroup: for every listed expert (active order, masked ones left
// out) its row-tile count and the item base (prefix of tiles x column blocks).
__global__ __launch_bounds__(64) void dense_plan_kernel(const int32_t* __restrict__ off,
                                                        const int32_t* __restrict__ active,
                                                        const int32_t* __restrict__ n_active,
                                                        const uint8_t* __restrict__ mask, int E,
                                                        int nNT, int32_t* __restrict__ plan) {
    const int lane = threadIdx.x;
    const int na = active ? *n_active : E;
    int base_items = 0, base_slots = 0;
    for (int s0 = 0; s0 < na; s0 += 64) {
        const int s = s0 + lane;
        int e = -1, nmt = 0;
        if (s < na) {
            e = active ? active[s] : s;
            if (e >= 0 && e < E && !(mask && !mask[e])) {
                const int cnt = off[e + 1] - off[e];
                nmt = (cnt + kBM - 1) / kBM;
            }
        }
        const int listed = nmt > 0 ? 1 : 0;
        // inclusive scans of listed experts and of items
        int incl_l = listed, incl_i = nmt * nNT;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int ol = __shfl_up(incl_l, d);
            const int oi = __shfl_up(incl_i, d);
            if (lane >= d) {
                incl_l += ol;
                incl_i += oi;
            }
        }
        if (listed) {
            int32_t* p = plan + 2 + 4 * (base_slots + incl_l - 1);
            p[0] = e;
            p[1] = off[e];
            p[2] = nmt;
            p[3] = base_items + incl_i - nmt * nNT;
        }
        base_slots += __shfl(incl_l, 63);
        base_items += __shfl(incl_i, 63);
    }
    if (lane == 0) {
        plan[0] = base_items;
        plan[1] = base_slots;
    }
}

// 256-column tiles: two waves per SIMD (256 registers: 128 accumulators, the
// 12 fragments of a 32-K step and the next step's 12 staged chunks), two 54 KB
// workgroups per CU.  128-column tiles: three waves per SIMD (at most 168
// registers), three workgroups per CU.
template <int PHASE, int BN>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(BN == 256 ? 2 : 3))) void dense_gemm_kernel(DenseArgs a) {
    constexpr int kBN = BN;
    constexpr int kChunksB = kBN * kBK / 8 / kThreads;  // 16-byte chunks per thread: weights
    constexpr int kWN = kBN / 2;                        // columns per wave (2 x 2 waves)
    constexpr int kNB = kWN / 16;                       // 16-column MFMA blocks per wave
    __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLdsRow];

    // ---- which item ----
    const int b = blockIdx.x;
    const int item = (b & 7) * (a.Wpad >> 3) + (b >> 3);
    const int nitems = a.plan[0];
    if (item >= nitems) return;
    // the listed expert holding this item (item bases increase)
    const int nexp = a.plan[1];
    int lo = 0, hi = nexp - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.plan[2 + 4 * mid + 3] <= item) lo = mid;
        else hi = mid - 1;
    }
    const int32_t* pe = a.plan + 2 + 4 * lo;
    const int e = pe[0];
    const int rbase = pe[1];
    const int nmt = pe[2];
    const int j = item - pe[3];
    const int nt = j / nmt;
    const int mt = j - nt * nmt;
    const int m0 = rbase + mt * kBM;
    const int r1 = a.off[e + 1];
    const uint16_t* W = (PHASE == 1) ? a.experts[e].w13 : a.experts[e].w2;
    if (!W) {
        if (threadIdx.x == 0 && nt == 0 && mt == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
        return;
    }
    const int K = a.K;

    // ---- this thread's global chunks (A: activation rows, B: weight rows),
    //      as element offsets (every operand holds < 2^31 elements) ----
    const int tid = threadIdx.x;
    int aoff[kChunksA], boff[kChunksB];
#pragma unroll
    for (int u = 0; u < kChunksA; ++u) {
        const int q = tid + u * kThreads;  // chunk: row q/8, 16-byte chunk q%8
        const int row = q >> 3;
        const int c = q & 7;
        const int r = m0 + row;
        // rows past the expert's group load nothing (zeros)
        aoff[u] = (r < r1) ? ((PHASE == 1) ? a.sorted_token[r] : r) * K + c * 8 : -1;
    }
#pragma unroll
    for (int u = 0; u < kChunksB; ++u) {
        const int q = tid + u * kThreads;
        const int row = q >> 3;
        const int c = q & 7;
        int n;
        if (PHASE == 1) {
            const int p = row >> 5, w = row & 31;  // pair p: 16 gate rows then 16 up rows
            const int hcol = nt * (kBN / 2) + 16 * p + (w & 15);
            n = (w < 16) ? hcol : a.I + hcol;
        } else {
            n = nt * kBN + row;
            if (n >= a.Ncol) n = a.Ncol - 1;  // past the last column: a valid row, not stored
        }
        boff[u] = n * K + c * 8;
    }

    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    f4_t acc[4][kNB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < kNB; ++jj) acc[i][jj] = f4_t{0.f, 0.f, 0.f, 0.f};

    const u4_t z4 = {0u, 0u, 0u, 0u};
    u4_t ra[kChunksA], rb[kChunksB];
    gptr<uint16_t> xg = as_global(a.xin);
    gptr<uint16_t> wg = as_global(W);
    auto load = [&](int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int u = 0; u < kChunksA; ++u)
            ra[u] = (aoff[u] >= 0) ? *reinterpret_cast<gptr<u4_t>>(xg + aoff[u] + k0) : z4;
#pragma unroll
        for (int u = 0; u < kChunksB; ++u)
            rb[u] = __builtin_nontemporal_load(reinterpret_cast<gptr<u4_t>>(wg + boff[u] + k0));
    };
    auto store = [&]() {
#pragma unroll
        for (int u = 0; u < kChunksA; ++u) {
            const int q = tid + u * kThreads;
            *reinterpret_cast<u4_t*>(As + (q >> 3) * kLdsRow + (q & 7) * 8) = ra[u];
        }
#pragma unroll
        for (int u = 0; u < kChunksB; ++u) {
            const int q = tid + u * kThreads;
            *reinterpret_cast<u4_t*>(Bs + (q >> 3) * kLdsRow + (q & 7) * 8) = rb[u];
        }
    };

    const int nkt = K / kBK;
    load(0);
    store();
    __syncthreads();
    const int frow = lane & 15;
    const int fk = 8 * (lane >> 4);
    for (int kt = 0; kt < nkt; ++kt) {
        if (kt + 1 < nkt) load(kt + 1);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            h8_t af[4], bf[kNB];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const h8_t*>(As + (64 * wm + 16 * i + frow) * kLdsRow +
                                                       sub * 32 + fk);
#pragma unroll
            for (int jj = 0; jj < kNB; ++jj)
                bf[jj] = *reinterpret_cast<const h8_t*>(Bs + (kWN * wn + 16 * jj + frow) * kLdsRow +
                                                        sub * 32 + fk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < kNB; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[jj], acc[i][jj],
                                                                         0, 0, 0);
        }
        __syncthreads();  // every wave is done reading this step's tiles
        if (kt + 1 < nkt) {
            store();
            __syncthreads();
        }
    }

    // ---- epilogue: D[row 4*(lane/16) + i][col lane%16] of each block ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = m0 + 64 * wm + 16 * i + 4 * (lane >> 4) + t;
            if (r >= r1) continue;
            if (PHASE == 1) {
#pragma unroll
                for (int q = 0; q < kNB / 2; ++q) {
                    const int hcol = nt * (kBN / 2) + 16 * ((kNB / 2) * wn + q) + (lane & 15);
                    const float v = silu_f(acc[i][2 * q][t]) * acc[i][2 * q + 1][t];
                    a.out[(size_t)r * a.Ncol + hcol] = f2h(v);
                }
            } else {
#pragma unroll
                for (int jj = 0; jj < kNB; ++jj) {
                    const int col = nt * kBN + kWN * wn + 16 * jj + (lane & 15);
                    if (col < a.Ncol) a.out[(size_t)r * a.Ncol + col] = f2h(acc[i][jj][t]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Ring form of the same tile (launches averaging a full row tile per expert).  The operands reach LDS through
// direct global->LDS loads into a workgroup-wide ring of NS stages of 32 K
// each, so no registers stage them and NS - 1 stages are in flight while one
// is multiplied; each stage costs one counter wait and one barrier (the form
// above stores every step through registers between two barriers).  A load
// instruction fills 1 KB: 16 tile rows x 64 bytes, lane l taking row l/4 and
// the 16-byte chunk (l%4) xor ring_swz(row%16), so the MFMA-layout fragment reads
// (row l%16, chunk l/16) of 16 lanes hit 16 different bank groups.  The
// fragment reads are one asm block per stage (the compiler would otherwise
// wait for every outstanding global->LDS load before each LDS read).  The
// MFMAs run over K in the same 32-K order into the same accumulators as the
// form above, so the outputs are bit-identical.  Rows past the expert's group
// load its first row of the tile; their outputs are not stored.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kRK = 32;             // K per ring stage
constexpr int kRRowBytes = 2 * kRK;  // bytes of one tile row in a stage

template <int N>
__device__ __forceinline__ void ring_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Chunk slot xor of tile row r (mod 16): rows r and r' of one 16-row
// fragment read that share a bank group without it (same r mod 2 among 8
// lanes, or same r mod 4 among 16) get different xors, so the reads are
// conflict-free whether 8 or 16 lanes are served per pass.
__device__ __forceinline__ int ring_swz(int r) { return ((r >> 1) + (r >> 3)) & 3; }

// Wait until at most `ahead` later stages' loads (LOADS each) are in flight.
template <int NS, int LOADS>
__device__ __forceinline__ void ring_wait_ahead(int ahead) {
    if (NS >= 5 && ahead >= 3) ring_wait_vmcnt<(NS >= 5 ? 3 * LOADS : 0)>();
    else if (NS >= 4 && ahead == 2) ring_wait_vmcnt<(NS >= 4 ? 2 * LOADS : 0)>();
    else if (NS >= 3 && ahead == 1) ring_wait_vmcnt<LOADS>();
    else ring_wait_vmcnt<0>();
}

// The 4 A fragments (at a, 1 KB apart) and NB B fragments (at b, 1 KB apart)
// of one stage, completed before the block ends.
template <int NB>
__device__ __forceinline__ void ring_frags(uint32_t a, uint32_t b, h8_t (&af)[4], h8_t (&bf)[NB]) {
    static_assert(NB == 4 || NB == 8, "B fragments per stage");
    if constexpr (NB == 4) {
        asm volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %8 offset:1024\n\t"
            "ds_read_b128 %2, %8 offset:2048\n\t"
            "ds_read_b128 %3, %8 offset:3072\n\t"
            "ds_read_b128 %4, %9\n\t"
            "ds_read_b128 %5, %9 offset:1024\n\t"
            "ds_read_b128 %6, %9 offset:2048\n\t"
            "ds_read_b128 %7, %9 offset:3072\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(bf[0]), "=&v"(bf[1]),
              "=&v"(bf[2]), "=&v"(bf[3])
            : "v"(a), "v"(b)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %12\n\t"
            "ds_read_b128 %1, %12 offset:1024\n\t"
            "ds_read_b128 %2, %12 offset:2048\n\t"
            "ds_read_b128 %3, %12 offset:3072\n\t"
            "ds_read_b128 %4, %13\n\t"
            "ds_read_b128 %5, %13 offset:1024\n\t"
            "ds_read_b128 %6, %13 offset:2048\n\t"
            "ds_read_b128 %7, %13 offset:3072\n\t"
            "ds_read_b128 %8, %13 offset:4096\n\t"
            "ds_read_b128 %9, %13 offset:5120\n\t"
            "ds_read_b128 %10, %13 offset:6144\n\t"
            "ds_read_b128 %11, %13 offset:7168\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(bf[0]), "=&v"(bf[1]),
              "=&v"(bf[2]), "=&v"(bf[3]), "=&v"(bf[4]), "=&v"(bf[5]), "=&v"(bf[6]), "=&v"(bf[7])
            : "v"(a), "v"(b)
            : "memory");
    }
}

template <int PHASE, int BN, int NS>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(BN == 256 ? 2 : 3))) void dense_ring_kernel(DenseArgs a) {
    constexpr int kWN = BN / 2;               // columns per wave (2 x 2 waves)
    constexpr int kNB = kWN / 16;             // 16-column MFMA blocks per wave
    constexpr int kAL = kBM / 16 / 4;         // A load instructions per wave and stage
    constexpr int kBL = BN / 16 / 4;          // B load instructions per wave and stage
    constexpr int LOADS = kAL + kBL;
    constexpr int kAOff = 0, kBOff = kBM * kRRowBytes;
    constexpr int STAGE = (kBM + BN) * kRRowBytes;
    static_assert(NS >= 2 && NS <= 5, "ring stages");
    __shared__ __attribute__((aligned(1024))) char ring[NS][STAGE];

    // ---- which item (as dense_gemm_kernel) ----
    const int b = blockIdx.x;
    const int item = (b & 7) * (a.Wpad >> 3) + (b >> 3);
    const int nitems = a.plan[0];
    if (item >= nitems) return;
    const int nexp = a.plan[1];
    int lo = 0, hi = nexp - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.plan[2 + 4 * mid + 3] <= item) lo = mid;
        else hi = mid - 1;
    }
    const int32_t* pe = a.plan + 2 + 4 * lo;
    const int e = pe[0];
    const int rbase = pe[1];
    const int nmt = pe[2];
    const int j = item - pe[3];
    const int nt = j / nmt;
    const int mt = j - nt * nmt;
    const int m0 = rbase + mt * kBM;
    const int r1 = a.off[e + 1];
    const uint16_t* W = (PHASE == 1) ? a.experts[e].w13 : a.experts[e].w2;
    if (!W) {
        if (threadIdx.x == 0 && nt == 0 && mt == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
        return;
    }
    const int K = a.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // ---- loader: instruction u of this wave fills tile rows 16 * (row
    //      block) + lane/4 at chunk slot lane%4 with global chunk
    //      (lane%4) ^ ((lane/4)/4) ----
    const int lrow = lane >> 2;
    const int lchunk = (lane & 3) ^ ring_swz(lrow);
    const uint16_t* asrc[kAL];
    const uint16_t* bsrc[kBL];
#pragma unroll
    for (int u = 0; u < kAL; ++u) {
        const int row = 16 * (kAL * wave + u) + lrow;
        const int r = (m0 + row < r1) ? m0 + row : m0;
        const int src = (PHASE == 1) ? a.sorted_token[r] : r;
        asrc[u] = a.xin + (size_t)src * K + 8 * lchunk;
    }
#pragma unroll
    for (int u = 0; u < kBL; ++u) {
        const int row = 16 * (kBL * wave + u) + lrow;
        int n;
        if (PHASE == 1) {
            const int p = row >> 5, w = row & 31;  // pair p: 16 gate rows then 16 up rows
            const int hcol = nt * (BN / 2) + 16 * p + (w & 15);
            n = (w < 16) ? hcol : a.I + hcol;
        } else {
            n = nt * BN + row;
            if (n >= a.Ncol) n = a.Ncol - 1;  // past the last column: a valid row, not stored
        }
        bsrc[u] = W + (size_t)n * K + 8 * lchunk;
    }
    auto issue = [&](int st) {
        char* stage = &ring[st % NS][0];
        const int k0 = st * kRK;
#pragma unroll
        for (int u = 0; u < kAL; ++u)
            __builtin_amdgcn_global_load_lds((const void*)(asrc[u] + k0),
                                             (lds_ptr_t)(stage + kAOff + (kAL * wave + u) * 1024),
                                             16, 0, 0);
#pragma unroll
        for (int u = 0; u < kBL; ++u)
            __builtin_amdgcn_global_load_lds((const void*)(bsrc[u] + k0),
                                             (lds_ptr_t)(stage + kBOff + (kBL * wave + u) * 1024),
                                             16, 0, 0);
    };

    // ---- reader: fragment row lane%16, chunk lane/16 at its swizzled slot ----
    const int wm = wave & 1, wn = wave >> 1;
    const uint32_t lane_off =
        (uint32_t)((lane & 15) * kRRowBytes + (((lane >> 4) ^ ring_swz(lane & 15)) << 4));
    const uint32_t a_rel = kAOff + (uint32_t)(64 * wm) * kRRowBytes + lane_off;
    const uint32_t b_rel = kBOff + (uint32_t)(kWN * wn) * kRRowBytes + lane_off;

    f4_t acc[4][kNB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < kNB; ++jj) acc[i][jj] = f4_t{0.f, 0.f, 0.f, 0.f};

    const int nst = K / kRK;
#pragma unroll
    for (int d = 0; d < NS - 1; ++d)
        if (d < nst) issue(d);
    for (int st = 0; st < nst; ++st) {
        // this wave's loads of stage st: loads of min(NS - 2, nst - 1 - st)
        // later stages may still be in flight
        ring_wait_ahead<NS, LOADS>(min(NS - 2, nst - 1 - st));
        // every wave's loads of stage st have landed and every wave has read
        // stage st - 1, whose slot the next issue refills
        __builtin_amdgcn_s_barrier();
        if (st + NS - 1 < nst) issue(st + NS - 1);
        const uint32_t base = (uint32_t)(uintptr_t)(lds_ptr_t)&ring[st % NS][0];
        h8_t af[4], bf[kNB];
        ring_frags<kNB>(base + a_rel, base + b_rel, af, bf);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < kNB; ++jj)
                acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[jj], acc[i][jj], 0, 0, 0);
    }

    // ---- epilogue (as dense_gemm_kernel) ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = m0 + 64 * wm + 16 * i + 4 * (lane >> 4) + t;
            if (r >= r1) continue;
            if (PHASE == 1) {
#pragma unroll
                for (int q = 0; q < kNB / 2; ++q) {
                    const int hcol = nt * (BN / 2) + 16 * ((kNB / 2) * wn + q) + (lane & 15);
                    const float v = silu_f(acc[i][2 * q][t]) * acc[i][2 * q + 1][t];
                    a.out[(size_t)r * a.Ncol + hcol] = f2h(v);
                }
            } else {
#pragma unroll
                for (int jj = 0; jj < kNB; ++jj) {
                    const int col = nt * BN + kWN * wn + 16 * jj + (lane & 15);
                    if (col < a.Ncol) a.out[(size_t)r * a.Ncol + col] = f2h(acc[i][jj][t]);
                }
            }
        }
    }
}

}  // namespace

namespace smoe {
// Tile widths: the gate/up projection (2I weight rows, many column blocks)
// takes 256-column tiles; the down projection (H columns, a few hundred work
// items at the Phi-3.5-MoE shape) keeps 128, whose twice as many items fill
// the CUs better (measured 460 vs 507 us at T = 2048).
constexpr int kBN1 = 256, kBN2 = 128;
size_t dense_plan_bytes(int E) { return (size_t)2 * (2 + 4 * E) * 4; }  // both projections

hipError_t launch_dense_ffn(const uint16_t* x, const int32_t* sorted_token, const int32_t* off,
                            const int32_t* active, const int32_t* n_active,
                            const smoe_f16_expert* experts, const uint8_t* mask, int rows, int H,
                            int I, int E, uint16_t* y, uint16_t* h, int32_t* plan, int32_t* err,
                            hipStream_t s) {
    const int slots = active ? (E < rows ? E : rows) : E;
    const int mt_bound = (rows + kBM - 1) / kBM + slots;  // row tiles of all experts, at most
    // The ring form where the touched experts average at least a full row
    // tile (measured at T = 2048 on the Phi-3.5-MoE shape, 256 rows per
    // expert: 1394 -> 1294 us per call); with fewer rows per expert (the
    // DeepSeek-V2-Lite shape at T = 700, about 66) the register-staged form's
    // 128-byte row runs stream the weights better (350 against 366 us).  The
    // ring's down projection takes 256-column tiles when H has no partial
    // one (half the work items, one round of two per CU at the Phi shape:
    // 1299 -> 1264 us; H = 384 keeps 128: 37 against 41 us).  Every choice
    // gives the same bits.
    const bool ring = rows >= kBM * slots;
    const int bn2 = (ring && H % 256 == 0) ? 256 : kBN2;
    DenseArgs a1{};
    a1.xin = x;
    a1.sorted_token = sorted_token;
    a1.off = off;
    a1.experts = experts;
    a1.plan = plan;
    a1.K = H;
    a1.Ncol = I;
    a1.I = I;
    a1.nNT = I / (kBN1 / 2);
    a1.Wpad = ((mt_bound * a1.nNT) + 7) & ~7;
    a1.out = h;
    a1.err = err;
    DenseArgs a2 = a1;
    a2.xin = h;
    a2.sorted_token = nullptr;
    a2.K = I;
    a2.Ncol = H;
    a2.nNT = (H + bn2 - 1) / bn2;
    a2.Wpad = ((mt_bound * a2.nNT) + 7) & ~7;
    a2.out = y;
    // the two projections list the same experts; each plan holds its own item bases
    int32_t* plan2 = plan + 2 + 4 * E;
    a2.plan = plan2;
    dense_plan_kernel<<<1, 64, 0, s>>>(off, active, n_active, mask, E, a1.nNT, plan);
    dense_plan_kernel<<<1, 64, 0, s>>>(off, active, n_active, mask, E, a2.nNT, plan2);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
    if (ring) {
        dense_ring_kernel<1, kBN1, SMOE_DENSE_STAGES><<<a1.Wpad, kThreads, 0, s>>>(a1);
        st = hipGetLastError();
        if (st != hipSuccess) return st;
        if (bn2 == 256)
            dense_ring_kernel<2, 256, SMOE_DENSE_STAGES><<<a2.Wpad, kThreads, 0, s>>>(a2);
        else
            dense_ring_kernel<2, kBN2, SMOE_DENSE_STAGES><<<a2.Wpad, kThreads, 0, s>>>(a2);
        return hipGetLastError();
    }
    dense_gemm_kernel<1, kBN1><<<a1.Wpad, kThreads, 0, s>>>(a1);
    st = hipGetLastError();
    if (st != hipSuccess) return st;
    dense_gemm_kernel<2, kBN2><<<a2.Wpad, kThreads, 0, s>>>(a2);
    return hipGetLastError();
}
}  // namespace smoe
