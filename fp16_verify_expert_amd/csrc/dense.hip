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
// row for the missing columns and does not store them.
#include "common.h"

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
    a2.nNT = (H + kBN2 - 1) / kBN2;
    a2.Wpad = ((mt_bound * a2.nNT) + 7) & ~7;
    a2.out = y;
    // the two projections list the same experts; each plan holds its own item bases
    int32_t* plan2 = plan + 2 + 4 * E;
    a2.plan = plan2;
    dense_plan_kernel<<<1, 64, 0, s>>>(off, active, n_active, mask, E, a1.nNT, plan);
    dense_plan_kernel<<<1, 64, 0, s>>>(off, active, n_active, mask, E, a2.nNT, plan2);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
    dense_gemm_kernel<1, kBN1><<<a1.Wpad, kThreads, 0, s>>>(a1);
    st = hipGetLastError();
    if (st != hipSuccess) return st;
    dense_gemm_kernel<2, kBN2><<<a2.Wpad, kThreads, 0, s>>>(a2);
    return hipGetLastError();
}
}  // namespace smoe
