// FP16 verification FFN over rows grouped by expert, on MFMA.
//
// Cited: "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step
// Speculative Offloading" (AI summary), Key Contributions 3-4 and Methodology
// in Plain English.  In verification each touched expert is evaluated once
// over all of its rows, a matrix product per expert in place of a
// matrix-vector product per (token, expert), with values equal to the
// per-token evaluation.  The optional expert mask lets the caller run the
// experts whose weights are already on the device while other experts'
// weights are still being copied in.
//
// A workgroup owns 16 output columns of one touched expert; its waves split
// the reduction and stream the weight rows of those columns, feeding
// v_mfma_f32_16x16x32_f16 directly from registers: lane l loads 16 bytes of
// weight row (n0 + l%16) at K offset 8*(l/16) -- exactly the B-operand layout
// -- and the matching activation row (l%16) of the expert's packed rows as the
// A operand.  Small work units keep the tail of the launch short.  Rows
// beyond the expert's count are zero, so the MFMA is only as wide as the data; at K+1 <= 33 tokens the kernel is bound by the HBM stream
// of the touched experts' weights.  Up to RB row blocks of 16 share one weight
// stream.  The gate/up projection applies SwiGLU in registers and writes h as
// fp16; the down projection writes y_sorted.
#include "common.h"
#include "gemv_core.h"

namespace {

constexpr int kTileBytes = 4096; // one 16-row x 128-K fp16 tile
constexpr int kKStep = 128;      // K per pipeline step

struct F16Args {
    const uint16_t* xin;          // phase 1: x [T, H]; phase 2: h [rows, I]
    const int32_t* sorted_token;  // phase 1
    const int32_t* off;
    const int32_t* active;        // nullable
    const int32_t* n_active;      // nullable
    const smoe_f16_expert* experts;
    const uint8_t* mask;          // nullable
    int K;      // H or I
    int Ncol;   // output columns: I (phase 1) or H (phase 2)
    int I;
    int H;
    int nCB;    // column blocks: 16 columns, kGemvWaves in the matrix-vector kernel
    uint16_t* out;  // phase 1: h [rows, I]; phase 2: y [rows, H]
    int32_t* err;
    // an always-on dense group (the shared expert) as the launch's first
    // ex_nCB work items, over token rows 0..ex_T-1: null ex_w = none
    const uint16_t* ex_w;   // phase 1: w13 [2 ex_I, H]; phase 2: w2 [H, ex_I]
    const uint16_t* ex_in;  // phase 2: its h [ex_T, ex_I]
    uint16_t* ex_out;       // phase 1: its h; phase 2: its output [ex_T, H]
    int ex_I, ex_nCB, ex_T;
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
}

// ---------------------------------------------------------------------------
// Register-pipelined variant (short reductions).  Same work unit: one
// workgroup per (expert, 16-column block), 4 waves splitting the reduction;
// weights and activations of step st+1 are loaded into registers straight in
// the MFMA operand layout (lane l: row l%16, 16 bytes at K offset 8*(l/16))
// while step st is multiplied.  No LDS ring, so several workgroups share a
// CU and their start-up latencies overlap; for long reductions the wide-run
// LDS variant below streams HBM better.
constexpr int kRegWaves = 4;

template <int PHASE, int RB>
__global__ __launch_bounds__(64 * kRegWaves) void f16_reg_kernel(F16Args a) {
    constexpr int NACC = (PHASE == 1) ? 2 : 1;
    constexpr int kUnroll = (PHASE == 1) ? 4 : 8;  // 32-K chunks per step
    __shared__ f4_t part[kRegWaves][NACC][RB][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int cb = blockIdx.x % a.nCB;
    const int slot = blockIdx.x / a.nCB;
    int e;
    if (a.active) {
        e = a.active[slot];  // -1 past the touched experts
        if (e < 0) return;
    } else {
        e = slot;
    }
    if (a.mask && !a.mask[e]) return;
    const int r0 = a.off[e];
    const int r1 = a.off[e + 1];
    if (r1 <= r0) return;
    const uint16_t* W = (PHASE == 1) ? a.experts[e].w13 : a.experts[e].w2;
    if (!W) {
        if (threadIdx.x == 0 && cb == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
        return;
    }
    const int K = a.K;
    const int n = cb * 16 + (lane & 15);
    const int kq = 8 * (lane >> 4);
    const h8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    // this wave's steps (32*kUnroll K each; the matrix's last step may be partial)
    const int nchunks = K / 32;
    const int nsteps = (nchunks + kUnroll - 1) / kUnroll;
    const int s0 = (nsteps * wave) / kRegWaves;
    const int s1 = (nsteps * (wave + 1)) / kRegWaves;

    gptr<h8_t> wg = as_global(reinterpret_cast<const h8_t*>(W + (size_t)n * K + kq));
    gptr<h8_t> wu = as_global(reinterpret_cast<const h8_t*>(
        W + (size_t)((PHASE == 1) ? a.I + n : n) * K + kq));

    for (int mb = r0; mb < r1; mb += 16 * RB) {
        gptr<h8_t> arow[RB];
        bool aok[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const int r = mb + 16 * b + (lane & 15);
            aok[b] = r < r1;
            const uint16_t* src;
            if (PHASE == 1)
                src = a.xin + (size_t)(aok[b] ? a.sorted_token[r] : 0) * K;
            else
                src = a.xin + (size_t)(aok[b] ? r : 0) * K;
            arow[b] = as_global(reinterpret_cast<const h8_t*>(src + kq));
        }
        f4_t accg[RB], accu[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            accg[b] = f4_t{0.f, 0.f, 0.f, 0.f};
            accu[b] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
        h8_t bg[kUnroll], bu[kUnroll], av[RB][kUnroll];
        if (s0 < s1) {
            const size_t o = (size_t)s0 * 4 * kUnroll;  // in h8 units
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const bool in = s0 * kUnroll + u < nchunks;
                bg[u] = in ? __builtin_nontemporal_load(wg + o + 4 * u) : zero8;
                if (PHASE == 1) bu[u] = in ? __builtin_nontemporal_load(wu + o + 4 * u) : zero8;
#pragma unroll
                for (int b = 0; b < RB; ++b) av[b][u] = (in && aok[b]) ? arow[b][o + 4 * u] : zero8;
            }
        }
        for (int st = s0; st < s1; ++st) {
            const size_t o = (size_t)(st + 1) * 4 * kUnroll;
            h8_t nbg[kUnroll], nbu[kUnroll], nav[RB][kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const bool in = st + 1 < s1 && (st + 1) * kUnroll + u < nchunks;
                nbg[u] = in ? __builtin_nontemporal_load(wg + o + 4 * u) : zero8;
                if (PHASE == 1) nbu[u] = in ? __builtin_nontemporal_load(wu + o + 4 * u) : zero8;
#pragma unroll
                for (int b = 0; b < RB; ++b) nav[b][u] = (in && aok[b]) ? arow[b][o + 4 * u] : zero8;
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    accg[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[b][u], bg[u], accg[b], 0, 0, 0);
                    if (PHASE == 1)
                        accu[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[b][u], bu[u], accu[b], 0, 0, 0);
                }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                bg[u] = nbg[u];
                if (PHASE == 1) bu[u] = nbu[u];
#pragma unroll
                for (int b = 0; b < RB; ++b) av[b][u] = nav[b][u];
            }
        }
        // ---- add the waves' partial tiles (fixed order) ----
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            part[wave][0][b][lane] = accg[b];
            if (PHASE == 1) part[wave][NACC - 1][b][lane] = accu[b];
        }
        __syncthreads();
        for (int b = wave; b < RB; b += kRegWaves) {
            f4_t g = part[0][0][b][lane];
            f4_t u = part[0][NACC - 1][b][lane];
            for (int w = 1; w < kRegWaves; ++w) {
                g += part[w][0][b][lane];
                if (PHASE == 1) u += part[w][NACC - 1][b][lane];
            }
            // D[row = 4*(lane/16) + i][col = lane%16]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = mb + 16 * b + 4 * (lane >> 4) + i;
                if (r < r1) {
                    const float v = (PHASE == 1) ? silu_f(g[i]) * u[i] : g[i];
                    a.out[(size_t)r * a.Ncol + n] = f2h(v);
                }
            }
        }
        __syncthreads();  // part is reused by the next row block
    }
}

// ---------------------------------------------------------------------------
// LDS-ring variant (long reductions).
// NT 16-byte LDS reads at byte addresses addr + t*4096, completed before the
// block ends.  Written as one asm block so the compiler's counter analysis
// (which cannot tell the ring stages apart and would otherwise drain every
// outstanding global->LDS load before any LDS read) leaves the explicit
// vmcnt waits of the pipeline in charge.
template <int NT>
__device__ __forceinline__ void lds_read_tiles(uint32_t addr, h8_t (&v)[NT]) {
    static_assert(NT >= 2 && NT <= 4, "tiles per step");
    if constexpr (NT == 2) {
        asm volatile(
            "ds_read_b128 %0, %2\n\t"
            "ds_read_b128 %1, %2 offset:4096\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1])
            : "v"(addr)
            : "memory");
    } else if constexpr (NT == 3) {
        asm volatile(
            "ds_read_b128 %0, %3\n\t"
            "ds_read_b128 %1, %3 offset:4096\n\t"
            "ds_read_b128 %2, %3 offset:8192\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2])
            : "v"(addr)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %4\n\t"
            "ds_read_b128 %1, %4 offset:4096\n\t"
            "ds_read_b128 %2, %4 offset:8192\n\t"
            "ds_read_b128 %3, %4 offset:12288\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
            : "v"(addr)
            : "memory");
    }
}

// NM weight-tile fragments at addr (+4096) and one activation-tile fragment
// at aaddr, completed before the block ends (as lds_read_tiles).
template <int NM>
__device__ __forceinline__ void lds_read_tiles_light(uint32_t addr, uint32_t aaddr,
                                                     h8_t (&v)[NM + 1]) {
    static_assert(NM == 1 || NM == 2, "weight tiles per step");
    if constexpr (NM == 1) {
        asm volatile(
            "ds_read_b128 %0, %2\n\t"
            "ds_read_b128 %1, %3\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1])
            : "v"(addr), "v"(aaddr)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %3\n\t"
            "ds_read_b128 %1, %3 offset:4096\n\t"
            "ds_read_b128 %2, %4\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2])
            : "v"(addr), "v"(aaddr)
            : "memory");
    }
}

template <int N>
struct IntC {
    static constexpr int value = N;
};

// One workgroup = one (expert, 16-column block); its waves split the
// reduction into contiguous step ranges.  Each wave streams its tiles through
// a private NSTAGE-deep LDS ring with direct global->LDS loads: a load
// instruction covers 4 rows x 256 contiguous bytes (lane l: row 4j + l/16,
// 16-byte chunk (l%16) xor row), which is what keeps HBM streaming near its
// peak; the xor swizzle makes the MFMA-layout reads (row l%16, chunk
// 4u + l/16) hit 16 different bank groups.  The activation rows of the step
// come through the same ring, so one counter wait covers a whole step.
template <int PHASE, int RB, int NSTAGE, int kVWaves>
__global__ __launch_bounds__(64 * kVWaves) void f16_kernel(F16Args a) {
    constexpr int NM = (PHASE == 1) ? 2 : 1;            // weight matrices per step
    constexpr int NT = NM + RB;                          // tiles per step
    constexpr int STAGE = NT * kTileBytes;
    constexpr int D = NSTAGE - 1;                        // steps in flight ahead
    __shared__ __attribute__((aligned(16))) char ring[kVWaves][NSTAGE][STAGE];
    __shared__ f4_t part[kVWaves][NM][RB][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // the dense group's items first, then the routed (expert, block) items
    const int exn = a.ex_w ? a.ex_nCB : 0;
    const bool ex = (int)blockIdx.x < exn;
    const int item = ex ? (int)blockIdx.x : (int)blockIdx.x - exn;
    int cb, r0, r1;
    const uint16_t* W;
    if (ex) {
        cb = item;
        r0 = 0;
        r1 = a.ex_T;
        W = a.ex_w;
    } else {
        cb = item % a.nCB;
        const int slot = item / a.nCB;
        int e;
        if (a.active) {
            e = a.active[slot];  // -1 past the touched experts
            if (e < 0) return;
        } else {
            e = slot;
        }
        if (a.mask && !a.mask[e]) return;
        r0 = a.off[e];
        r1 = a.off[e + 1];
        if (r1 <= r0) return;
        W = (PHASE == 1) ? a.experts[e].w13 : a.experts[e].w2;
        if (!W) {
            if (threadIdx.x == 0 && cb == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
            return;
        }
    }
    const int K = (ex && PHASE == 2) ? a.ex_I : a.K;
    const int Iup = ex ? a.ex_I : a.I;                  // up rows of w13 start here
    const int Ncol = (ex && PHASE == 1) ? a.ex_I : a.Ncol;
    const uint16_t* xin = (ex && PHASE == 2) ? a.ex_in : a.xin;
    const int32_t* tok = ex ? nullptr : a.sorted_token;
    uint16_t* out = ex ? a.ex_out : a.out;
    const int nsteps = K / kKStep;
    const int s0 = (nsteps * wave) / kVWaves;
    const int s1 = (nsteps * (wave + 1)) / kVWaves;
    const int n0 = cb * 16;

    // loader geometry: instruction j covers tile rows 4j + lane/16
    const int lrow = lane >> 4;          // + 4j
    const int lslot = lane & 15;
    // reader geometry: row lane%16, chunk 4u + lane/16 at slot chunk ^ row
    const int rrow = lane & 15;
    const int rq = lane >> 4;

    // global source row pointers of this lane (4 tile rows per matrix)
    const uint16_t* wrow[NM][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * j + lrow;
        wrow[0][j] = W + (size_t)(n0 + r) * K;
        if (PHASE == 1) wrow[NM - 1][j] = W + (size_t)(Iup + n0 + r) * K;
    }

    // One row block; AQ = activation load instructions per tile and step (4
    // rows each).  A block of at most 4 rows (the usual case at K+1 <= 33:
    // about 2.3 rows per touched expert) takes AQ = 1: its rows land in the
    // tile's first 1 KB, and the A operand repeats them in rows 4-15, whose
    // outputs are not stored (measured 2% faster on the Phi-shaped verify
    // than loading all 16 rows).
    auto row_block = [&](int mb, auto aq) {
        constexpr int AQ = decltype(aq)::value;
        constexpr int LOADS = 4 * NM + AQ * RB;  // load instructions per step
        // activation rows of this lane's loads (rows past the group repeat a
        // valid row; they only feed output rows that are not stored)
        const uint16_t* arow[RB][4];
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int r = mb + 16 * b + 4 * j + lrow;
                if (r >= r1) r = r0;
                arow[b][j] = (PHASE == 1) ? xin + (size_t)(tok ? tok[r] : r) * K
                                          : xin + (size_t)r * K;
            }
        auto issue = [&](int st) {
            char* stage = &ring[wave][st % NSTAGE][0];
            const int k0 = st * kKStep;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = lslot ^ (4 * j + lrow);  // swizzled 16-byte chunk
                const int koff = k0 + 8 * c;
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    __builtin_amdgcn_global_load_lds(
                        (const void*)(wrow[m][j] + koff),
                        (lds_ptr_t)(stage + m * kTileBytes + j * 1024), 16, 0, 0);
#pragma unroll
                for (int b = 0; b < RB; ++b)
                    if (j < AQ)
                        __builtin_amdgcn_global_load_lds(
                            (const void*)(arow[b][j] + koff),
                            (lds_ptr_t)(stage + (NM + b) * kTileBytes + j * 1024), 16, 0, 0);
            }
        };

        f4_t accg[RB], accu[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            accg[b] = f4_t{0.f, 0.f, 0.f, 0.f};
            accu[b] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
        wait_lgkm0();  // the ring of the previous row block has been read
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (s0 + d < s1) issue(s0 + d);
        for (int st = s0; st < s1; ++st) {
            wait_lgkm0();  // reads of the stage about to be refilled are done
            if (st + D < s1) issue(st + D);
            // loads issued after step st's: min(D, s1-1-st) steps
            const int ahead = min(D, s1 - 1 - st);
            if (ahead >= D) wait_vmcnt<D * LOADS>();
            else if (D >= 2 && ahead == 1) wait_vmcnt<LOADS>();
            else if (D >= 3 && ahead == 2) wait_vmcnt<(D >= 3 ? 2 * LOADS : 0)>();
            else wait_vmcnt<0>();
            const uint32_t stage_addr =
                (uint32_t)(uintptr_t)(lds_ptr_t)&ring[wave][st % NSTAGE][0];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t off = rrow * 256 + (((4 * u + rq) ^ rrow) << 4);
                h8_t t[NT];  // weight tile(s), then RB activation tiles
                if constexpr (AQ == 4) {
                    lds_read_tiles<NT>(stage_addr + off, t);
                } else {
                    static_assert(RB == 1, "short row blocks hold one tile of rows");
                    const int ar = rrow & 3;  // the block's rows 0-3, repeated
                    const uint32_t aoff = NM * kTileBytes + ar * 256 + (((4 * u + rq) ^ ar) << 4);
                    lds_read_tiles_light<NM>(stage_addr + off, stage_addr + aoff,
                                             *reinterpret_cast<h8_t(*)[NM + 1]>(&t[0]));
                }
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    accg[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(t[NM + b], t[0], accg[b], 0, 0, 0);
                    if (PHASE == 1)
                        accu[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(t[NM + b], t[1], accu[b], 0, 0, 0);
                }
            }
        }
        // ---- add the waves' partial tiles (fixed order) ----
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            part[wave][0][b][lane] = accg[b];
            if (PHASE == 1) part[wave][NM - 1][b][lane] = accu[b];
        }
        __syncthreads();
        for (int b = wave; b < RB; b += kVWaves) {
            f4_t g = part[0][0][b][lane];
            f4_t u = part[0][NM - 1][b][lane];
            for (int w = 1; w < kVWaves; ++w) {
                g += part[w][0][b][lane];
                if (PHASE == 1) u += part[w][NM - 1][b][lane];
            }
            // D[row = 4*(lane/16) + i][col = lane%16]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = mb + 16 * b + 4 * (lane >> 4) + i;
                if (r < r1) {
                    const float v = (PHASE == 1) ? silu_f(g[i]) * u[i] : g[i];
                    out[(size_t)r * Ncol + n0 + (lane & 15)] = f2h(v);
                }
            }
        }
        __syncthreads();  // part is reused by the next row block
    };
    for (int mb = r0; mb < r1; mb += 16 * RB) {
        if constexpr (RB == 1) {
            if (r1 - mb <= 4) {
                row_block(mb, IntC<1>{});
                continue;
            }
        }
        row_block(mb, IntC<4>{});
    }
}

// ---------------------------------------------------------------------------
// Matrix-vector variant (a few rows per expert: the shared expert of a
// one-token draft step, any call with T <= kGemvMaxT).  With one row the
// MFMA tiles would idle 15 of their 16 rows and the 16-column work units
// leave most of the weight stream waiting on short per-wave pipelines; here
// every weight byte of the launch is requested at once instead.  One wave
// per output column: lane l holds the 16-byte chunks l, l + 64, ... of the
// column's weight row (and of its up row in the gate/up projection), so each
// load is 1 KB of one row, and the same chunks of the expert's rows, one row
// at a time (the weights stay in registers for the next row).  Each lane
// dots its chunks (v_dot2_f32_f16, fp32 sums in chunk order) and the wave's
// 64 lane sums are added in a fixed order (the routines of gemv_core.h, also
// used by the one-token draft launches for a dense shared expert).  Measured
// against staging RB rows in LDS per workgroup: one row at a time is faster
// up to four rows (the LDS staging waits for every load of the launch first).
constexpr int kGemvWaves = 4;      // columns per workgroup
constexpr int kGemvMaxT = 4;       // tokens per call at or below which it runs
constexpr int kGemvMaxChunks = smoe_gemv::kMaxChunks; // 16-byte chunks per lane and row

template <int PHASE, int CPL>
__global__ __launch_bounds__(64 * kGemvWaves) void f16_gemv_kernel(F16Args a) {
    constexpr int NM = (PHASE == 1) ? 2 : 1;  // weight rows per column
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cb = blockIdx.x % a.nCB;
    const int slot = blockIdx.x / a.nCB;
    int e;
    if (a.active) {
        e = a.active[slot];  // -1 past the touched experts
        if (e < 0) return;
    } else {
        e = slot;
    }
    if (a.mask && !a.mask[e]) return;
    const int r0 = a.off[e];
    const int r1 = a.off[e + 1];
    if (r1 <= r0) return;
    const uint16_t* W = (PHASE == 1) ? a.experts[e].w13 : a.experts[e].w2;
    if (!W) {
        if (tid == 0 && cb == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
        return;
    }
    const int K = a.K;
    const int n = cb * kGemvWaves + wave;
    const int nc = (n < a.Ncol) ? n : a.Ncol - 1;  // clamped column: loads stay in the matrix
    auto xrow = [&](int r) {
        const size_t src = (PHASE == 1) ? (size_t)a.sorted_token[r] : (size_t)r;
        return a.xin + src * K;
    };
    // the column's weight chunks, all of them, then the first row
    u4_t wv[NM][CPL];
    smoe_gemv::gemv_load_w<NM, CPL>(W, K, a.I, nc, lane, wv);
    uint4 xr[CPL];
    smoe_gemv::gemv_load_x<CPL>(xrow(r0), K, lane, xr);
    // keep every load above ahead of the first use (the scheduler would
    // otherwise start on the first chunks and issue the last ones a round
    // trip later)
    __builtin_amdgcn_sched_barrier(0);

    auto one_row = [&](int r) {
        const uint16_t v = smoe_gemv::gemv_dot<NM, CPL>(wv, xr, K, lane);
        if (lane == 0 && n < a.Ncol) a.out[(size_t)r * a.Ncol + n] = v;
    };
    // the first row straight-line (its waits then cover only what each step
    // needs), further rows of the group in a loop
    one_row(r0);
    for (int r = r0 + 1; r < r1; ++r) {
        smoe_gemv::gemv_load_x<CPL>(xrow(r), K, lane, xr);
        one_row(r);
    }
}

template <int PHASE, int CPL>
hipError_t launch_gemv_cpl(const F16Args& a, int slots, hipStream_t s) {
    hipLaunchKernelGGL((f16_gemv_kernel<PHASE, CPL>), dim3(slots * a.nCB),
                       dim3(64 * kGemvWaves), 0, s, a);
    return hipGetLastError();
}

// a.nCB must be ceil(Ncol / kGemvWaves) and K at most 512 * kGemvMaxChunks.
template <int PHASE>
hipError_t launch_gemv_phase(const F16Args& a, int slots, hipStream_t s) {
    const int need = (a.K / 8 + 63) / 64;  // chunks per lane and row
    if (need <= 2) return launch_gemv_cpl<PHASE, 2>(a, slots, s);
    if (need <= 4) return launch_gemv_cpl<PHASE, 4>(a, slots, s);
    if (need <= 6) return launch_gemv_cpl<PHASE, 6>(a, slots, s);
    if (need <= 8) return launch_gemv_cpl<PHASE, 8>(a, slots, s);
    if (need <= 12) return launch_gemv_cpl<PHASE, 12>(a, slots, s);
    return launch_gemv_cpl<PHASE, kGemvMaxChunks>(a, slots, s);
}

#ifndef SMOE_DENSE_MIN_ROWS
#define SMOE_DENSE_MIN_ROWS 64  // mean rows per expert from which the tiled GEMM is used
#endif
#ifndef SMOE_VF_GEMV
#define SMOE_VF_GEMV 1  // the one-wave-per-column kernel for T <= kGemvMaxT
#endif
#ifndef SMOE_VF_LONG
// 128-K steps per wave from which the LDS-ring kernel runs.  Measured on the
// Qwen1.5-MoE shapes: at 4 steps (hidden 2048) the ring kernel streams the
// shared expert (intermediate 5632, a few hundred workgroups) 20-27% faster
// and the routed experts as fast; at 2-3 steps (the routed down projection,
// intermediate 1408) the register kernel is 7% faster.
#define SMOE_VF_LONG 4
#endif

// One always-on group (a shared expert): waves per workgroup and ring depth
// of each projection (gate/up, down).  Measured on the Qwen1.5-MoE shared
// expert (intermediate 5632, 352 gate/up and 128 down workgroups; kernel
// trace, weights from HBM): gate/up with 2 waves and 2 stages (48 KB of LDS,
// three workgroups per CU, so all 352 start in one round) 12.3 us against
// 15.2 us with 4 waves and 3 stages (144 KB: one per CU, a second round of
// 96); the down projection stays at 4 waves and 3 stages (2, 6 or 8 waves,
// 2 or 3 stages: no better).
// (SMOE_SH_GU_WAVES and SMOE_SH_DN_WAVES live in common.h: the multi-row
// draft launches compute the same items with the same wave split.)
#ifndef SMOE_SH_GU_STAGES
#define SMOE_SH_GU_STAGES 2
#endif
#ifndef SMOE_SH_DN_STAGES
#define SMOE_SH_DN_STAGES 3
#endif

template <int PHASE, int W, int S>
hipError_t launch_ring(const F16Args& a, int slots, int RB, hipStream_t s) {
    const dim3 grid(slots * a.nCB + (a.ex_w ? a.ex_nCB : 0));
    if (RB == 1) {
        hipLaunchKernelGGL((f16_kernel<PHASE, 1, S, W>), grid, dim3(64 * W), 0, s, a);
    } else {
        // two row blocks: two stages, and at most the waves whose rings fit
        // in LDS (4 x 2 x 16 KB for gate/up, 6 x 2 x 12 KB for down)
        constexpr int W2 = (PHASE == 1) ? (W > 4 ? 4 : W) : (W > 6 ? 6 : W);
        hipLaunchKernelGGL((f16_kernel<PHASE, 2, 2, W2>), grid, dim3(64 * W2), 0, s, a);
    }
    return hipGetLastError();
}

// Which kernel launch_phase runs for the routed items: 0 the register
// kernel, 1 the 2-wave ring, 2 the 4-wave ring, 3 the one-group ring.
int phase_kernel(const F16Args& a, int slots) {
    if (slots == 1 && a.K / kKStep >= 8) return 3;
    const int nsteps = a.K / kKStep;
    const long long wgs = (long long)slots * a.nCB;
    if (nsteps / 2 >= SMOE_VF_LONG && (nsteps < 16 || (nsteps == 16 && wgs > 1024))) return 1;
    return (nsteps / 4 >= SMOE_VF_LONG) ? 2 : 0;
}

template <int PHASE>
hipError_t launch_phase(const F16Args& a, int slots, int RB, hipStream_t s) {
    const int exn = a.ex_w ? a.ex_nCB : 0;  // ring kernels only (see launch_verify_ffn_shared)
    if (slots == 1 && a.K / kKStep >= 8) {
        if constexpr (PHASE == 1)
            return launch_ring<PHASE, SMOE_SH_GU_WAVES, SMOE_SH_GU_STAGES>(a, slots, RB, s);
        else
            return launch_ring<PHASE, SMOE_SH_DN_WAVES, SMOE_SH_DN_STAGES>(a, slots, RB, s);
    }
    // Reductions with at least SMOE_VF_LONG 128-K steps per wave take the
    // LDS-ring kernel (4 waves; LDS per workgroup: 4 x NSTAGE x (NM + RB) x
    // 4 KB <= 160 KB), shorter ones the register-pipelined kernel.  Reductions
    // of 8-16 steps run the ring kernel with 2 waves instead (half the LDS, so
    // two or three workgroups share a CU), 16 steps only over more than 1024
    // work units.  Measured on the Qwen1.5-MoE shapes: the routed down
    // projection (K = 1408) 3-4% faster than the register kernel, the routed
    // gate/up projection (K = 2048) 5-7% faster than 4 waves; with 4 waves
    // the Phi-shaped reductions (32 and 50 steps) stay 7% faster and the
    // shared expert (352 workgroups) 6% faster.
    const int nsteps = a.K / kKStep;
    const bool ring = nsteps / 4 >= SMOE_VF_LONG;
    const long long wgs = (long long)slots * a.nCB;
    const bool two = nsteps / 2 >= SMOE_VF_LONG && (nsteps < 16 || (nsteps == 16 && wgs > 1024));
    if (two) {
        const dim3 grid2(slots * a.nCB + exn), block2(128);
        if (RB == 1)
            hipLaunchKernelGGL((f16_kernel<PHASE, 1, 3, 2>), grid2, block2, 0, s, a);
        else
            hipLaunchKernelGGL((f16_kernel<PHASE, 2, 2, 2>), grid2, block2, 0, s, a);
        return hipGetLastError();
    }
    const dim3 grid(slots * a.nCB + (ring ? exn : 0)), block(256);
    if (ring) {
        if (RB == 1)
            hipLaunchKernelGGL((f16_kernel<PHASE, 1, 3, 4>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((f16_kernel<PHASE, 2, 2, 4>), grid, block, 0, s, a);
    } else {
        if (RB == 1)
            hipLaunchKernelGGL((f16_reg_kernel<PHASE, 1>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((f16_reg_kernel<PHASE, 2>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

namespace smoe {
// h [rows, I] fp16, then the dense regime's plan
size_t verify_workspace_bytes(int /*T*/, int rows, int /*H*/, int I, int E) {
    const size_t hb = (((size_t)rows * I * 2) + 255) & ~(size_t)255;
    return hb + ((dense_plan_bytes(E) + 255) & ~(size_t)255);
}

hipError_t launch_verify_ffn(const uint16_t* x, const int32_t* sorted_token, const int32_t* off,
                             const int32_t* active, const int32_t* n_active,
                             const smoe_f16_expert* experts, const uint8_t* mask, int T, int rows,
                             int H, int I, int E, uint16_t* y, void* ws, int32_t* err,
                             hipStream_t s) {
    uint16_t* h = static_cast<uint16_t*>(ws);
    // Many rows per expert: the tiled GEMM of dense.hip.
    const int groups = (E < rows) ? E : rows;
    const long long kMax32 = 0x7fffffffLL;  // its element offsets are 32-bit
    const bool fits32 = (long long)T * H < kMax32 && (long long)rows * I < kMax32 &&
                        2LL * I * H < kMax32 && (long long)rows * H < kMax32;
    if (fits32 && rows >= SMOE_DENSE_MIN_ROWS * groups) {
        int32_t* plan = reinterpret_cast<int32_t*>(
            static_cast<char*>(ws) + ((((size_t)rows * I * 2) + 255) & ~(size_t)255));
        return launch_dense_ffn(x, sorted_token, off, active, n_active, experts, mask, rows, H, I,
                                E, y, h, plan, err, s);
    }
    F16Args a1{};
    a1.xin = x;
    a1.sorted_token = sorted_token;
    a1.off = off;
    a1.active = active;
    a1.n_active = n_active;
    a1.experts = experts;
    a1.mask = mask;
    a1.K = H;
    a1.Ncol = I;
    a1.I = I;
    a1.H = H;
    a1.out = h;
    a1.err = err;
    F16Args a2 = a1;
    a2.xin = h;
    a2.sorted_token = nullptr;
    a2.K = I;
    a2.Ncol = H;
    a2.out = y;
    const int slots = active ? (E < rows ? E : rows) : E;
    // A few tokens (each at most once per expert, so at most T rows per
    // group; a longer group just takes more rows in turn): one wave per column.
    if (SMOE_VF_GEMV && T <= kGemvMaxT && H <= 512 * kGemvMaxChunks &&
        I <= 512 * kGemvMaxChunks) {
        a1.nCB = (I + kGemvWaves - 1) / kGemvWaves;
        a2.nCB = (H + kGemvWaves - 1) / kGemvWaves;
        hipError_t st = launch_gemv_phase<1>(a1, slots, s);
        if (st != hipSuccess) return st;
        return launch_gemv_phase<2>(a2, slots, s);
    }
    // row blocks of 16 held per weight stream, sized for the largest group
    // expected: all rows when there is one expert (a shared expert), else
    // about twice the mean plus slack (bigger groups take extra passes)
    const int mean = (rows + E - 1) / E;
    int est = (E == 1) ? rows : 2 * mean + 8;
    if (est > T) est = T;
    const int RB = (est <= 16) ? 1 : 2;
    a1.nCB = I / 16;
    a2.nCB = H / 16;
    hipError_t st = launch_phase<1>(a1, slots, RB, s);
    if (st != hipSuccess) return st;
    return launch_phase<2>(a2, slots, RB, s);
}

// The dense shared expert's two projections on their own: launches of its
// items only (token rows 0..T-1 of x), the one-group ring geometry.
hipError_t launch_dense_group(const uint16_t* x, int T, int H, const uint16_t* w13,
                                     const uint16_t* w2, int Is, uint16_t* sh_h,
                                     uint16_t* sh_out, int32_t* err, hipStream_t s) {
    F16Args g{};
    g.xin = x;
    g.K = H;
    g.H = H;
    g.err = err;
    g.ex_w = w13;
    g.ex_out = sh_h;
    g.ex_I = Is;
    g.ex_nCB = Is / 16;
    g.ex_T = T;
    const int RB = (T <= 16) ? 1 : 2;
    hipError_t st = launch_ring<1, SMOE_SH_GU_WAVES, SMOE_SH_GU_STAGES>(g, 0, RB, s);
    if (st != hipSuccess) return st;
    g.Ncol = H;
    g.ex_w = w2;
    g.ex_in = sh_h;
    g.ex_out = sh_out;
    g.ex_nCB = H / 16;
    return launch_ring<2, SMOE_SH_DN_WAVES, SMOE_SH_DN_STAGES>(g, 0, RB, s);
}

hipError_t launch_verify_ffn_shared(const uint16_t* x, const int32_t* sorted_token,
                                    const int32_t* off, const int32_t* active,
                                    const int32_t* n_active, const smoe_f16_expert* experts,
                                    const uint8_t* mask, int T, int rows, int H, int I, int E,
                                    uint16_t* y, void* ws, const uint16_t* sw13,
                                    const uint16_t* sw2, int Is, uint16_t* sh_h,
                                    uint16_t* sh_out, int32_t* err, hipStream_t s) {
    // the routed launches' geometry, as launch_verify_ffn picks it
    const int groups = (E < rows) ? E : rows;
    const long long kMax32 = 0x7fffffffLL;
    const bool fits32 = (long long)T * H < kMax32 && (long long)rows * I < kMax32 &&
                        2LL * I * H < kMax32 && (long long)rows * H < kMax32;
    const bool dense = fits32 && rows >= SMOE_DENSE_MIN_ROWS * groups;
    const bool gemv = SMOE_VF_GEMV && T <= kGemvMaxT && H <= 512 * kGemvMaxChunks &&
                      I <= 512 * kGemvMaxChunks;
    const int slots = active ? (E < rows ? E : rows) : E;
    const int mean = (rows + E - 1) / E;
    int est = (E == 1) ? rows : 2 * mean + 8;
    if (est > T) est = T;
    const int RB = (est <= 16) ? 1 : 2;
    F16Args a1{};
    a1.xin = x;
    a1.sorted_token = sorted_token;
    a1.off = off;
    a1.active = active;
    a1.n_active = n_active;
    a1.experts = experts;
    a1.mask = mask;
    a1.K = H;
    a1.Ncol = I;
    a1.I = I;
    a1.H = H;
    a1.out = static_cast<uint16_t*>(ws);
    a1.err = err;
    a1.nCB = I / 16;
    F16Args a2 = a1;
    a2.xin = a1.out;
    a2.sorted_token = nullptr;
    a2.K = I;
    a2.Ncol = H;
    a2.out = y;
    a2.nCB = H / 16;
    // fused: the shared expert's items lead the routed ring launches when
    // both projections run a ring kernel and its rows take no extra pass
    const int k1 = phase_kernel(a1, slots), k2 = phase_kernel(a2, slots);
    // a shared group of 17-32 rows: the launches take 32-row blocks
    const int RBf = (T > 16 && T <= 32) ? 2 : RB;
    if (!dense && !gemv && slots > 1 && (k1 == 1 || k1 == 2) && (k2 == 1 || k2 == 2) &&
        T <= 16 * RBf) {
        a1.ex_w = sw13;
        a1.ex_out = sh_h;
        a1.ex_I = Is;
        a1.ex_nCB = Is / 16;
        a1.ex_T = T;
        a2.ex_w = sw2;
        a2.ex_in = sh_h;
        a2.ex_out = sh_out;
        a2.ex_I = Is;
        a2.ex_nCB = H / 16;
        a2.ex_T = T;
        hipError_t st = launch_phase<1>(a1, slots, RBf, s);
        if (st != hipSuccess) return st;
        return launch_phase<2>(a2, slots, RBf, s);
    }
    hipError_t st = launch_verify_ffn(x, sorted_token, off, active, n_active, experts, mask, T,
                                      rows, H, I, E, y, ws, err, s);
    if (st != hipSuccess) return st;
    return launch_dense_group(x, T, H, sw13, sw2, Is, sh_h, sh_out, err, s);
}
}  // namespace smoe
