// FP16 verification FFN over rows grouped by expert, on MFMA.
//
// "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step Speculative
// Offloading" (AI summary), Key Contributions 4 and Methodology: the K+1 tokens
// routed to one expert are packed together so that the per-token
// matrix-vector products become one matrix-matrix product per expert (same
// result, the routing and masking being unchanged).  Key Contributions 3:
// experts already resident are computed first while missing ones load, hence
// the optional expert mask.
//
// Each wave owns 16 output columns of one touched expert and streams the
// weight rows of those columns over the whole reduction, feeding
// v_mfma_f32_16x16x32_f16 directly from registers: lane l loads 16 bytes of
// weight row (n0 + l%16) at K offset 8*(l/16) -- exactly the B-operand layout
// -- and the matching activation row (l%16) of the expert's packed rows as the
// A operand.  Rows beyond the expert's count are zero, so the MFMA is only as
// wide as the data; at K+1 <= 33 tokens the kernel is bound by the HBM stream
// of the touched experts' weights.  Up to RB row blocks of 16 share one weight
// stream.  The gate/up projection applies SwiGLU in registers and writes h as
// fp16; the down projection writes y_sorted.
#include "common.h"

namespace {

constexpr int kF16Threads = 256;  // 4 waves, 16 columns each
constexpr int kF16Waves = 4;
constexpr int kUnroll = 4;        // 4 x 32 K per step

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
    int nWB;    // workgroup column blocks (64 columns each)
    uint16_t* out;  // phase 1: h [rows, I]; phase 2: y [rows, H]
    int32_t* err;
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

template <int PHASE, int RB>
__global__ __launch_bounds__(kF16Threads) void f16_kernel(F16Args a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wb = blockIdx.x % a.nWB;
    const int slot = blockIdx.x / a.nWB;
    int e;
    if (a.active) {
        if (slot >= *a.n_active) return;
        e = a.active[slot];
    } else {
        e = slot;
    }
    if (a.mask && !a.mask[e]) return;
    const int r0 = a.off[e];
    const int r1 = a.off[e + 1];
    if (r1 <= r0) return;
    const uint16_t* W = (PHASE == 1) ? a.experts[e].w13 : a.experts[e].w2;
    if (!W) {
        if (threadIdx.x == 0 && wb == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
        return;
    }
    const int K = a.K;
    const int n = (wb * kF16Waves + wave) * 16 + (lane & 15);
    if ((wb * kF16Waves + wave) * 16 >= a.Ncol) return;  // whole wave past the end
    const bool colok = n < a.Ncol;
    const int kq = 8 * (lane >> 4);
    const h8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

    const h8_t* wg = reinterpret_cast<const h8_t*>(W + (size_t)(colok ? n : 0) * K + kq);
    const h8_t* wu = (PHASE == 1)
                         ? reinterpret_cast<const h8_t*>(W + (size_t)(a.I + (colok ? n : 0)) * K + kq)
                         : wg;

    for (int mb = r0; mb < r1; mb += 16 * RB) {
        const h8_t* arow[RB];
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
            arow[b] = reinterpret_cast<const h8_t*>(src + kq);
        }
        f4_t accg[RB], accu[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            accg[b] = f4_t{0.f, 0.f, 0.f, 0.f};
            accu[b] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
        // software pipeline: weights for step s+1 are in flight while step s
        // is multiplied
        h8_t bg[kUnroll], bu[kUnroll], nbg[kUnroll], nbu[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            bg[u] = colok ? __builtin_nontemporal_load(wg + 4 * u) : zero8;
            if (PHASE == 1) bu[u] = colok ? __builtin_nontemporal_load(wu + 4 * u) : zero8;
        }
        for (int k0 = 0; k0 < K; k0 += 32 * kUnroll) {
            const int kn = k0 + 32 * kUnroll;
            const bool more = kn < K;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const size_t o = (size_t)(kn >> 3) + 4 * u;  // in h8 units
                nbg[u] = (more && colok) ? __builtin_nontemporal_load(wg + o) : zero8;
                if (PHASE == 1) nbu[u] = (more && colok) ? __builtin_nontemporal_load(wu + o) : zero8;
            }
            h8_t av[RB][kUnroll];
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    av[b][u] = aok[b] ? arow[b][(k0 >> 3) + 4 * u] : zero8;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    accg[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[b][u], bg[u], accg[b], 0, 0, 0);
                    if (PHASE == 1)
                        accu[b] =
                            __builtin_amdgcn_mfma_f32_16x16x32_f16(av[b][u], bu[u], accu[b], 0, 0, 0);
                }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                bg[u] = nbg[u];
                if (PHASE == 1) bu[u] = nbu[u];
            }
        }
        // D[row = 4*(lane/16) + i][col = lane%16]
        if (colok) {
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = mb + 16 * b + 4 * (lane >> 4) + i;
                    if (r < r1) {
                        float v;
                        if (PHASE == 1)
                            v = silu_f(accg[b][i]) * accu[b][i];
                        else
                            v = accg[b][i];
                        a.out[(size_t)r * a.Ncol + n] = f2h(v);
                    }
                }
        }
    }
}

template <int PHASE>
hipError_t launch_phase(const F16Args& a, int slots, int RB, hipStream_t s) {
    const dim3 grid(slots * a.nWB), block(kF16Threads);
    switch (RB) {
        case 1: hipLaunchKernelGGL((f16_kernel<PHASE, 1>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((f16_kernel<PHASE, 2>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((f16_kernel<PHASE, 4>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace

namespace smoe {
size_t verify_workspace_bytes(int /*T*/, int rows, int /*H*/, int I, int /*E*/) {
    return (((size_t)rows * I * 2) + 255) & ~(size_t)255;
}

hipError_t launch_verify_ffn(const uint16_t* x, const int32_t* sorted_token, const int32_t* off,
                             const int32_t* active, const int32_t* n_active,
                             const smoe_f16_expert* experts, const uint8_t* mask, int T, int rows,
                             int H, int I, int E, uint16_t* y, void* ws, int32_t* err,
                             hipStream_t s) {
    // row blocks held per weight stream: enough for the largest possible
    // expert group (<= T rows) up to 64
    const int RB = (T <= 16) ? 1 : (T <= 32) ? 2 : 4;
    const int slots = active ? (E < rows ? E : rows) : E;
    uint16_t* h = static_cast<uint16_t*>(ws);
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
    a1.nWB = (I + 63) / 64;
    a1.out = h;
    a1.err = err;
    hipError_t st = launch_phase<1>(a1, slots, RB, s);
    if (st != hipSuccess) return st;
    F16Args a2 = a1;
    a2.xin = h;
    a2.sorted_token = nullptr;
    a2.K = I;
    a2.Ncol = H;
    a2.nWB = (H + 63) / 64;
    a2.out = y;
    return launch_phase<2>(a2, slots, RB, s);
}
}  // namespace smoe
