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
// Work decomposition.  A workgroup (4 waves) owns one (touched expert, block
// of 256 weight columns, range of 4 K-groups).  Lane l of a wave reads 16
// bytes = 4 adjacent columns of one packed row, so a wave load is 1 KB of
// contiguous qweight (two 512-byte runs in the gate/up projection, whose block
// is 128 gate columns next to the matching 128 up columns).  Each wave streams
// whole 128-row groups (16 packed rows, 16 loads in flight per lane).
//
// Dequantisation.  For a packed word w, (w & 0x000F000F) | 0x64006400 is the
// fp16 pair (1024 + q_i, 1024 + q_(i+4)) and (w & 0x00F000F0) | 0x64006400 is
// (1024 + 16 q_(i+1), 1024 + 16 q_(i+5)); a shift by 8 gives the other four
// codes.  These pairs go straight into v_dot2_f32_f16 against the matching
// activation pairs (fp32 accumulate).  Per group and column the constant
// parts are removed once:
//   sum_k (q_k - z) x_k = A_even + A_odd / 16 - (1024 + z) S_even - (64 + z) S_odd
// where S_even / S_odd are the group's sums of x over even / odd k; the group
// result is then multiplied by the fp16 scale.  Cost: 5 integer ops per packed
// word plus 4 dot2 per word per row.
//
// Split-K.  Partial sums of the K ranges of one (expert, column block) are
// written to the workspace; the last workgroup to finish (an atomic counter)
// adds them in a fixed order and applies the epilogue (SwiGLU -> fp16 h for
// the gate/up projection; fp16 y for the down projection), then resets the
// counter.  No floating-point atomics: the output is deterministic.
#include "common.h"

namespace {

constexpr int kW4Threads = 256;
constexpr int kW4Waves = 4;
constexpr int kGroupsPerWave = 1;
constexpr int kGroupsPerBlock = kW4Waves * kGroupsPerWave;
constexpr int kRowsPerGroup = 16;  // packed rows (8 K each) per 128-K group
constexpr uint32_t kMagic = 0x64006400u;
constexpr int kMaxM = 8;

struct W4Args {
    const uint16_t* xin;          // phase 1: x [T, H]; phase 2: h [rows, I]
    const int32_t* sorted_token;  // phase 1 only
    const int32_t* off;
    const int32_t* active;
    const int32_t* n_active;
    const smoe_w4_expert* experts;
    int K;       // reduction length: H (phase 1) or I (phase 2)
    int N;       // weight columns: 2I or H
    int I;
    int nCB;     // column blocks of 256 logical columns
    int KS;      // K splits (workgroups per column block)
    float* part;     // [KS][rows_total][N] fp32
    int32_t* cnt;    // [slots][nCB] completion counters
    uint16_t* out;   // phase 1: h [rows_total, I]; phase 2: y [rows_total, H]
    int32_t* err;
    int rows_total;  // rows of the partial buffer (T*k)
};

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// One 128-K group for M rows: accumulate the four dot2 streams of every row
// and column, then fold the constants, zero and scale into tot.
template <int M>
__device__ __forceinline__ void group_dot(const u4_t (&wv)[kRowsPerGroup], const uint4* xs_g,
                                          int xs_stride, const float2* sg, uint2 sv, uint32_t zw,
                                          float (&tot)[kMaxM][4]) {
    float ae[M][4], ao[M][4];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) ae[m][c] = ao[m][c] = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowsPerGroup; ++i) {
        uint4 xp[M];
#pragma unroll
        for (int m = 0; m < M; ++m) xp[m] = xs_g[m * xs_stride + i];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t w = wv[i][c];
            const uint32_t b = w >> 8;
            const h2_t e0 = as_h2((w & 0x000F000Fu) | kMagic);
            const h2_t o0 = as_h2((w & 0x00F000F0u) | kMagic);
            const h2_t e1 = as_h2((b & 0x000F000Fu) | kMagic);
            const h2_t o1 = as_h2((b & 0x00F000F0u) | kMagic);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                ae[m][c] = __builtin_amdgcn_fdot2(e0, as_h2(xp[m].x), ae[m][c], false);
                ao[m][c] = __builtin_amdgcn_fdot2(o0, as_h2(xp[m].y), ao[m][c], false);
                ae[m][c] = __builtin_amdgcn_fdot2(e1, as_h2(xp[m].z), ae[m][c], false);
                ao[m][c] = __builtin_amdgcn_fdot2(o1, as_h2(xp[m].w), ao[m][c], false);
            }
        }
    }
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
            t -= ce * sg[m].x;
            t -= co * sg[m].y;
            tot[m][c] += s * t;
        }
    }
}

template <int PHASE>
__global__ __launch_bounds__(kW4Threads) void w4_kernel(W4Args a) {
    __shared__ uint4 xs[kMaxM][kGroupsPerBlock * kRowsPerGroup];  // permuted x pairs
    __shared__ float2 sums[kMaxM][kGroupsPerBlock];               // (S_even, S_odd)
    __shared__ float red[kW4Waves][kMaxM][256];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ks = blockIdx.x % a.KS;
    const int rest = blockIdx.x / a.KS;
    const int cb = rest % a.nCB;
    const int slot = rest / a.nCB;
    if (slot >= *a.n_active) return;
    const int e = a.active[slot];
    const int r0 = a.off[e];
    const int r1 = a.off[e + 1];
    const smoe_w4_mat wm = (PHASE == 1) ? a.experts[e].w13 : a.experts[e].w2;
    if (!wm.qweight || !wm.scales || !wm.qzeros) {
        if (tid == 0 && ks == 0 && cb == 0) flag_error(a.err, SMOE_DERR_NULL_EXPERT);
        return;
    }
    const int K = a.K, N = a.N;
    const int G = K >> 7;
    const int g0 = ks * kGroupsPerBlock;
    const int g1 = min(G, g0 + kGroupsPerBlock);
    const int nrow_local = (g1 - g0) * kRowsPerGroup;

    // this lane's 4 adjacent weight columns
    int col;
    bool colok;
    if (PHASE == 1) {
        col = (lane < 32) ? cb * 128 + 4 * lane : a.I + cb * 128 + 4 * (lane - 32);
        colok = true;
    } else {
        col = cb * 256 + 4 * lane;
        colok = col < N;
    }
    const int N4 = N >> 2;

    for (int mc = r0; mc < r1; mc += kMaxM) {
        const int M = min(kMaxM, r1 - mc);
        __syncthreads();  // xs / sums / red reuse across row chunks
        // ---- stage x (permuted into dot2 pairs) for rows mc .. mc+M-1 ----
        for (int idx = tid; idx < M * nrow_local; idx += kW4Threads) {
            const int m = idx / nrow_local;
            const int rr = idx - m * nrow_local;
            const uint16_t* src;
            if (PHASE == 1)
                src = a.xin + (size_t)a.sorted_token[mc + m] * K;
            else
                src = a.xin + (size_t)(mc + m) * K;
            const uint4 d = reinterpret_cast<const uint4*>(src)[(g0 * kRowsPerGroup + rr)];
            uint4 p;
            p.x = (d.x & 0xFFFFu) | (d.z << 16);          // (x0, x4)
            p.y = (d.x >> 16) | (d.z & 0xFFFF0000u);      // (x1, x5)
            p.z = (d.y & 0xFFFFu) | (d.w << 16);          // (x2, x6)
            p.w = (d.y >> 16) | (d.w & 0xFFFF0000u);      // (x3, x7)
            xs[m][rr] = p;
        }
        __syncthreads();
        if (tid < M * (g1 - g0)) {
            const int m = tid / (g1 - g0);
            const int gl = tid - m * (g1 - g0);
            float se = 0.0f, so = 0.0f;
            for (int i = 0; i < kRowsPerGroup; ++i) {
                const uint4 p = xs[m][gl * kRowsPerGroup + i];
                const h2_t x04 = as_h2(p.x), x15 = as_h2(p.y), x26 = as_h2(p.z),
                           x37 = as_h2(p.w);
                se += (float)x04.x + (float)x04.y + (float)x26.x + (float)x26.y;
                so += (float)x15.x + (float)x15.y + (float)x37.x + (float)x37.y;
            }
            sums[m][gl] = make_float2(se, so);
        }
        __syncthreads();

        // ---- stream this wave's groups ----
        float tot[kMaxM][4];
#pragma unroll
        for (int m = 0; m < kMaxM; ++m)
#pragma unroll
            for (int c = 0; c < 4; ++c) tot[m][c] = 0.0f;

        for (int g = g0 + wave; g < g1; g += kW4Waves) {
            const int gl = g - g0;
            u4_t wv[kRowsPerGroup];
            const u4_t* qp =
                reinterpret_cast<const u4_t*>(wm.qweight + (size_t)(g * kRowsPerGroup) * N + col);
#pragma unroll
            for (int i = 0; i < kRowsPerGroup; ++i)
                wv[i] = colok ? __builtin_nontemporal_load(qp + (size_t)i * N4) : u4_t{0, 0, 0, 0};
            uint2 sv = make_uint2(0, 0);
            uint32_t zw = 0;
            if (colok) {
                sv = *reinterpret_cast<const uint2*>(wm.scales + (size_t)g * N + col);
                zw = (uint32_t)wm.qzeros[(size_t)g * (N >> 3) + (col >> 3)] >> (4 * (col & 7));
            }
            const uint4* xg = &xs[0][gl * kRowsPerGroup];
            const float2* sg = &sums[0][gl];
            constexpr int xstr = kGroupsPerBlock * kRowsPerGroup;
            switch (M) {
                case 1: group_dot<1>(wv, xg, xstr, sg, sv, zw, tot); break;
                case 2: {
                    const float2 s2[2] = {sums[0][gl], sums[1][gl]};
                    group_dot<2>(wv, xg, xstr, s2, sv, zw, tot);
                } break;
                default: {
                    float2 s8[kMaxM];
#pragma unroll
                    for (int m = 0; m < kMaxM; ++m) s8[m] = sums[m][gl];
                    if (M <= 4)
                        group_dot<4>(wv, xg, xstr, s8, sv, zw, tot);
                    else
                        group_dot<8>(wv, xg, xstr, s8, sv, zw, tot);
                }
            }
        }
        // ---- reduce the 4 waves (fixed order) ----
#pragma unroll
        for (int m = 0; m < kMaxM; ++m)
            if (m < M)
#pragma unroll
                for (int c = 0; c < 4; ++c) red[wave][m][4 * lane + c] = tot[m][c];
        __syncthreads();
        for (int m = 0; m < M; ++m) {
            const float v = ((red[0][m][tid] + red[1][m][tid]) + red[2][m][tid]) + red[3][m][tid];
            red[0][m][tid] = v;
        }
        __syncthreads();

        if (a.KS == 1) {
            // ---- epilogue straight from LDS ----
            if (PHASE == 1) {
                for (int idx = tid; idx < M * 128; idx += kW4Threads) {
                    const int m = idx >> 7, j = idx & 127;
                    const float gv = red[0][m][j], uv = red[0][m][128 + j];
                    a.out[(size_t)(mc + m) * a.I + cb * 128 + j] = f2h(silu_f(gv) * uv);
                }
            } else if (cb * 256 + tid < N) {
                for (int m = 0; m < M; ++m)
                    a.out[(size_t)(mc + m) * N + cb * 256 + tid] = f2h(red[0][m][tid]);
            }
        } else {
            // ---- write this K range's partial ----
            int pcol;
            bool pok;
            if (PHASE == 1) {
                pcol = (tid < 128) ? cb * 128 + tid : a.I + cb * 128 + (tid - 128);
                pok = true;
            } else {
                pcol = cb * 256 + tid;
                pok = pcol < N;
            }
            if (pok)
                for (int m = 0; m < M; ++m)
                    a.part[((size_t)ks * a.rows_total + (mc + m)) * N + pcol] = red[0][m][tid];
        }
    }
    if (a.KS == 1) return;

    // ---- last workgroup of this (expert, column block) finishes ----
    __threadfence();
    __syncthreads();
    int32_t* ctr = a.cnt + (size_t)slot * a.nCB + cb;
    if (tid == 0) s_last = (atomicAdd(ctr, 1) == a.KS - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const size_t kstride = (size_t)a.rows_total * N;
    if (PHASE == 1) {
        for (int idx = tid; idx < (r1 - r0) * 128; idx += kW4Threads) {
            const int r = r0 + (idx >> 7), j = idx & 127;
            const float* pg = a.part + (size_t)r * N + cb * 128 + j;
            const float* pu = a.part + (size_t)r * N + a.I + cb * 128 + j;
            float gv = 0.0f, uv = 0.0f;
            for (int s = 0; s < a.KS; ++s) {
                gv += __builtin_nontemporal_load(pg + s * kstride);
                uv += __builtin_nontemporal_load(pu + s * kstride);
            }
            a.out[(size_t)r * a.I + cb * 128 + j] = f2h(silu_f(gv) * uv);
        }
    } else {
        const int n = cb * 256 + tid;
        if (n < N)
            for (int r = r0; r < r1; ++r) {
                const float* pp = a.part + (size_t)r * N + n;
                float v = 0.0f;
                for (int s = 0; s < a.KS; ++s) v += __builtin_nontemporal_load(pp + s * kstride);
                a.out[(size_t)r * N + n] = f2h(v);
            }
    }
    if (tid == 0) atomicExch(ctr, 0);
}

struct W4Plan {
    int slots, rows, G1, G2, nCB1, nCB2, KS1, KS2;
    size_t off_cnt2, off_h, off_p1, off_p2, total;
};

__host__ inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

W4Plan plan_w4(int T, int k, int H, int I, int E) {
    W4Plan p{};
    p.rows = T * k;
    p.slots = E < p.rows ? E : p.rows;
    p.G1 = H / 128;
    p.G2 = I / 128;
    p.nCB1 = I / 128;
    p.nCB2 = (H + 255) / 256;
    p.KS1 = (p.G1 + kGroupsPerBlock - 1) / kGroupsPerBlock;
    p.KS2 = (p.G2 + kGroupsPerBlock - 1) / kGroupsPerBlock;
    size_t o = 0;
    o += align256((size_t)p.slots * p.nCB1 * 4);
    p.off_cnt2 = o;
    o += align256((size_t)p.slots * p.nCB2 * 4);
    p.off_h = o;
    o += align256((size_t)p.rows * I * 2);
    p.off_p1 = o;
    o += align256((size_t)(p.KS1 > 1 ? p.KS1 : 0) * p.rows * (2 * (size_t)I) * 4);
    p.off_p2 = o;
    o += align256((size_t)(p.KS2 > 1 ? p.KS2 : 0) * p.rows * (size_t)H * 4);
    p.total = o;
    return p;
}

}  // namespace

namespace smoe {
size_t w4a16_workspace_bytes(int T, int k, int H, int I, int E) {
    return plan_w4(T, k, H, I, E).total;
}

hipError_t launch_w4a16_ffn(const uint16_t* x, const int32_t* sorted_token, const int32_t* off,
                            const int32_t* active, const int32_t* n_active,
                            const smoe_w4_expert* experts, int T, int k, int H, int I, int E,
                            uint16_t* y, void* ws, int32_t* err, hipStream_t s) {
    const W4Plan p = plan_w4(T, k, H, I, E);
    char* base = static_cast<char*>(ws);
    uint16_t* h = reinterpret_cast<uint16_t*>(base + p.off_h);
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
    a1.nCB = p.nCB1;
    a1.KS = p.KS1;
    a1.part = reinterpret_cast<float*>(base + p.off_p1);
    a1.cnt = reinterpret_cast<int32_t*>(base);
    a1.out = h;
    a1.err = err;
    a1.rows_total = p.rows;
    hipLaunchKernelGGL(w4_kernel<1>, dim3(p.slots * p.nCB1 * p.KS1, 1, 1), dim3(kW4Threads), 0,
                       s, a1);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
    W4Args a2 = a1;
    a2.xin = h;
    a2.sorted_token = nullptr;
    a2.K = I;
    a2.N = H;
    a2.nCB = p.nCB2;
    a2.KS = p.KS2;
    a2.part = reinterpret_cast<float*>(base + p.off_p2);
    a2.cnt = reinterpret_cast<int32_t*>(base + p.off_cnt2);
    a2.out = y;
    hipLaunchKernelGGL(w4_kernel<2>, dim3(p.slots * p.nCB2 * p.KS2, 1, 1), dim3(kW4Threads), 0,
                       s, a2);
    return hipGetLastError();
}
}  // namespace smoe
