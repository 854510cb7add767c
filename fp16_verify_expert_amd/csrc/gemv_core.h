// One-row FP16 matrix-vector product, one wave per output column: the
// arithmetic shared by the matrix-vector verify kernel (a few tokens) and the
// dense shared expert folded into the one-token draft launches, so both give
// bit-identical outputs.
//
// A column's weight row is read as 16-byte chunks, lane l holding chunks l,
// l + 64, ... (each load instruction is 1 KB of one row); the activation row
// the same way.  Each lane dots its chunks in increasing order with
// v_dot2_f32_f16 (fp32 sums), then the wave's 64 lane sums are added in a
// fixed order (wave_sum).  The gate/up projection holds the gate row n and the
// up row I + n of w13 and applies SwiGLU (silu(g) * u) before the one
// rounding to fp16; the down projection holds row n of w2.
#pragma once
#include "common.h"

namespace smoe_gemv {

SMOE_DEV h2_t as_h2v(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

SMOE_DEV float dot8(u4_t w, uint4 x, float acc) {
    acc = __builtin_amdgcn_fdot2(as_h2v(w.x), as_h2v(x.x), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2v(w.y), as_h2v(x.y), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2v(w.z), as_h2v(x.z), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2v(w.w), as_h2v(x.w), acc, false);
    return acc;
}

// Sum over the wave in a fixed order: within each row of 16 lanes by DPP
// (swap neighbours, swap pairs, rotate by 4, rotate by 8), then the four row
// sums read from lanes 0, 16, 32 and 48.
template <int CTRL>
SMOE_DEV float dpp_add(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
    return v + __builtin_bit_cast(float, t);
}
SMOE_DEV float lane_value(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
SMOE_DEV float wave_sum(float v) {
    v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x124>(v);  // row_ror 4
    v = dpp_add<0x128>(v);  // row_ror 8
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

SMOE_DEV float silu(float g) { return g / (1.0f + expf(-g)); }

// Weight chunks of column nc (clamped into the matrix by the caller): the
// gate row nc and the up row I + nc (NM = 2) or row nc (NM = 1) of W [., K].
// Chunks past the row re-read its last chunk; they are masked in gemv_dot.
template <int NM, int CPL>
SMOE_DEV void gemv_load_w(const uint16_t* W, int K, int I, int nc, int lane, u4_t (&wv)[NM][CPL]) {
    const int kc = K >> 3;  // 16-byte chunks per row
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const size_t row = (m == 0) ? (size_t)nc : (size_t)I + nc;
        gptr<u4_t> wr = as_global(reinterpret_cast<const u4_t*>(W + row * K));
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lane + 64 * j;
            wv[m][j] = __builtin_nontemporal_load(wr + (c < kc ? c : kc - 1));
        }
    }
}

// Activation chunks of one row (same chunk assignment as the weights).
template <int CPL>
SMOE_DEV void gemv_load_x(const uint16_t* xrow, int K, int lane, uint4 (&xr)[CPL]) {
    const int kc = K >> 3;
    const uint4* x4 = reinterpret_cast<const uint4*>(xrow);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        xr[j] = x4[c < kc ? c : kc - 1];
    }
}

// The column's output for one row, as the fp16 bits the kernels store
// (every lane returns the same value).
template <int NM, int CPL>
SMOE_DEV uint16_t gemv_dot(const u4_t (&wv)[NM][CPL], const uint4 (&xr)[CPL], int K, int lane) {
    const int kc = K >> 3;
    const u4_t wzero = {0u, 0u, 0u, 0u};
    float acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const bool in = lane + 64 * j < kc;
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] = dot8(in ? wv[m][j] : wzero, xr[j], acc[m]);
    }
    float tot[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) tot[m] = wave_sum(acc[m]);
    const float v = (NM == 2) ? silu(tot[0]) * tot[NM - 1] : tot[0];
    return f2h(v);
}

// Chunks per lane and row for a reduction of K (rounded up to an
// instantiated width).
constexpr int kMaxChunks = 16;  // K <= 8192
inline int chunks_for(int K) {
    const int need = (K / 8 + 63) / 64;
    if (need <= 2) return 2;
    if (need <= 4) return 4;
    if (need <= 6) return 6;
    if (need <= 8) return 8;
    if (need <= 12) return 12;
    return kMaxChunks;
}

}  // namespace smoe_gemv
