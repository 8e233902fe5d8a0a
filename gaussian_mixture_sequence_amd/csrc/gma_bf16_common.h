// Building blocks of the bf16 MFMA path (gfx950, wave64, v_mfma_f32_32x32x16_bf16).
//
// Scores (Sec. 4.1 Eq. 16 of "Gaussian Mixture Attention", expanded):
//   s_k = c_k + sum_d ( x_d a_kd + x_d^2 b_kd ),   a = mu / sigma2,  b = -1 / (2 sigma2),
//   c_k = log pi_k - 1/2 sum_d ( log sigma2_kd + mu_kd^2 / sigma2_kd )
// all pre-multiplied by log2(e) so the softmax of Eq. 3b is taken with exp2.  The
// contraction over d runs on bf16 MFMA with split operands: x is exact in bf16, x^2 is
// exact as hi + lo bf16, and a, b are carried as hi + lo bf16 pairs, so that
//   s = c + x.a_hi + x.a_lo + x2_hi.b_hi + x2_hi.b_lo + x2_lo.b_hi
// (the dropped x2_lo.b_lo term is ~2^-16 relative).  Accumulation is fp32.
//
// MFMA register layouts used throughout (lane l, lh = l / 32):
//   A operand (32 x 16): row i = l % 32, k = 8*lh + v for the 8 bf16 values v
//   B operand (16 x 32): col j = l % 32, k = 8*lh + v
//   D (32 x 32, 16 floats): col j = l % 32, row i = 8*(r/4) + 4*lh + r%4 for register r
// Scores are produced as S^T (rows = components, cols = tokens): every lane owns one
// token and 16 components of each 32-component tile, so the softmax over components is
// an in-lane reduction plus one exchange with lane l ^ 32.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "gma_device.h"

namespace gma {
namespace bf {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Both values of (x at lane l, x at lane l ^ 32), in some order.
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float xmax32(float x) { float a, b; swap32(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float xsum32(float x) { float a, b; swap32(x, a, b); return a + b; }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return uint32_t(f32_to_bf16_bits(lo)) | (uint32_t(f32_to_bf16_bits(hi)) << 16);
}

// x^2 split into hi + lo bf16 (exact: the square of an 8-bit significand has 16 bits).
__device__ __forceinline__ void square_split(bf16x8 x, bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float f0 = float(x[2 * q]), f1 = float(x[2 * q + 1]);
        float s0 = f0 * f0, s1 = f1 * f1;
        uint16_t h0 = f32_to_bf16_bits(s0), h1 = f32_to_bf16_bits(s1);
        float r0 = s0 - bf16_bits_to_f32(h0), r1 = s1 - bf16_bits_to_f32(h1);
        h[q] = uint32_t(h0) | (uint32_t(h1) << 16);
        l[q] = pack_bf16x2(r0, r1);
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Transposed fragment read from a row-major bf16 tile in LDS (ds_read_b64_tr_b16).
// Returns, for this lane, the 8 values  tile[row0 + 8*lh + v][col0 + (l % 32)],  v = 0..7,
// i.e. an MFMA A or B fragment whose k index runs down a column of the tile.
// Within each 16-lane group, the transposing read gives output lane q, element v, the
// value that source lane 4v + q/4 addressed, at offset q % 4; so source lane m points at
// row (m / 4) and columns 4 * (m % 4) .. + 3 of the group's 16-column strip.
__device__ __forceinline__ bf16x8 read_colfrag(const uint16_t* tile, int ld /*elements*/, int row0, int col0) {
    const int l = threadIdx.x & 63;
    const int lh = l >> 5;
    const int grp = (l >> 4) & 1;  // which 16-column strip of the 32 columns
    const int m = l & 15;
    const uint16_t* base = tile + (row0 + 8 * lh + (m >> 2)) * ld + col0 + 16 * grp + 4 * (m & 3);
    i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
    i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 4 * ld));
    i16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

// Row fragment: the 8 contiguous values tile[row][col0 + 8*lh .. + 7] (16-byte LDS read).
__device__ __forceinline__ bf16x8 read_rowfrag(const uint16_t* tile, int ld, int row, int col0) {
    const int lh = (threadIdx.x & 63) >> 5;
    return *reinterpret_cast<const bf16x8*>(tile + row * ld + col0 + 8 * lh);
}

// Wave-level work split of the score computation: CS waves share the components of one
// token subtile (each holds KT / CS component tiles of the parameter planes in
// registers), TS = NW / CS token subtiles of 32 tokens are processed side by side.
template <int DR, int KT>
struct Split {
    static constexpr int CS0 = (KT * DR) / 64;  // keeps the register-resident planes <= 64 VGPRs
    static constexpr int CS = CS0 < 1 ? 1 : (CS0 > KT ? KT : CS0);
    static constexpr int CTW = KT / CS;         // component tiles per wave
    static constexpr int NW = CS > 4 ? CS : 4;  // waves per workgroup
    static constexpr int TS = NW / CS;          // token subtiles per round
    static constexpr int ROUND = 32 * TS;       // tokens per round
    static constexpr int KS = DR / 16;          // k-steps of the d contraction
};

// Parameter planes of one wave: 4 bf16 planes (a_hi, a_lo, b_hi, b_lo) for its CTW
// component tiles, as MFMA A fragments, and the score constants in D-row order.
template <int DR, int CTW>
struct WaveParams {
    bf16x8 w[CTW][DR / 16][4];
    float c[CTW][16];

    // planes: [4][Kp][DR] bf16 of one head; cvec: [Kp] fp32 of one head; ct0: first tile
    __device__ __forceinline__ void load(const uint16_t* __restrict__ planes, const float* __restrict__ cvec,
                                         int Kp, int ct0) {
        const int l = threadIdx.x & 63, lh = l >> 5, i = l & 31;
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int comp = (ct0 + ct) * 32 + i;
#pragma unroll
            for (int ks = 0; ks < DR / 16; ++ks)
#pragma unroll
                for (int pl = 0; pl < 4; ++pl)
                    w[ct][ks][pl] = *reinterpret_cast<const bf16x8*>(
                        planes + (size_t(pl) * Kp + comp) * DR + 16 * ks + 8 * lh);
#pragma unroll
            for (int r = 0; r < 16; ++r) c[ct][r] = cvec[(ct0 + ct) * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)];
        }
    }
};

// B fragments of one 32-token subtile starting at row `n0` of X (row-major [N][DR] bf16
// of one problem): lane (lh, j) gets x[n0 + j][16 ks + 8 lh .. + 7].  Rows >= `valid`
// read as zero (no memory access).
template <int DR>
__device__ __forceinline__ void load_x(const uint16_t* __restrict__ X, int64_t n0, int valid, bf16x8 (&xs)[DR / 16]) {
    const int l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const bool ok = j < valid;
    const uint16_t* row = X + (n0 + (ok ? j : 0)) * DR + 8 * lh;
#pragma unroll
    for (int ks = 0; ks < DR / 16; ++ks)
        xs[ks] = ok ? *reinterpret_cast<const bf16x8*>(row + 16 * ks) : zero_bf16x8();
}

// S^T for one 32-token subtile from its B fragments: acc[ct] holds the scores of
// component tile ct (rows = components, cols = tokens).
template <int DR, int CTW>
__device__ __forceinline__ void scores_x(const WaveParams<DR, CTW>& P, const bf16x8 (&xs)[DR / 16],
                                         f32x16 (&acc)[CTW]) {
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ct][r] = P.c[ct][r];
#pragma unroll
    for (int ks = 0; ks < DR / 16; ++ks) {
        bf16x8 x2h, x2l;
        square_split(xs[ks], x2h, x2l);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            acc[ct] = mfma(P.w[ct][ks][0], xs[ks], acc[ct]);
            acc[ct] = mfma(P.w[ct][ks][1], xs[ks], acc[ct]);
            acc[ct] = mfma(P.w[ct][ks][2], x2h, acc[ct]);
            acc[ct] = mfma(P.w[ct][ks][3], x2h, acc[ct]);
            acc[ct] = mfma(P.w[ct][ks][2], x2l, acc[ct]);
        }
    }
}

// load_x + scores_x.
template <int DR, int CTW>
__device__ __forceinline__ void scores(const WaveParams<DR, CTW>& P, const uint16_t* __restrict__ X, int64_t n0,
                                       int valid, f32x16 (&acc)[CTW]) {
    bf16x8 xs[DR / 16];
    load_x<DR>(X, n0, valid, xs);
    scores_x<DR, CTW>(P, xs, acc);
}

// Softmax statistics of one wave's components for its lane's token: max m, sum of
// exp2(s - m), optional sum of exp2(s - m) * z_k.  acc is overwritten by exp2(s - m).
template <int CTW, bool WITH_Z>
__device__ __forceinline__ void local_softmax(f32x16 (&acc)[CTW], const float (&zr)[CTW][16], float& m,
                                              float& L, float& D) {
    m = -INFINITY;
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[ct][r]);
    m = xmax32(m);
    L = 0.0f;
    D = 0.0f;
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float e = __builtin_amdgcn_exp2f(acc[ct][r] - m);
            acc[ct][r] = e;
            L += e;
            if (WITH_Z) D = fmaf(e, zr[ct][r], D);
        }
    L = xsum32(L);
    if (WITH_Z) D = xsum32(D);
}

// Store scaled probabilities of this wave's component tiles into a row-major bf16 LDS
// tile G[row][comp] (row = token within the round): 4 consecutive components per store.
template <int CTW>
__device__ __forceinline__ void store_gamma_lds(const f32x16 (&e)[CTW], float scale, uint16_t* G, int ld, int row,
                                                int ct0) {
    const int lh = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u32x2 v;
            v[0] = pack_bf16x2(e[ct][4 * q + 0] * scale, e[ct][4 * q + 1] * scale);
            v[1] = pack_bf16x2(e[ct][4 * q + 2] * scale, e[ct][4 * q + 3] * scale);
            *reinterpret_cast<u32x2*>(G + row * ld + (ct0 + ct) * 32 + 8 * q + 4 * lh) = v;
        }
}

}  // namespace bf
}  // namespace gma
