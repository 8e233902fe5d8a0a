// Backward passes of the GMA forward with fp32 arithmetic (Sec. 4.1 of "Gaussian Mixture
// Attention"): the bidirectional and causal forwards, fp32 or bf16 I/O (bf16 is staged
// through fp32 copies).  Register-tiled passes where K, d_r, d_v <= 64 fit the LDS; one
// element per thread otherwise.  The score tables, responsibility tiles and the split
// write / combine / prefix kernels come from gma_f32_common.h.
#include <algorithm>

#include "gma_f32_common.h"

namespace gma {

// ============================================================================ backward
// Gradients of <dO, O> for the bidirectional forward (Sec. 4.1 of "Gaussian Mixture
// Attention": the softmax Jacobian of Eq. 17, the centred score gradient of Eq. 18 and the
// chain rule of Eq. 19-20 through the direct-form score of Eq. 16), fp32.  With
// D_i = gamma^Q_i . Z + eps, dO'_i = dO_i / D_i and a'_i = dO_i . O_i / D_i:
//   g^Q_ik = dO'_i . Vt_k - a'_i Z_k,            dVt_k = sum_i gamma^Q_ik dO'_i,
//   dZ_k = -sum_i gamma^Q_ik a'_i,                dV_j = sum_k gamma^K_jk dVt_k,
//   g^K_jk = dVt_k . V_j + dZ_k,                  ds_ik = gamma_ik (g_ik - sum_l gamma_il g_il),
//   dx_id = -sum_k ds_ik (x_id - mu_kd) / sigma2_kd.
// The mixture parameters see every row of both sides through three moments per split,
//   S0_k = sum_i ds_ik,  S1_kd = sum_i ds_ik (x_id - mu_kd),  S2_kd = sum_i ds_ik (x_id - mu_kd)^2,
// kept in the direct (centred) form, from which dmu_kd = S1_kd / sigma2_kd,
// dsigma2_kd = (S2_kd / sigma2_kd^2 - S0_k / sigma2_kd) / 2 and dpi_k = S0_k / pi_k.
// Partial records per (problem, split): [S1 (K d_r) | S2 (K d_r) | S0 (K)].
namespace {

// gamma_tile with fp32 tables in LDS: c [K], 1/sigma2 and mu as [K][LR] rows (LR = d_r + 1),
// the direct-form score of Eq. 16 in fp32, then the softmax of Eq. 3b.  Same contract as gamma_tile.
__device__ void gamma_tile_lds(const float* __restrict__ X, int64_t n0, int rows, int T, int dr, int K,
                               const float* c_l, const float* inv_l, const float* mu_l, float* xs, float* g) {
    const int LR = dr + 1;
    for (int i = threadIdx.x; i < T * dr; i += kThreads) {
        const int t = i / dr;
        xs[i] = (t < rows) ? X[(n0 + t) * dr + (i - t * dr)] : 0.0f;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int t = wave; t < T; t += kThreads / kWave) {
        float* gt = g + size_t(t) * K;
        if (t >= rows) {
            for (int k = lane; k < K; k += kWave) gt[k] = 0.0f;
            continue;
        }
        const float* xt = xs + t * dr;
        float sc[4], m = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = lane + j * kWave;
            sc[j] = -INFINITY;
            if (k < K) {
                const float *mk = mu_l + k * LR, *ik = inv_l + k * LR;
                float q = 0.0f;
                for (int d = 0; d < dr; ++d) {
                    const float df = xt[d] - mk[d];
                    q = fmaf(df * df, ik[d], q);
                }
                sc[j] = c_l[k] - 0.5f * q;
                m = fmaxf(m, sc[j]);
            }
        }
        m = wave_max(m);
        float ev[4], sum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ev[j] = (lane + j * kWave < K) ? expf(sc[j] - m) : 0.0f;
            sum += ev[j];
        }
        sum = wave_sum(sum);
        const float r = 1.0f / sum;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (lane + j * kWave < K) gt[lane + j * kWave] = ev[j] * r;
    }
    __syncthreads();
}

// ---- general sizes: one thread per output element, LDS tiles of T rows
size_t bwd_lds_bytes(int T, int dr, int dv, int K) { return size_t(T) * (dr + 2 * K + dv + 2) * sizeof(float); }

// Grid (G, P): rows [g seg, (g + 1) seg) of problem p in tiles of T.  QUERY: the query side
// (reads the memory mem = [Vt | Z], writes dX_Q and the partial [dVt | dZ] of its rows);
// otherwise the key side (reads dmem = [dVt | dZ], writes dV and dX_K).  Both write the
// block's moment record pp (first tile writes, later tiles add: each entry has one owner).
// FAST: the per-head tables (fp32) sit in LDS (rows padded by one element), and the memory too
// when mem_lds is set; the scores, dX and moments are then fp32.  Otherwise everything comes from
// the fp64 tables and the memory in the workspace.
template <bool QUERY, bool FAST>
__global__ void __launch_bounds__(kThreads)
    f32_bwd_side_kernel(const float* __restrict__ X, const float* __restrict__ Y, int64_t N, int H, int dr, int dv,
                        int K, int64_t seg, int G, int T, const double* c, const double* inv, const float* mu,
                        const float* __restrict__ mem, float eps, float* __restrict__ dX, float* __restrict__ dY,
                        float* __restrict__ mem_part, float* __restrict__ param_part, int mem_lds) {
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int gi = blockIdx.x, h = int(p % H);
    float* xs = lds;          // T*dr: the tile's routing vectors (left by gamma_tile)
    float* gm = xs + T * dr;  // T*K: responsibilities
    float* gg = gm + T * K;   // T*K: upstream gradient, then the score gradient
    float* ys = gg + T * K;   // T*dv: dO (query side) or V (key side)
    float* dd = ys + T * dv;  // T: D_i
    float* aa = dd + T;       // T: a_i
    const int LR = dr + 1, LV = dv + 1;
    float* mT = aa + T;           // FAST: [K][LR] mu
    float* iT = mT + K * LR;      // FAST: [K][LR] 1 / sigma2
    float* cT = iT + K * LR;      // FAST: [K] score constants
    float* Ml = cT + K;           // FAST: [K][LV] the memory (or its gradient)
    float* Zl = Ml + K * LV;      // FAST: [K] its Z column
    const double *ch = c + size_t(h) * K, *ih = inv + size_t(h) * K * dr;
    const float* mh = mu + size_t(h) * K * dr;
    const float* Vg = mem + size_t(p) * K * (dv + 1);  // [K][dv], then Z (or dVt, dZ)
    const bool ML = FAST && mem_lds;
    const float* Vt = ML ? Ml : Vg;
    const float* Z = ML ? Zl : Vg + size_t(K) * dv;
    const int SV = ML ? LV : dv;
    if (FAST) {
        for (int i = threadIdx.x; i < K * dr; i += kThreads) {
            const int k = i / dr, d = i - k * dr;
            mT[k * LR + d] = mh[i];
            iT[k * LR + d] = float(ih[i]);
        }
        for (int k = threadIdx.x; k < K; k += kThreads) {
            cT[k] = float(ch[k]);
            if (ML) Zl[k] = Vg[K * dv + k];
        }
        if (ML)
            for (int i = threadIdx.x; i < K * dv; i += kThreads) Ml[(i / dv) * LV + i % dv] = Vg[i];
        __syncthreads();
    }
    const int E = K * (dv + 1), PE = 2 * K * dr + K;
    float* mp = mem_part ? mem_part + (size_t(p) * G + gi) * E : nullptr;
    float* pp = param_part + (size_t(p) * G + gi) * PE;
    const int64_t lo = int64_t(gi) * seg, hi = min<int64_t>(lo + seg, N);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    bool first = true;
    for (int64_t n0 = lo; n0 < hi; n0 += T) {
        const int rows = int(min<int64_t>(T, hi - n0));
        if (FAST)
            gamma_tile_lds(X + p * N * dr, n0, rows, T, dr, K, cT, iT, mT, xs, gm);
        else
            gamma_tile(X + p * N * dr, n0, rows, T, dr, K, ch, ih, mh, xs, gm);
        for (int i = threadIdx.x; i < T * dv; i += kThreads) {
            const int t = i / dv;
            ys[i] = t < rows ? Y[(p * N + n0) * dv + i] : 0.0f;
        }
        __syncthreads();
        if (QUERY) {  // D_t and a_t = dO_t . O_t, one wave per row
            for (int t = wave; t < rows; t += kThreads / kWave) {
                float d = 0.0f;
                for (int k = lane; k < K; k += kWave) d = fmaf(gm[t * K + k], Z[k], d);
                d = wave_sum(d) + eps;
                float a = 0.0f;
                for (int cc = lane; cc < dv; cc += kWave) {
                    float nn = 0.0f;
                    for (int k = 0; k < K; ++k) nn = fmaf(gm[t * K + k], Vt[size_t(k) * SV + cc], nn);
                    a = fmaf(ys[t * dv + cc], nn / d, a);
                }
                a = wave_sum(a);
                if (lane == 0) {
                    dd[t] = d;
                    aa[t] = a;
                }
            }
            __syncthreads();
        } else {  // dV_tc = sum_k gamma^K_tk dVt_kc
            for (int i = threadIdx.x; i < rows * dv; i += kThreads) {
                const int t = i / dv, cc = i - t * dv;
                float acc = 0.0f;
                for (int k = 0; k < K; ++k) acc = fmaf(gm[t * K + k], Vt[size_t(k) * SV + cc], acc);
                dY[(p * N + n0) * dv + i] = acc;
            }
        }
        // upstream gradient at the responsibilities
        for (int i = threadIdx.x; i < T * K; i += kThreads) {
            const int t = i / K, k = i - t * K;
            float acc = 0.0f;
            if (t < rows) {
                for (int cc = 0; cc < dv; ++cc) acc = fmaf(ys[t * dv + cc], Vt[size_t(k) * SV + cc], acc);
                acc = QUERY ? (acc - aa[t] * Z[k]) / dd[t] : acc + Z[k];
            }
            gg[i] = acc;
        }
        __syncthreads();
        // Eq. 18: ds = gamma (g - gamma . g), one wave per row
        for (int t = wave; t < T; t += kThreads / kWave) {
            float w = 0.0f;
            for (int k = lane; k < K; k += kWave) w = fmaf(gm[t * K + k], gg[t * K + k], w);
            w = wave_sum(w);
            for (int k = lane; k < K; k += kWave) gg[t * K + k] = gm[t * K + k] * (gg[t * K + k] - w);
        }
        __syncthreads();
        // routing-vector gradient
        for (int i = threadIdx.x; i < rows * dr; i += kThreads) {
            const int t = i / dr, d = i - t * dr;
            float acc = 0.0f;
            if (FAST) {
                const float x = xs[t * dr + d];
                for (int k = 0; k < K; ++k) acc = fmaf(gg[t * K + k] * iT[k * LR + d], x - mT[k * LR + d], acc);
            } else {
                for (int k = 0; k < K; ++k)
                    acc = fmaf(gg[t * K + k], float((double(xs[t * dr + d]) - double(mh[size_t(k) * dr + d])) * ih[size_t(k) * dr + d]), acc);
            }
            dX[(p * N + n0) * dr + i] = -acc;
        }
        // moments of these rows
        for (int e = threadIdx.x; e < K * dr; e += kThreads) {
            const int k = e / dr, d = e - k * dr;
            float a1, a2;
            if (FAST) {
                const float m = mT[k * LR + d];
                a1 = 0.0f, a2 = 0.0f;
                for (int t = 0; t < rows; ++t) {
                    const float df = xs[t * dr + d] - m, w = gg[t * K + k] * df;
                    a1 += w;
                    a2 = fmaf(w, df, a2);
                }
            } else {
                const double m = double(mh[e]);
                double b1 = 0.0, b2 = 0.0;
                for (int t = 0; t < rows; ++t) {
                    const double df = double(xs[t * dr + d]) - m, w = double(gg[t * K + k]) * df;
                    b1 += w;
                    b2 += w * df;
                }
                a1 = float(b1), a2 = float(b2);
            }
            pp[e] = first ? a1 : pp[e] + a1;
            pp[K * dr + e] = first ? a2 : pp[K * dr + e] + a2;
        }
        for (int k = threadIdx.x; k < K; k += kThreads) {
            float acc = 0.0f;
            for (int t = 0; t < rows; ++t) acc += gg[t * K + k];
            pp[2 * K * dr + k] = first ? acc : pp[2 * K * dr + k] + acc;
        }
        if (QUERY) {  // partial [dVt | dZ] of these rows, in the memory's layout
            for (int e = threadIdx.x; e < E; e += kThreads) {
                float acc = 0.0f;
                if (e < K * dv) {
                    const int k = e / dv, cc = e - k * dv;
                    for (int t = 0; t < rows; ++t) acc = fmaf(gm[t * K + k], ys[t * dv + cc] / dd[t], acc);
                } else {
                    const int k = e - K * dv;
                    for (int t = 0; t < rows; ++t) acc -= gm[t * K + k] * aa[t] / dd[t];
                }
                mp[e] = first ? acc : mp[e] + acc;
            }
        }
        first = false;
        __syncthreads();  // the tile's LDS is free
    }
    if (first) {  // empty block
        for (int e = threadIdx.x; e < PE; e += kThreads) pp[e] = 0.0f;
        if (QUERY)
            for (int e = threadIdx.x; e < E; e += kThreads) mp[e] = 0.0f;
    }
}

// ---- register-tiled passes for K, d_r, d_v <= 64 (multiples of 4)
// 16 row groups of 64 / TW threads: a thread owns rows r0 .. r0 + 3 and columns m0 .. m0 + TW - 1
// of every 64 x 64 product of a tile (1024 / TW threads; TW = 2 gives eight waves, two per SIMD
// where the LDS allows one workgroup per CU).  Row operands are read from LDS as 16-byte vectors,
// column operands as TW-wide ones.  The threads of a row group are adjacent lanes of one wave, so
// row reductions are shuffles within the group.
constexpr int kBT = 64;        // rows per tile
constexpr int kLDT = kBT + 4;  // row stride of the transposed ([L][T]) tiles
// BWD_CQUERY / BWD_CKEY: the causal passes (the memory a tile sees is the running prefix or
// suffix, plus the masked in-tile products)
enum { BWD_WRITE = 0, BWD_QUERY = 1, BWD_KEY = 2, BWD_CQUERY = 3, BWD_CKEY = 4 };
constexpr int kTiledTW = 2;  // register tile width of these passes (eight waves)

bool bwd_tiled_applies(const Plan& p) {
    return p.K % 4 == 0 && p.dr % 4 == 0 && p.dv % 4 == 0 && p.K <= 64 && p.dr <= 64 && p.dv <= 64;
}

size_t bwd_tiled_lds_bytes(int mode, int K, int dr, int dv) {
    const bool qk = mode != BWD_WRITE, causal = mode >= BWD_CQUERY;
    const bool qside = mode == BWD_QUERY || mode == BWD_CQUERY, kside = mode == BWD_KEY || mode == BWD_CKEY;
    size_t f = size_t(2 * dr * (K + 4) + K);                 // mu^T, (1/sigma2)^T, c
    if (qk) f += size_t(2 * K * dv + K);                     // memory (or its gradient), transposed, and Z
    if (qk) f += size_t(dr * kLDT) + size_t(K * kLDT) + size_t(kBT * K);  // X^T, gamma^T (then ds^T), gamma (then ds)
    else f += size_t(max(dr * kLDT, kBT * K));               // X^T, then gamma in the same space
    if (!kside) f += size_t(kBT * dv);                       // V (write) or dO / D (query)
    if (qk) f += size_t(dv * kLDT);                          // (dO / D)^T (query) or V^T (key)
    if (qside || causal) f += 2 * kBT;                       // D, a'
    if (causal)  // the other side's gamma in both layouts, V (query) or dO / D (key) rows, C and A
        f += size_t(kBT * (K + 4) + K * kLDT + kBT * (dv + 4) + kBT * kLDT * (qside ? 1 : 2));
    return f * sizeof(float);
}

__device__ __forceinline__ float4 lds4(const float* q) { return *reinterpret_cast<const float4*>(q); }
__device__ __forceinline__ void put4(float* q, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(q) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void unpack(const float4 v, float (&a)[4]) {
    a[0] = v.x, a[1] = v.y, a[2] = v.z, a[3] = v.w;
}
// TW columns of a row read from LDS (TW = 2 or 4, 8- or 16-byte aligned).
template <int TW>
__device__ __forceinline__ void ldsw(const float* q, float (&a)[TW]) {
    if constexpr (TW == 4) {
        const float4 v = *reinterpret_cast<const float4*>(q);
        a[0] = v.x, a[1] = v.y, a[2] = v.z, a[3] = v.w;
    } else {
        const float2 v = *reinterpret_cast<const float2*>(q);
        a[0] = v.x, a[1] = v.y;
    }
}
template <int TW>
__device__ __forceinline__ void stsw(float* q, const float (&a)[TW]) {
    if constexpr (TW == 4) *reinterpret_cast<float4*>(q) = make_float4(a[0], a[1], a[2], a[3]);
    else *reinterpret_cast<float2*>(q) = make_float2(a[0], a[1]);
}

__device__ __forceinline__ float sum16(float v) {
    for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 16);
    return v;
}
__device__ __forceinline__ float max16(float v) {
    for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 16));
    return v;
}
// Sum and maximum over the W consecutive lanes of a row group (W = 16 or 32).
template <int W>
__device__ __forceinline__ float sum_lanes(float v) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, W);
    return v;
}
template <int W>
__device__ __forceinline__ float max_lanes(float v) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, W));
    return v;
}

// Responsibilities of the tile in xT (rows t = r0 + i, columns k = m0 + j, j < TW):
// the direct-form score of Eq. 16 from the LDS tables, then the softmax of Eq. 3b over the
// 64 / TW lanes of the row group.  Rows at or beyond `rows` get zeros.
template <int TW>
__device__ __forceinline__ void tile_gamma(const float* xT, const float* muT, const float* ivT, const float* cK,
                                           int K, int dr, int LDK, int r0, int m0, int rows, float (&gam)[4][TW]) {
    constexpr int CG = 64 / TW;
    float q[4][TW] = {};
    if (m0 < K) {
#pragma unroll 4
        for (int d = 0; d < dr; ++d) {
            float xa[4], ma[TW], ia[TW];
            unpack(lds4(xT + d * kLDT + r0), xa);
            ldsw<TW>(muT + d * LDK + m0, ma);
            ldsw<TW>(ivT + d * LDK + m0, ia);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < TW; ++j) {
                    const float df = xa[i] - ma[j];
                    q[i][j] = fmaf(df * df, ia[j], q[i][j]);
                }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float sc[TW], m = -INFINITY;
#pragma unroll
        for (int j = 0; j < TW; ++j) {
            sc[j] = m0 < K ? cK[m0 + j] - 0.5f * q[i][j] : -INFINITY;
            m = fmaxf(m, sc[j]);
        }
        m = max_lanes<CG>(m);
        float e[TW], sum = 0.0f;
#pragma unroll
        for (int j = 0; j < TW; ++j) {
            e[j] = m0 < K ? expf(sc[j] - m) : 0.0f;
            sum += e[j];
        }
        sum = sum_lanes<CG>(sum);
        const float r = r0 + i < rows ? 1.0f / sum : 0.0f;
#pragma unroll
        for (int j = 0; j < TW; ++j) gam[i][j] = e[j] * r;
    }
}

// The 4 x TW responsibility block (rows r0.., components m0..) of the tile at n0 from a cache
// [.][K] (zeros beyond `rows` or K), and its store.
template <int TW>
__device__ __forceinline__ void gamma_from(const float* Gp, int64_t n0, int rows, int K, int r0, int m0,
                                           float (&gam)[4][TW]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool ok = m0 < K && r0 + i < rows;
        if (ok) ldsw<TW>(Gp + (n0 + r0 + i) * K + m0, gam[i]);
        else
#pragma unroll
            for (int j = 0; j < TW; ++j) gam[i][j] = 0.0f;
    }
}
template <int TW>
__device__ __forceinline__ void gamma_to(float* Gp, int64_t n0, int rows, int K, int r0, int m0,
                                         const float (&gam)[4][TW]) {
    if (m0 < K)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (r0 + i < rows) stsw<TW>(Gp + (n0 + r0 + i) * K + m0, gam[i]);
}

// Load rows [n0, n0 + rows) of X [.][dr] into xT [dr][kLDT] (zeros beyond `rows`) with NTH threads.
template <int NTH = kThreads>
__device__ __forceinline__ void load_xT(const float* Xp, int64_t n0, int rows, int dr, float* xT) {
    for (int i = threadIdx.x; i < kBT * (dr / 4); i += NTH) {
        const int t = i / (dr / 4), d = (i - t * (dr / 4)) * 4;
        const float4 v = t < rows ? *reinterpret_cast<const float4*>(Xp + (n0 + t) * dr + d) : make_float4(0, 0, 0, 0);
        xT[(d + 0) * kLDT + t] = v.x;
        xT[(d + 1) * kLDT + t] = v.y;
        xT[(d + 2) * kLDT + t] = v.z;
        xT[(d + 3) * kLDT + t] = v.w;
    }
}

// Grid (G, P), one split of one problem per workgroup.
//   WRITE: X = X_K, Y = V; mem_part gets the split's [Vt | Z] (the forward's memory, Eq. 5-6).
//   QUERY: X = X_Q, Y = dO, mem = [Vt | Z]; writes dX_Q, mem_part gets the split's [dVt | dZ].
//   KEY:   X = X_K, Y = V, mem = [dVt | dZ]; writes dX_K and dY = dV.
// QUERY and KEY write the split's moment record to param_part.
//   CQUERY, CKEY: the causal passes over segment g of problem p.  X2 holds the other side's routing
//   vectors (CQUERY: X_K, CKEY: X_Q) and Y2 the other side's rows (CQUERY: V, CKEY: dO); mem is the
//   per-segment record [P][G][K (dv + 1)] of the memory before the segment (CQUERY) or of what the
//   later segments' queries send (CKEY), advanced in LDS tile by tile.  CQUERY writes D_i and a_i
//   of its rows to rowda and the segment's total of what its queries send to mem_part; CKEY reads
//   rowda.
// Responsibility cache ([P][N][K] fp32, or NULL): gsave receives this pass's own responsibilities,
// gload supplies them instead of the score loop, goload supplies the other side's (causal).
// A cached value is the one the score loop would compute, so the results do not change.
template <int MODE, int TW>
__global__ void __launch_bounds__(1024 / TW)
    f32_bwd_tiled_kernel(const float* __restrict__ X, const float* __restrict__ Y, int64_t N, int H, int dr, int dv,
                         int K, int64_t seg, int G, const double* __restrict__ c, const double* __restrict__ inv,
                         const float* __restrict__ mu, const float* __restrict__ mem, float eps,
                         float* __restrict__ dX, float* __restrict__ dY, float* __restrict__ mem_part,
                         float* __restrict__ param_part, const float* __restrict__ X2, const float* __restrict__ Y2,
                         float* __restrict__ rowda, float* __restrict__ gsave, const float* __restrict__ gload,
                         const float* __restrict__ goload) {
    constexpr bool QK = MODE != BWD_WRITE, CAUSAL = MODE >= BWD_CQUERY;
    constexpr bool QS = MODE == BWD_QUERY || MODE == BWD_CQUERY, KS = MODE == BWD_KEY || MODE == BWD_CKEY;
    constexpr int NTH = 1024 / TW, CG = 64 / TW;  // threads; column groups of a row group
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int gi = blockIdx.x, h = int(p % H);
    const int tid = threadIdx.x, r0 = (tid / CG) * 4, m0 = (tid % CG) * TW;
    const int LDK = K + 4;
    float* muT = lds;                              // [dr][LDK]
    float* ivT = muT + dr * LDK;                   // [dr][LDK]
    float* cK = ivT + dr * LDK;                    // [K]
    float* M = cK + K;                             // [K][dv]   Vt (query) or dVt (key)
    float* MT = M + (QK ? K * dv : 0);             // [dv][K]
    float* Zm = MT + (QK ? dv * K : 0);            // [K]       Z or dZ
    float* xT = Zm + (QK ? K : 0);                 // [dr][kLDT]
    float* gT = xT + dr * kLDT;                    // [K][kLDT] gamma^T, then ds^T
    float* g = QK ? gT + K * kLDT : xT;            // [kBT][K]  gamma, then ds (write: in the space of X^T)
    float* Yr = QK ? g + kBT * K : xT + max(dr * kLDT, kBT * K);  // [kBT][dv] V (write) or dO / D (query)
    float* YT = Yr + (!KS ? kBT * dv : 0);         // [dv][kLDT]
    float* Dv = YT + (QK ? dv * kLDT : 0);         // [kBT]
    float* Av = Dv + kBT;                          // [kBT]
    const int LG = K + 4, LV4 = dv + 4;
    float* Go = Av + kBT;                          // causal: [kBT][LG] the other side's gamma
    float* GoT = Go + kBT * LG;                    // causal: [K][kLDT] the same, transposed
    float* Rw = GoT + K * kLDT;                    // causal: [kBT][LV4] V (query) or dO / D (key) rows
    float* Cm = Rw + kBT * LV4;                    // causal: query: C^T, then A^T; key: C ([i][j], stride kLDT)
    float* Am = Cm + kBT * kLDT;                   // causal key: A ([i][j], stride kLDT)

    {   // per-head tables and (query, key) the problem's memory: each thread's 16-byte loads are
        // issued together, then stored (K, d_r, d_v <= 64 and multiples of 4, so every 4-element
        // group lies in one row and starts on a 16-byte boundary)
        constexpr int PER = 64 * 64 / 4 / NTH;  // 4-element groups per thread at K = d = 64
        const double *ch = c + size_t(h) * K, *ih = inv + size_t(h) * K * dr;
        const float* mh = mu + size_t(h) * K * dr;
        const float* src = QK ? mem + (CAUSAL ? size_t(p) * G + gi : size_t(p)) * K * (dv + 1) : nullptr;
        float4 tm[PER], tmem[PER];
        double2 tv[PER][2];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = 4 * (tid + u * NTH);
            if (e < K * dr) {
                tm[u] = *reinterpret_cast<const float4*>(mh + e);
                tv[u][0] = *reinterpret_cast<const double2*>(ih + e);
                tv[u][1] = *reinterpret_cast<const double2*>(ih + e + 2);
            }
            if (QK && e < K * dv) tmem[u] = *reinterpret_cast<const float4*>(src + e);
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = 4 * (tid + u * NTH);
            if (e < K * dr) {
                const int k = e / dr, d = e - k * dr;
                muT[(d + 0) * LDK + k] = tm[u].x;
                muT[(d + 1) * LDK + k] = tm[u].y;
                muT[(d + 2) * LDK + k] = tm[u].z;
                muT[(d + 3) * LDK + k] = tm[u].w;
                ivT[(d + 0) * LDK + k] = float(tv[u][0].x);
                ivT[(d + 1) * LDK + k] = float(tv[u][0].y);
                ivT[(d + 2) * LDK + k] = float(tv[u][1].x);
                ivT[(d + 3) * LDK + k] = float(tv[u][1].y);
            }
            if (QK && e < K * dv) {
                const int k = e / dv, cc = e - k * dv;
                *reinterpret_cast<float4*>(M + e) = tmem[u];
                MT[(cc + 0) * K + k] = tmem[u].x;
                MT[(cc + 1) * K + k] = tmem[u].y;
                MT[(cc + 2) * K + k] = tmem[u].z;
                MT[(cc + 3) * K + k] = tmem[u].w;
            }
        }
        for (int k = tid; k < K; k += NTH) cK[k] = float(ch[k]);
        if (QK)
            for (int k = tid; k < K; k += NTH) Zm[k] = src[K * dv + k];
    }
    __syncthreads();
    // moment accumulators (rows d = r0 + i, columns k = m0 + j) and their mu
    float mreg[4][TW], s1[4][TW] = {}, s2[4][TW] = {}, s0[TW] = {};
    // memory-like accumulators (rows k = r0 + i, columns c = m0 + j): Vt, Z (write) or dVt, dZ (query)
    float mv[4][TW] = {}, mz[4] = {};
    const bool mom = QK && r0 < dr && m0 < K;
    if (mom)
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < TW; ++j) mreg[i][j] = muT[(r0 + i) * LDK + m0 + j];

    const int64_t lo = int64_t(gi) * seg, hi = min<int64_t>(lo + seg, N);
    const float* Xp = X + size_t(p) * N * dr;
    const float* Yp = Y + size_t(p) * N * dv;
    const int ntiles = int((hi - lo + kBT - 1) / kBT);
    for (int it = 0; it < ntiles; ++it) {
        const int64_t n0 = lo + int64_t(MODE == BWD_CKEY ? ntiles - 1 - it : it) * kBT;  // the key pass runs backward
        const int rows = int(min<int64_t>(kBT, hi - n0));
        __syncthreads();  // the previous tile's reads are done
        if (CAUSAL) {  // the other side's responsibilities, in both layouts
            float go[4][TW];
            if (goload) {
                gamma_from<TW>(goload + size_t(p) * N * K, n0, rows, K, r0, m0, go);
            } else {
                load_xT<NTH>(X2 + size_t(p) * N * dr, n0, rows, dr, xT);
                __syncthreads();
                tile_gamma<TW>(xT, muT, ivT, cK, K, dr, LDK, r0, m0, rows, go);
            }
            if (m0 < K) {
#pragma unroll
                for (int i = 0; i < 4; ++i) stsw<TW>(Go + (r0 + i) * LG + m0, go[i]);
#pragma unroll
                for (int j = 0; j < TW; ++j) put4(GoT + (m0 + j) * kLDT + r0, go[0][j], go[1][j], go[2][j], go[3][j]);
            }
            // V rows (query) or dO / D rows with D, a' (key)
            const float* Y2p = Y2 + size_t(p) * N * dv;
            for (int i = tid; i < kBT * (dv / 4); i += NTH) {
                const int t = i / (dv / 4), cc = (i - t * (dv / 4)) * 4;
                float4 v = t < rows ? *reinterpret_cast<const float4*>(Y2p + (n0 + t) * dv + cc) : make_float4(0, 0, 0, 0);
                if (MODE == BWD_CKEY && t < rows) {
                    const float rD = 1.0f / rowda[(size_t(p) * N + n0 + t) * 2];
                    v.x *= rD, v.y *= rD, v.z *= rD, v.w *= rD;
                }
                *reinterpret_cast<float4*>(Rw + t * LV4 + cc) = v;
            }
            if (MODE == BWD_CKEY)
                for (int t = tid; t < kBT; t += NTH) {
                    const float D = t < rows ? rowda[(size_t(p) * N + n0 + t) * 2] : 1.0f;
                    Dv[t] = D;
                    Av[t] = t < rows ? rowda[(size_t(p) * N + n0 + t) * 2 + 1] / D : 0.0f;
                }
            __syncthreads();  // xT is free again
        }
        load_xT<NTH>(Xp, n0, rows, dr, xT);
        for (int i = tid; i < kBT * (dv / 4); i += NTH) {
            const int t = i / (dv / 4), cc = (i - t * (dv / 4)) * 4;
            const float4 v = t < rows ? *reinterpret_cast<const float4*>(Yp + (n0 + t) * dv + cc) : make_float4(0, 0, 0, 0);
            if (KS) {
                YT[(cc + 0) * kLDT + t] = v.x;
                YT[(cc + 1) * kLDT + t] = v.y;
                YT[(cc + 2) * kLDT + t] = v.z;
                YT[(cc + 3) * kLDT + t] = v.w;
            } else {
                *reinterpret_cast<float4*>(Yr + t * dv + cc) = v;
            }
        }
        __syncthreads();

        // responsibilities (rows t, columns k): direct-form score of Eq. 16, softmax of Eq. 3b
        float gam[4][TW];
        if (gload)
            gamma_from<TW>(gload + size_t(p) * N * K, n0, rows, K, r0, m0, gam);
        else
            tile_gamma<TW>(xT, muT, ivT, cK, K, dr, LDK, r0, m0, rows, gam);
        if (gsave) gamma_to<TW>(gsave + size_t(p) * N * K, n0, rows, K, r0, m0, gam);
        if (MODE == BWD_WRITE) __syncthreads();  // gamma overwrites X^T
        if (m0 < K) {
            if (!KS)
#pragma unroll
                for (int i = 0; i < 4; ++i) stsw<TW>(g + (r0 + i) * K + m0, gam[i]);
            if (QK)
#pragma unroll
                for (int j = 0; j < TW; ++j) put4(gT + (m0 + j) * kLDT + r0, gam[0][j], gam[1][j], gam[2][j], gam[3][j]);
        }
        __syncthreads();

        if (MODE == BWD_WRITE) {  // Vt += gamma^T V, Z += gamma^T 1 (rows k, columns c)
            if (r0 < K && m0 < dv)
#pragma unroll 4
                for (int t = 0; t < rows; ++t) {
                    float ga[4], ya[TW];
                    unpack(lds4(g + t * K + r0), ga);
                    ldsw<TW>(Yr + t * dv + m0, ya);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        mz[i] += ga[i];
#pragma unroll
                        for (int j = 0; j < TW; ++j) mv[i][j] = fmaf(ga[i], ya[j], mv[i][j]);
                    }
                }
            continue;
        }

        // causal: C_ij = gamma^Q_i . gamma^K_j for key j <= query i (rows i = r0.., columns j = m0..);
        // the query pass keeps C^T and its row sums, the key pass C and A_ij = dO'_i . V_j - a'_i
        float cs[4] = {};
        if (CAUSAL) {
            const float* gqT = QS ? gT : GoT;  // [K][kLDT] gamma^Q transposed
            const float* gkT = QS ? GoT : gT;  // [K][kLDT] gamma^K transposed
            float ca[4][TW] = {}, aa[4][TW] = {};
            const bool live = m0 <= r0 + 3 && r0 < rows;  // the block has entries with j <= i
            if (live) {
#pragma unroll 4
                for (int k = 0; k < K; ++k) {
                    float qa[4], ka[TW];
                    unpack(lds4(gqT + k * kLDT + r0), qa);
                    ldsw<TW>(gkT + k * kLDT + m0, ka);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < TW; ++j) ca[i][j] = fmaf(qa[i], ka[j], ca[i][j]);
                }
                if (MODE == BWD_CKEY) {
#pragma unroll 4
                    for (int cc = 0; cc < dv; ++cc) {
                        float va[TW], oa[4];
                        ldsw<TW>(YT + cc * kLDT + m0, va);  // V^T
#pragma unroll
                        for (int i = 0; i < 4; ++i) oa[i] = Rw[(r0 + i) * LV4 + cc];  // dO'
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < TW; ++j) aa[i][j] = fmaf(oa[i], va[j], aa[i][j]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < TW; ++j) {
                    const bool in = live && m0 + j <= r0 + i && r0 + i < rows;
                    ca[i][j] = in ? ca[i][j] : 0.0f;
                    aa[i][j] = in ? aa[i][j] - Av[r0 + i] : 0.0f;
                    cs[i] += ca[i][j];
                }
            if (QS) {
#pragma unroll
                for (int j = 0; j < TW; ++j) put4(Cm + (m0 + j) * kLDT + r0, ca[0][j], ca[1][j], ca[2][j], ca[3][j]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    stsw<TW>(Cm + (r0 + i) * kLDT + m0, ca[i]);
                    stsw<TW>(Am + (r0 + i) * kLDT + m0, aa[i]);
                }
            }
            __syncthreads();
        }
        const int tmax = min(r0 + 4, rows);  // causal: in-tile keys j <= the block's last query row

        float gg[4][TW] = {};  // upstream gradient at the responsibilities (rows t, columns k)
        if (QS) {
            // N = gamma Vt (rows t, columns c); D = gamma Z + eps; dO . N
            float nv[4][TW] = {};
            if (m0 < dv)
#pragma unroll 4
                for (int k = 0; k < K; ++k) {
                    float ga[4], va[TW];
                    unpack(lds4(gT + k * kLDT + r0), ga);
                    ldsw<TW>(M + k * dv + m0, va);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < TW; ++j) nv[i][j] = fmaf(ga[i], va[j], nv[i][j]);
                }
            if (CAUSAL && m0 < dv)  // + sum_{j <= t} C_tj V_j
                for (int j = 0; j < tmax; ++j) {
                    float ca[4], va[TW];
                    unpack(lds4(Cm + j * kLDT + r0), ca);
                    ldsw<TW>(Rw + j * LV4 + m0, va);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int jj = 0; jj < TW; ++jj) nv[i][jj] = fmaf(ca[i], va[jj], nv[i][jj]);
                }
            float Dt[4], An[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float dp = cs[i], ap = 0.0f;
                if (m0 < K)
#pragma unroll
                    for (int j = 0; j < TW; ++j) dp = fmaf(gam[i][j], Zm[m0 + j], dp);
                if (m0 < dv) {
                    float ya[TW];
                    ldsw<TW>(Yr + (r0 + i) * dv + m0, ya);
#pragma unroll
                    for (int j = 0; j < TW; ++j) ap = fmaf(ya[j], nv[i][j], ap);
                }
                Dt[i] = sum_lanes<CG>(dp) + eps;
                An[i] = sum_lanes<CG>(ap);
            }
            // dO' = dO / D in both layouts (each thread rescales its own entries), D and a' = dO . N / D^2
            float sy[4][TW];
            if (m0 < dv) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float ya[TW];
                    ldsw<TW>(Yr + (r0 + i) * dv + m0, ya);
                    const float rD = 1.0f / Dt[i];
#pragma unroll
                    for (int j = 0; j < TW; ++j) sy[i][j] = ya[j] * rD;
                    stsw<TW>(Yr + (r0 + i) * dv + m0, sy[i]);
                }
#pragma unroll
                for (int j = 0; j < TW; ++j) put4(YT + (m0 + j) * kLDT + r0, sy[0][j], sy[1][j], sy[2][j], sy[3][j]);
            }
            if (m0 == 0)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Dv[r0 + i] = Dt[i];
                    Av[r0 + i] = An[i] / (Dt[i] * Dt[i]);
                    if (CAUSAL && r0 + i < rows) {
                        rowda[(size_t(p) * N + n0 + r0 + i) * 2 + 0] = Dt[i];
                        rowda[(size_t(p) * N + n0 + r0 + i) * 2 + 1] = An[i] / Dt[i];
                    }
                }
            __syncthreads();
            // causal: A^T (A_tj = dO'_t . V_j - a'_t for j <= t) over C^T, whose reads are done
            if (CAUSAL) {
                float aa[4][TW] = {};
                const bool live = m0 <= r0 + 3 && r0 < rows;
                if (live)
#pragma unroll 4
                    for (int cc = 0; cc < dv; ++cc) {
                        float oa[4], va[4];
                        unpack(lds4(YT + cc * kLDT + r0), oa);  // dO'^T
#pragma unroll
                        for (int j = 0; j < TW; ++j) va[j] = Rw[(m0 + j) * LV4 + cc];  // V
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < TW; ++j) aa[i][j] = fmaf(oa[i], va[j], aa[i][j]);
                    }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j)
                        aa[i][j] = live && m0 + j <= r0 + i && r0 + i < rows ? aa[i][j] - Av[r0 + i] : 0.0f;
#pragma unroll
                for (int j = 0; j < TW; ++j) put4(Cm + (m0 + j) * kLDT + r0, aa[0][j], aa[1][j], aa[2][j], aa[3][j]);
            }
            // dVt += gamma^T dO', dZ -= gamma^T a' (rows k, columns c)
            if (r0 < K && m0 < dv)
#pragma unroll 4
                for (int t = 0; t < rows; ++t) {
                    float ga[4], ya[TW];
                    unpack(lds4(g + t * K + r0), ga);
                    ldsw<TW>(Yr + t * dv + m0, ya);
                    const float at = Av[t];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        mz[i] = fmaf(-ga[i], at, mz[i]);
#pragma unroll
                        for (int j = 0; j < TW; ++j) mv[i][j] = fmaf(ga[i], ya[j], mv[i][j]);
                    }
                }
            // g = dO' Vt^T - a' Z
            if (m0 < K) {
#pragma unroll 4
                for (int cc = 0; cc < dv; ++cc) {
                    float ya[4], va[TW];
                    unpack(lds4(YT + cc * kLDT + r0), ya);
                    ldsw<TW>(MT + cc * K + m0, va);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < TW; ++j) gg[i][j] = fmaf(ya[i], va[j], gg[i][j]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) gg[i][j] = fmaf(-Av[r0 + i], Zm[m0 + j], gg[i][j]);
            }
            if (CAUSAL) {  // + sum_{j <= t} A_tj gamma^K_j
                __syncthreads();
                if (m0 < K)
                    for (int j = 0; j < tmax; ++j) {
                        float ta[4], ka[TW];
                        unpack(lds4(Cm + j * kLDT + r0), ta);
                        ldsw<TW>(Go + j * LG + m0, ka);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int jj = 0; jj < TW; ++jj) gg[i][jj] = fmaf(ta[i], ka[jj], gg[i][jj]);
                    }
            }
        } else {
            // dV = gamma dVt (rows t, columns c)
            if (m0 < dv) {
                float nv[4][TW] = {};
#pragma unroll 4
                for (int k = 0; k < K; ++k) {
                    float ga[4], va[TW];
                    unpack(lds4(gT + k * kLDT + r0), ga);
                    ldsw<TW>(M + k * dv + m0, va);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < TW; ++j) nv[i][j] = fmaf(ga[i], va[j], nv[i][j]);
                }
                if (CAUSAL)  // + sum_{i >= j} C_ij dO'_i (rows j = r0.., queries i >= r0)
                    for (int i2 = r0; i2 < rows; ++i2) {
                        float ca[4], oa[TW];
                        unpack(lds4(Cm + i2 * kLDT + r0), ca);
                        ldsw<TW>(Rw + i2 * LV4 + m0, oa);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < TW; ++j) nv[i][j] = fmaf(ca[i], oa[j], nv[i][j]);
                    }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (r0 + i < rows)
                        stsw<TW>(dY + (size_t(p) * N + n0 + r0 + i) * dv + m0, nv[i]);
            }
            // g = V dVt^T + dZ
            if (m0 < K) {
#pragma unroll 4
                for (int cc = 0; cc < dv; ++cc) {
                    float ya[4], va[TW];
                    unpack(lds4(YT + cc * kLDT + r0), ya);
                    ldsw<TW>(MT + cc * K + m0, va);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < TW; ++j) gg[i][j] = fmaf(ya[i], va[j], gg[i][j]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) gg[i][j] += Zm[m0 + j];
                if (CAUSAL)  // + sum_{i >= j} A_ij gamma^Q_i
                    for (int i2 = r0; i2 < rows; ++i2) {
                        float ta[4], qa[TW];
                        unpack(lds4(Am + i2 * kLDT + r0), ta);
                        ldsw<TW>(Go + i2 * LG + m0, qa);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < TW; ++j) gg[i][j] = fmaf(ta[i], qa[j], gg[i][j]);
                    }
            }
        }
        // Eq. 18: ds = gamma (g - gamma . g)
        float ds[4][TW];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float w = 0.0f;
#pragma unroll
            for (int j = 0; j < TW; ++j) w = fmaf(gam[i][j], gg[i][j], w);
            w = sum_lanes<CG>(w);
#pragma unroll
            for (int j = 0; j < TW; ++j) ds[i][j] = gam[i][j] * (gg[i][j] - w);
        }
        __syncthreads();  // every read of gamma is done
        if (m0 < K) {
#pragma unroll
            for (int i = 0; i < 4; ++i) stsw<TW>(g + (r0 + i) * K + m0, ds[i]);
#pragma unroll
            for (int j = 0; j < TW; ++j) put4(gT + (m0 + j) * kLDT + r0, ds[0][j], ds[1][j], ds[2][j], ds[3][j]);
        }
        __syncthreads();
        // dX (rows d, columns t): dx_td = -sum_k ds_tk (x_td - mu_kd) / sigma2_kd
        if (r0 < dr) {
            float xa[4][TW], acc[4][TW] = {};
#pragma unroll
            for (int i = 0; i < 4; ++i) ldsw<TW>(xT + (r0 + i) * kLDT + m0, xa[i]);
#pragma unroll 4
            for (int k = 0; k < K; ++k) {
                float da[TW], ma[4], ia[4];
                ldsw<TW>(gT + k * kLDT + m0, da);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ma[i] = muT[(r0 + i) * LDK + k];
                    ia[i] = ivT[(r0 + i) * LDK + k];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) acc[i][j] = fmaf(da[j] * ia[i], xa[i][j] - ma[i], acc[i][j]);
            }
#pragma unroll
            for (int j = 0; j < TW; ++j)
                if (m0 + j < rows)
                    *reinterpret_cast<float4*>(dX + (size_t(p) * N + n0 + m0 + j) * dr + r0) =
                        make_float4(-acc[0][j], -acc[1][j], -acc[2][j], -acc[3][j]);
        }
        // moments (rows d, columns k)
        if (mom)
#pragma unroll 4
            for (int t = 0; t < rows; ++t) {
                float da[TW], xa[4];
                ldsw<TW>(g + t * K + m0, da);
#pragma unroll
                for (int i = 0; i < 4; ++i) xa[i] = xT[(r0 + i) * kLDT + t];
#pragma unroll
                for (int j = 0; j < TW; ++j) s0[j] += da[j];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) {
                        const float df = xa[i] - mreg[i][j], w = da[j] * df;
                        s1[i][j] += w;
                        s2[i][j] = fmaf(w, df, s2[i][j]);
                    }
            }
        if (CAUSAL && r0 < K && m0 < dv) {
            // advance the memory past the tile (its last reads were before the ds barriers):
            // query: + gamma^K^T [V | 1] (Eq. 6b); key: + gamma^Q^T [dO' | -a']
            float ua[4][TW] = {}, uz[4] = {};
            for (int t = 0; t < rows; ++t) {
                float ga[4], ya[TW];
                unpack(lds4(Go + t * LG + r0), ga);
                ldsw<TW>(Rw + t * LV4 + m0, ya);
                const float zt = QS ? 1.0f : -Av[t];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uz[i] = fmaf(ga[i], zt, uz[i]);
#pragma unroll
                    for (int j = 0; j < TW; ++j) ua[i][j] = fmaf(ga[i], ya[j], ua[i][j]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float mm[TW];
                ldsw<TW>(M + (r0 + i) * dv + m0, mm);
#pragma unroll
                for (int j = 0; j < TW; ++j) mm[j] += ua[i][j];
                stsw<TW>(M + (r0 + i) * dv + m0, mm);
#pragma unroll
                for (int j = 0; j < TW; ++j) MT[(m0 + j) * K + r0 + i] = mm[j];
                if (m0 == 0) Zm[r0 + i] += uz[i];
            }
        }
    }
    // the split's records (zeros for a split without rows)
    if (!KS && r0 < K && m0 < dv) {
        float* mp = mem_part + (size_t(p) * G + gi) * size_t(K) * (dv + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            stsw<TW>(mp + (r0 + i) * dv + m0, mv[i]);
        if (m0 == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) mp[K * dv + r0 + i] = mz[i];
    }
    if (mom) {
        float* pp = param_part + (size_t(p) * G + gi) * size_t(2 * K * dr + K);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                pp[(m0 + j) * dr + r0 + i] = s1[i][j];
                pp[K * dr + (m0 + j) * dr + r0 + i] = s2[i][j];
            }
        if (r0 == 0)
#pragma unroll
            for (int j = 0; j < TW; ++j) pp[2 * K * dr + m0 + j] = s0[j];
    }
}

// Grid (ceil((K d_r + K) / kThreads), H): the parameter gradients of head h from the moments,
// summed in fp64 over the query and key sides, the batch and the splits in that fixed order.
// With B == 0 it writes zeros (no rows, no gradient) and reads neither moments nor tables.
__global__ void __launch_bounds__(kThreads)
    f32_bwd_param_reduce_kernel(const float* __restrict__ part, int B, int H, int G, int K, int dr,
                                const double* __restrict__ inv, const float* __restrict__ pi,
                                float* __restrict__ dmu, float* __restrict__ ds2, float* __restrict__ dpi) {
    const int h = blockIdx.y, PE = 2 * K * dr + K;
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= K * dr + K) return;
    const size_t P = size_t(B) * H;
    const int k = e < K * dr ? e / dr : e - K * dr;
    const int i1 = e < K * dr ? e : 2 * K * dr + k;  // S1 (or S0 for dpi)
    // records in (side, b, g) order, loads issued eight records at a time, sums in that order
    double s1 = 0.0, s2 = 0.0, s0 = 0.0;
    const int R = 2 * B * G;
    for (int r = 0; r < R; r += 8) {
        float v1[8], v2[8], v0[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            v1[u] = v2[u] = v0[u] = 0.0f;
            const int q = r + u;
            if (q < R) {
                const int side = q / (B * G), b = (q / G) % B, g = q % G;
                const float* rec = part + ((side * P + size_t(b) * H + h) * G + g) * PE;
                v1[u] = rec[i1];
                if (e < K * dr) {
                    v2[u] = rec[K * dr + e];
                    v0[u] = rec[2 * K * dr + k];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            s1 += double(v1[u]);
            s2 += double(v2[u]);
            s0 += double(v0[u]);
        }
    }
    if (e < K * dr) {
        const double iv = B > 0 ? inv[size_t(h) * K * dr + e] : 0.0;
        dmu[size_t(h) * K * dr + e] = float(iv * s1);
        ds2[size_t(h) * K * dr + e] = float(0.5 * (iv * iv * s2 - iv * s0));
    } else {
        dpi[size_t(h) * K + k] = B > 0 ? float(s1 / double(pi[size_t(h) * K + k])) : 0.0f;
    }
}

hipError_t reduce_params(const Plan& p, const float* part, int B, const double* inv, const float* pi, float* dmu,
                         float* ds2, float* dpi, hipStream_t st) {
    const int n = int(p.K * p.dr + p.K);
    GMA_LAUNCH("f32_bwd_params", f32_bwd_param_reduce_kernel, dim3(unsigned((n + kThreads - 1) / kThreads), unsigned(p.H)),
               dim3(kThreads), 0, st, part, B, int(p.H), int(p.G), int(p.K), int(p.dr), inv, pi, dmu, ds2, dpi);
    return hipGetLastError();
}

// ---- K-blocked passes of the bidirectional backward (64 < K <= 256; d_r, d_v <= 64, multiples
// of 4): 64 x 64 products over 16 row groups of 4 x TW register blocks (1024 / TW threads; TW = 2
// keeps two waves per SIMD where the LDS allows one workgroup per CU), the components taken in
// blocks of 64.  Row passes (one workgroup per split) compute each side's responsibilities for all K
// from the LDS tables of one block at a time, cache them ([P][N][K] fp32) and form the per-row
// sums over every component; block passes (one workgroup per split and component block) read
// the cached responsibilities and produce what each component owns: the moments, the memory
// gradient and the block's share of dX, summed over the blocks afterwards in block order.
// The sums over all components that Eq. 18 needs reduce to per-row closed forms:
//   query: sum_k gamma_ik g_ik = dO'_i . N_i - a'_i (D_i - eps) = eps a'_i,
//   key:   sum_k gamma_jk g_jk = V_j . dV_j + sum_k gamma_jk dZ_k,
// with N_i = gamma^Q_i Vt, D_i = gamma^Q_i Z + eps, dO'_i = dO_i / D_i and a'_i = dO_i . N_i / D_i^2.
constexpr int kKB = 64;          // components per block
constexpr int kLB = kKB + 4;     // row stride of [.][block] LDS arrays

int kb_blocks(int64_t K) { return int((K + kKB - 1) / kKB); }

// Responsibilities of rows [n0, n0 + rows) of one problem for all K components: the direct-form
// score of Eq. 16 from fp32 tables of one block at a time, then the softmax of Eq. 3b over all
// blocks (row maximum and sum over the lanes of the row group).  Into S ([64][LK], zero past
// `rows` and K) and the cache rows gc ([.][K] of this problem).  LDS: xT [dr][kLDT], muT and ivT
// [dr][kLB], cB [kKB].
// One component block's score tables (mu and 1 / sigma2 of components k0 .. k0 + 63, d_r <= 64)
// on their way from the head's rows to LDS ([dr][kLB], transposed): each thread issues all its
// 16-byte loads before any is needed, so the loads of the next block can be in flight while the
// current block is scored.
template <int NTH>
struct KbTables {
    static constexpr int PER = kKB * 64 / 4 / NTH;  // 4-element groups per thread at d_r = 64
    float4 m[PER];
    double2 v[PER][2];
    __device__ __forceinline__ void load(const float* __restrict__ mh, const double* __restrict__ ih, int K, int dr,
                                         int k0) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = 4 * (int(threadIdx.x) + u * NTH), kl = e / dr, d = e - kl * dr, k = k0 + kl;
            if (e < kKB * dr && k < K) {
                m[u] = *reinterpret_cast<const float4*>(mh + size_t(k) * dr + d);
                v[u][0] = *reinterpret_cast<const double2*>(ih + size_t(k) * dr + d);
                v[u][1] = *reinterpret_cast<const double2*>(ih + size_t(k) * dr + d + 2);
            } else {
                m[u] = make_float4(0, 0, 0, 0);
                v[u][0] = v[u][1] = make_double2(0, 0);
            }
        }
    }
    __device__ __forceinline__ void store(float* muT, float* ivT, int dr) const {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = 4 * (int(threadIdx.x) + u * NTH), kl = e / dr, d = e - kl * dr;
            if (e < kKB * dr) {
                muT[(d + 0) * kLB + kl] = m[u].x;
                muT[(d + 1) * kLB + kl] = m[u].y;
                muT[(d + 2) * kLB + kl] = m[u].z;
                muT[(d + 3) * kLB + kl] = m[u].w;
                ivT[(d + 0) * kLB + kl] = float(v[u][0].x);
                ivT[(d + 1) * kLB + kl] = float(v[u][0].y);
                ivT[(d + 2) * kLB + kl] = float(v[u][1].x);
                ivT[(d + 3) * kLB + kl] = float(v[u][1].y);
            }
        }
    }
};

// One component block of a memory [Vt (K x dv) | Z (K)] (rows k0 .. k0 + 63, dv <= 64) on its way
// to LDS (Mb [64][dv + 4], Zb [64]), loaded ahead of its use as KbTables.
template <int NTH>
struct KbMemBlock {
    static constexpr int PER = kKB * 64 / 4 / NTH;  // 4-element groups per thread at dv = 64
    float4 m[PER];
    float z;
    __device__ __forceinline__ void load(const float* __restrict__ mp, int K, int dv, int k0) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = 4 * (int(threadIdx.x) + u * NTH), kl = e / dv, cc = e - kl * dv, k = k0 + kl;
            m[u] = (e < kKB * dv && k < K) ? *reinterpret_cast<const float4*>(mp + size_t(k) * dv + cc)
                                           : make_float4(0, 0, 0, 0);
        }
        const int k = k0 + int(threadIdx.x);
        z = (threadIdx.x < kKB && k < K) ? mp[size_t(K) * dv + k] : 0.0f;
    }
    __device__ __forceinline__ void store(float* Mb, float* Zb, int dv) const {
        const int LY = dv + 4;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = 4 * (int(threadIdx.x) + u * NTH), kl = e / dv, cc = e - kl * dv;
            if (e < kKB * dv) *reinterpret_cast<float4*>(Mb + kl * LY + cc) = m[u];
        }
        if (threadIdx.x < kKB) Zb[threadIdx.x] = z;
    }
};

template <int KB, int TW>
__device__ void kb_gamma(const float* Xp, int64_t n0, int rows, int dr, int K, const double* ch, const double* ih,
                         const float* mh, float* xT, float* muT, float* ivT, float* cB, float* S, int LK, float* gc) {
    constexpr int NTH = 1024 / TW, CG = 64 / TW;
    const int tid = threadIdx.x, r0 = (tid / CG) * 4, m0 = (tid % CG) * TW;
    KbTables<NTH> tb;
    tb.load(mh, ih, K, dr, 0);
    load_xT<NTH>(Xp, n0, rows, dr, xT);
    float mrow[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        __syncthreads();  // the previous block's tables are consumed (and xT is in place)
        tb.store(muT, ivT, dr);
        for (int kl = tid; kl < kKB; kl += NTH) cB[kl] = kb * kKB + kl < K ? float(ch[kb * kKB + kl]) : -INFINITY;
        __syncthreads();
        if (kb + 1 < KB) tb.load(mh, ih, K, dr, (kb + 1) * kKB);  // in flight while this block is scored
        float q[4][TW] = {};
#pragma unroll 4
        for (int d = 0; d < dr; ++d) {
            float xa[4], ma[TW], ia[TW];
            unpack(lds4(xT + d * kLDT + r0), xa);
            ldsw<TW>(muT + d * kLB + m0, ma);
            ldsw<TW>(ivT + d * kLB + m0, ia);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < TW; ++j) {
                    const float df = xa[i] - ma[j];
                    q[i][j] = fmaf(df * df, ia[j], q[i][j]);
                }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float s[TW];
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                s[j] = cB[m0 + j] - 0.5f * q[i][j];
                mrow[i] = fmaxf(mrow[i], s[j]);
            }
            stsw<TW>(S + (r0 + i) * LK + kb * kKB + m0, s);
        }
    }
    // each thread reads back only what it wrote: no barrier
    float rr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        mrow[i] = max_lanes<CG>(mrow[i]);
        float l = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            float* sp = S + (r0 + i) * LK + kb * kKB + m0;
            float s[TW];
            ldsw<TW>(sp, s);
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                s[j] = expf(s[j] - mrow[i]);
                l += s[j];
            }
            stsw<TW>(sp, s);
        }
        rr[i] = r0 + i < rows ? 1.0f / sum_lanes<CG>(l) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            float* sp = S + (r0 + i) * LK + kb * kKB + m0;
            float s[TW];
            ldsw<TW>(sp, s);
#pragma unroll
            for (int j = 0; j < TW; ++j) s[j] *= rr[i];
            const int k = kb * kKB + m0;
            if (r0 + i < rows) {
                if (K % TW == 0) {  // k < K covers the TW columns
                    if (k < K) stsw<TW>(gc + (n0 + r0 + i) * K + k, s);
                } else {
#pragma unroll
                    for (int j = 0; j < TW; ++j)
                        if (k + j < K) gc[(n0 + r0 + i) * K + k + j] = s[j];
                }
            }
            stsw<TW>(sp, s);
        }
    __syncthreads();
}

// Responsibilities [t][k0 .. k0 + 63] of the tile's rows from the cache rows gc ([.][K]) into Gb
// ([64][kLB]), zero past `rows` and K; 16-byte loads when K is a multiple of 4.
__device__ __forceinline__ void load_gamma_block(const float* __restrict__ gc, int64_t n0, int rows, int K, int k0,
                                                 float* Gb) {
    if ((K & 3) == 0) {
        for (int i = threadIdx.x; i < kBT * (kKB / 4); i += kThreads) {
            const int t = i / (kKB / 4), kq = (i - t * (kKB / 4)) * 4;
            const float4 v = (t < rows && k0 + kq < K) ? *reinterpret_cast<const float4*>(gc + (n0 + t) * K + k0 + kq)
                                                       : make_float4(0, 0, 0, 0);
            *reinterpret_cast<float4*>(Gb + t * kLB + kq) = v;
        }
    } else {
        for (int i = threadIdx.x; i < kBT * kKB; i += kThreads) {
            const int t = i / kKB, kl = i - t * kKB;
            Gb[t * kLB + kl] = (t < rows && k0 + kl < K) ? gc[(n0 + t) * K + k0 + kl] : 0.0f;
        }
    }
}

template <int KB>
size_t kb_rows_lds_bytes(int dr, int dv) {
    return size_t(dr * kLDT + 2 * dr * kLB + kKB + kBT * (KB * kKB + 4) + kKB * (dv + 4) + kKB + kBT * (dv + 4)) *
           sizeof(float);
}

// Row passes, grid (G, P): rows [g seg, (g + 1) seg) of problem p in tiles of 64.
//   KB_KEY: responsibilities of X = X_K into the cache gc, and the split's partial [Vt | Z]
//     (Eq. 5-6) of Y = V into mem_part;
//   KB_QUERY: responsibilities of X = X_Q into gc; with the memory mem = [Vt | Z] and Y = dO,
//     D_i and a'_i of every row into rowda ([.][2] per problem);
//   KB_GAMMA: the responsibilities of X into gc only.
enum { KB_KEY = 0, KB_QUERY = 1, KB_GAMMA = 2 };
constexpr int kRowsTW = 2;  // register tile width of the row passes (eight waves)
template <int KB, int MODE, int TW>
__global__ void __launch_bounds__(1024 / TW)
    f32_bwd_kb_rows_kernel(const float* __restrict__ X, const float* __restrict__ Y, int64_t N, int H, int dr, int dv,
                           int K, int64_t seg, int G, const double* __restrict__ c, const double* __restrict__ inv,
                           const float* __restrict__ mu, const float* __restrict__ mem, float eps,
                           float* __restrict__ gcache, float* __restrict__ mem_part, float* __restrict__ rowda) {
    constexpr bool QUERY = MODE == KB_QUERY;
    constexpr int NTH = 1024 / TW, CG = 64 / TW;  // threads; column groups of a row group
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int gi = blockIdx.x, h = int(p % H);
    const int tid = threadIdx.x, r0 = (tid / CG) * 4, m0 = (tid % CG) * TW;
    const int LK = KB * kKB + 4, LY = dv + 4;
    float* xT = lds;                   // [dr][kLDT]
    float* muT = xT + dr * kLDT;       // [dr][kLB]
    float* ivT = muT + dr * kLB;       // [dr][kLB]
    float* cB = ivT + dr * kLB;        // [kKB]
    float* S = cB + kKB;               // [64][LK] responsibilities
    float* Mb = S + kBT * LK;          // [kKB][dv + 4] a block of Vt (query)
    float* Zb = Mb + kKB * LY;         // [kKB]
    float* Yr = Zb + kKB;              // [64][dv + 4] V (key) or dO (query) rows
    const double *ch = c + size_t(h) * K, *ih = inv + size_t(h) * K * dr;
    const float* mh = mu + size_t(h) * K * dr;
    const int64_t lo = int64_t(gi) * seg, hi = min<int64_t>(lo + seg, N);
    const float* Xp = X + size_t(p) * N * dr;
    const float* Yp = Y + size_t(p) * N * dv;
    float* gc = gcache + size_t(p) * N * K;
    float mv[KB][4][TW] = {}, mz[KB][4] = {};  // key side: Vt rows k = kb 64 + r0.., columns c = m0..
    for (int64_t n0 = lo; n0 < hi; n0 += kBT) {
        const int rows = int(min<int64_t>(kBT, hi - n0));
        __syncthreads();  // the previous tile's reads are done
        if (MODE != KB_GAMMA)
            for (int i = tid; i < kBT * (dv / 4); i += NTH) {
                const int t = i / (dv / 4), cc = (i - t * (dv / 4)) * 4;
                const float4 v =
                    t < rows ? *reinterpret_cast<const float4*>(Yp + (n0 + t) * dv + cc) : make_float4(0, 0, 0, 0);
                *reinterpret_cast<float4*>(Yr + t * LY + cc) = v;
            }
        KbMemBlock<NTH> mb;  // query: the memory's first block, in flight while the tile is scored
        if (QUERY) mb.load(mem + size_t(p) * K * (dv + 1), K, dv, 0);
        kb_gamma<KB, TW>(Xp, n0, rows, dr, K, ch, ih, mh, xT, muT, ivT, cB, S, LK, gc);
        if (MODE == KB_GAMMA) continue;
        if (!QUERY) {
            if (m0 < dv)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll 4
                    for (int t = 0; t < rows; ++t) {
                        float ga[4], ya[TW];
                        unpack(lds4(S + t * LK + kb * kKB + r0), ga);
                        ldsw<TW>(Yr + t * LY + m0, ya);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            mz[kb][i] += ga[i];
#pragma unroll
                            for (int j = 0; j < TW; ++j) mv[kb][i][j] = fmaf(ga[i], ya[j], mv[kb][i][j]);
                        }
                    }
            continue;
        }
        // query: N_t = gamma_t Vt (rows t = r0.., columns c = m0..) and gamma_t Z, block by block
        float nv[4][TW] = {}, dz[4] = {};
        const float* mp = mem + size_t(p) * K * (dv + 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            __syncthreads();  // the previous block of the memory is consumed
            mb.store(Mb, Zb, dv);
            __syncthreads();
            if (kb + 1 < KB) mb.load(mp, K, dv, (kb + 1) * kKB);  // in flight during this block's products
#pragma unroll 4
            for (int kl = 0; kl < kKB; ++kl) {
                float ga[4], va[TW];
#pragma unroll
                for (int i = 0; i < 4; ++i) ga[i] = S[(r0 + i) * LK + kb * kKB + kl];
                ldsw<TW>(Mb + kl * LY + (m0 < dv ? m0 : 0), va);
                const float z = Zb[kl];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dz[i] = fmaf(ga[i], z, dz[i]);
#pragma unroll
                    for (int j = 0; j < TW; ++j) nv[i][j] = fmaf(ga[i], va[j], nv[i][j]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float dot = 0.0f;
            if (m0 < dv) {
                float oa[TW];
                ldsw<TW>(Yr + (r0 + i) * LY + m0, oa);
#pragma unroll
                for (int j = 0; j < TW; ++j) dot = fmaf(oa[j], nv[i][j], dot);
            }
            dot = sum_lanes<CG>(dot);
            const float D = dz[i] + eps;
            if (m0 == 0 && r0 + i < rows) {
                rowda[(size_t(p) * N + n0 + r0 + i) * 2] = D;
                rowda[(size_t(p) * N + n0 + r0 + i) * 2 + 1] = dot / (D * D);
            }
        }
    }
    if (MODE == KB_KEY) {  // the split's partial [Vt | Z]
        float* out = mem_part + (size_t(p) * G + gi) * size_t(K) * (dv + 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = kb * kKB + r0 + i;
                if (k >= K) continue;
                if (m0 < dv)
#pragma unroll
                    for (int j = 0; j < TW; ++j) out[size_t(k) * dv + m0 + j] = mv[kb][i][j];
                if (m0 == 0) out[size_t(K) * dv + k] = mz[kb][i];
            }
    }
}


// Responsibilities [t][k0 .. k0 + 63] of the tile's rows into Gb ([64][kLB]) as load_gamma_block,
// for a workgroup of NTH threads.
template <int NTH>
__device__ __forceinline__ void load_gamma_block_n(const float* __restrict__ gc, int64_t n0, int rows, int K, int k0,
                                                   float* Gb) {
    if ((K & 3) == 0) {
        for (int i = threadIdx.x; i < kBT * (kKB / 4); i += NTH) {
            const int t = i / (kKB / 4), kq = (i - t * (kKB / 4)) * 4;
            const float4 v = (t < rows && k0 + kq < K) ? *reinterpret_cast<const float4*>(gc + (n0 + t) * K + k0 + kq)
                                                       : make_float4(0, 0, 0, 0);
            *reinterpret_cast<float4*>(Gb + t * kLB + kq) = v;
        }
    } else {
        for (int i = threadIdx.x; i < kBT * kKB; i += NTH) {
            const int t = i / kKB, kl = i - t * kKB;
            Gb[t * kLB + kl] = (t < rows && k0 + kl < K) ? gc[(n0 + t) * K + k0 + kl] : 0.0f;
        }
    }
}

// The block of a memory [Vt (K x dv) | ...] with rows k0 .. k0 + 63 into MT ([dv][kLB], transposed,
// zero past K), by NTH threads: 16-byte row reads when the memory's rows start on 16-byte
// boundaries (K a multiple of 4), else one element at a time.
template <int NTH>
__device__ __forceinline__ void load_mem_block_t(const float* __restrict__ mp, int K, int dv, int k0, float* MT) {
    if ((K & 3) == 0) {
        for (int i = threadIdx.x; i < kKB * (dv / 4); i += NTH) {
            const int kl = i / (dv / 4), cc = (i - kl * (dv / 4)) * 4, k = k0 + kl;
            const float4 v = k < K ? *reinterpret_cast<const float4*>(mp + size_t(k) * dv + cc) : make_float4(0, 0, 0, 0);
            MT[(cc + 0) * kLB + kl] = v.x;
            MT[(cc + 1) * kLB + kl] = v.y;
            MT[(cc + 2) * kLB + kl] = v.z;
            MT[(cc + 3) * kLB + kl] = v.w;
        }
    } else {
        for (int i = threadIdx.x; i < kKB * dv; i += NTH) {
            const int kl = i / dv, cc = i - kl * dv, k = k0 + kl;
            MT[cc * kLB + kl] = k < K ? mp[size_t(k) * dv + cc] : 0.0f;
        }
    }
}

size_t kb_block_lds_bytes(int dr, int dv) {
    return size_t(2 * kBT * kLB + kBT * (dv + 4) + dv * kLB + kKB + 3 * kBT + kBT * (dr + 4) + 2 * kKB * (dr + 4)) *
           sizeof(float);
}
constexpr int kBlockTW = 2;  // register tile width of the bidirectional block passes (eight waves)

// Block passes, grid (G, P, KB): component block kb = blockIdx.z of split g of problem p.
//   QUERY: Y = dO, mem = [Vt | Z], rowda = (D, a') per row; g_ik = (dO_i . Vt_k) / D_i - a'_i Z_k and
//     ds = gamma (g - eps a'); the block's rows of the partial [dVt | dZ] into mem_part;
//   key: Y = V, mem = [dVt | dZ], rowda = w per row (the key-side closed form); g_jk = V_j . dVt_k + dZ_k.
// Both: the block's entries of the moment record (S1, S2, S0) into param_part, and the block's
// share of dX (-sum_k ds_ik (x_id - mu_kd) / sigma2_kd over its components) into dX_part[kb].
// Each thread holds 4 x TW register tiles of the 64 x 64 products: 1024 / TW threads, so TW = 2
// gives eight waves (two per SIMD) where the 123 KB of LDS allow one workgroup per CU.
template <bool QUERY, int TW>
__global__ void __launch_bounds__(1024 / TW)
    f32_bwd_kb_block_kernel(const float* __restrict__ X, const float* __restrict__ Y, int64_t N, int H, int dr, int dv,
                            int K, int64_t seg, int G, const double* __restrict__ inv, const float* __restrict__ mu,
                            const float* __restrict__ mem, float eps, const float* __restrict__ gcache,
                            const float* __restrict__ rowda, float* __restrict__ mem_part,
                            float* __restrict__ param_part, float* __restrict__ dX_part) {
    constexpr int NTH = 1024 / TW, CG = 64 / TW;  // threads; column groups of a row group
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int gi = blockIdx.x, kb = blockIdx.z, h = int(p % H);
    const int tid = threadIdx.x, r0 = (tid / CG) * 4, m0 = (tid % CG) * TW;
    const int LY = dv + 4, LX = dr + 4, k0 = kb * kKB;
    float* Gb = lds;                  // [64][kLB] responsibilities of the block
    float* Db = Gb + kBT * kLB;       // [64][kLB] ds
    float* Yr = Db + kBT * kLB;       // [64][dv + 4] dO / D (query) or V (key) rows
    float* MT = Yr + kBT * LY;        // [dv][kLB] the block of Vt (query) or dVt (key), transposed
    float* Zb = MT + dv * kLB;        // [kKB] Z or dZ
    float* Av = Zb + kKB;             // [64] a' (query)
    float* Wv = Av + kBT;             // [64] sum_k gamma g of the row
    float* Dv = Wv + kBT;             // [64] D (query)
    float* Xr = Dv + kBT;             // [64][dr + 4] x rows
    float* muR = Xr + kBT * LX;       // [kKB][dr + 4] mu of the block
    float* ivR = muR + kKB * LX;      // [kKB][dr + 4] 1 / sigma2 of the block
    const double* ih = inv + size_t(h) * K * dr;
    const float* mh = mu + size_t(h) * K * dr;
    const float* mp = mem + size_t(p) * K * (dv + 1);
    for (int i = tid; i < kKB * dr; i += NTH) {
        const int kl = i / dr, d = i - kl * dr, k = k0 + kl;
        muR[kl * LX + d] = k < K ? mh[size_t(k) * dr + d] : 0.0f;
        ivR[kl * LX + d] = k < K ? float(ih[size_t(k) * dr + d]) : 0.0f;
    }
    load_mem_block_t<NTH>(mp, K, dv, k0, MT);
    for (int kl = tid; kl < kKB; kl += NTH) Zb[kl] = k0 + kl < K ? mp[size_t(K) * dv + k0 + kl] : 0.0f;
    __syncthreads();
    // moment accumulators (rows d = r0.., columns k = m0..) with their mu; memory-gradient
    // accumulators (query: rows k = r0.., columns c = m0..)
    const bool mom = r0 < dr;
    float mreg[4][TW], s1[4][TW] = {}, s2[4][TW] = {}, s0[TW] = {}, mv[4][TW] = {}, mz[4] = {};
    if (mom)
#pragma unroll
        for (int j = 0; j < TW; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) mreg[i][j] = muR[(m0 + j) * LX + r0 + i];
    const int64_t lo = int64_t(gi) * seg, hi = min<int64_t>(lo + seg, N);
    const float* Xp = X + size_t(p) * N * dr;
    const float* Yp = Y + size_t(p) * N * dv;
    const float* gc = gcache + size_t(p) * N * K;
    float* dXp = dX_part + (size_t(kb) * gridDim.y + p) * N * dr;
    for (int64_t n0 = lo; n0 < hi; n0 += kBT) {
        const int rows = int(min<int64_t>(kBT, hi - n0));
        __syncthreads();  // the previous tile's reads are done
        load_gamma_block_n<NTH>(gc, n0, rows, K, k0, Gb);
        for (int t = tid; t < kBT; t += NTH) {
            if (QUERY) {
                const float D = t < rows ? rowda[(size_t(p) * N + n0 + t) * 2] : 1.0f;
                const float a = t < rows ? rowda[(size_t(p) * N + n0 + t) * 2 + 1] : 0.0f;
                Dv[t] = D;
                Av[t] = a;
                Wv[t] = eps * a;
            } else {
                Wv[t] = t < rows ? rowda[size_t(p) * N + n0 + t] : 0.0f;
            }
        }
        for (int i = tid; i < kBT * (dr / 4); i += NTH) {
            const int t = i / (dr / 4), d = (i - t * (dr / 4)) * 4;
            *reinterpret_cast<float4*>(Xr + t * LX + d) =
                t < rows ? *reinterpret_cast<const float4*>(Xp + (n0 + t) * dr + d) : make_float4(0, 0, 0, 0);
        }
        __syncthreads();  // Dv before the scaled rows
        for (int i = tid; i < kBT * (dv / 4); i += NTH) {
            const int t = i / (dv / 4), cc = (i - t * (dv / 4)) * 4;
            float4 v = t < rows ? *reinterpret_cast<const float4*>(Yp + (n0 + t) * dv + cc) : make_float4(0, 0, 0, 0);
            if (QUERY) {
                const float rD = 1.0f / Dv[t];
                v.x *= rD, v.y *= rD, v.z *= rD, v.w *= rD;
            }
            *reinterpret_cast<float4*>(Yr + t * LY + cc) = v;
        }
        __syncthreads();
        {   // g (rows t = r0.., components k = m0..), then ds = gamma (g - w_t) into Db
            float gg[4][TW] = {};
#pragma unroll 4
            for (int cc = 0; cc < dv; ++cc) {
                float ya[4], ma[TW];
#pragma unroll
                for (int i = 0; i < 4; ++i) ya[i] = Yr[(r0 + i) * LY + cc];
                ldsw<TW>(MT + cc * kLB + m0, ma);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) gg[i][j] = fmaf(ya[i], ma[j], gg[i][j]);
            }
            float za[TW];
            ldsw<TW>(Zb + m0, za);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float ga[TW], ds[TW];
                ldsw<TW>(Gb + (r0 + i) * kLB + m0, ga);
                const float w = Wv[r0 + i];
#pragma unroll
                for (int j = 0; j < TW; ++j) {
                    const float g = QUERY ? gg[i][j] - Av[r0 + i] * za[j] : gg[i][j] + za[j];
                    ds[j] = ga[j] * (g - w);
                }
                stsw<TW>(Db + (r0 + i) * kLB + m0, ds);
            }
        }
        if (QUERY && m0 < dv)  // dVt (rows k = r0.., columns c = m0..), dZ
#pragma unroll 4
            for (int t = 0; t < rows; ++t) {
                float ga[4], ya[TW];
                unpack(lds4(Gb + t * kLB + r0), ga);
                ldsw<TW>(Yr + t * LY + m0, ya);
                const float a = Av[t];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (m0 == 0) mz[i] = fmaf(-ga[i], a, mz[i]);
#pragma unroll
                    for (int j = 0; j < TW; ++j) mv[i][j] = fmaf(ga[i], ya[j], mv[i][j]);
                }
            }
        __syncthreads();  // ds in Db
        if (mom)  // moments (rows d = r0.., columns k = m0..), direct (centred) form
#pragma unroll 4
            for (int t = 0; t < rows; ++t) {
                float xa[4], da[TW];
                unpack(lds4(Xr + t * LX + r0), xa);
                ldsw<TW>(Db + t * kLB + m0, da);
#pragma unroll
                for (int j = 0; j < TW; ++j) {
                    s0[j] += da[j];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float df = xa[i] - mreg[i][j], w = da[j] * df;
                        s1[i][j] += w;
                        s2[i][j] = fmaf(w, df, s2[i][j]);
                    }
                }
            }
        if (m0 < dr) {  // this block's share of dX (rows t = r0.., columns d = m0..)
            float xa[4][TW], acc[4][TW] = {};
#pragma unroll
            for (int i = 0; i < 4; ++i) ldsw<TW>(Xr + (r0 + i) * LX + m0, xa[i]);
            const int kn = min(kKB, K - k0);
#pragma unroll 4
            for (int kl = 0; kl < kn; ++kl) {
                float ma[TW], ia[TW], da[4];
                ldsw<TW>(muR + kl * LX + m0, ma);
                ldsw<TW>(ivR + kl * LX + m0, ia);
#pragma unroll
                for (int i = 0; i < 4; ++i) da[i] = Db[(r0 + i) * kLB + kl];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) acc[i][j] = fmaf(da[i] * ia[j], xa[i][j] - ma[j], acc[i][j]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (r0 + i < rows) {
                    float o[TW];
#pragma unroll
                    for (int j = 0; j < TW; ++j) o[j] = -acc[i][j];
                    stsw<TW>(dXp + (n0 + r0 + i) * dr + m0, o);
                }
        }
    }
    // the block's entries of the moment record [S1 (K dr) | S2 (K dr) | S0 (K)]
    float* pp = param_part + (size_t(p) * G + gi) * size_t(2 * K * dr + K);
    if (mom)
#pragma unroll
        for (int j = 0; j < TW; ++j) {
            const int k = k0 + m0 + j;
            if (k >= K) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pp[size_t(k) * dr + r0 + i] = s1[i][j];
                pp[size_t(K) * dr + size_t(k) * dr + r0 + i] = s2[i][j];
            }
            if (r0 == 0) pp[2 * size_t(K) * dr + k] = s0[j];
        }
    if (QUERY) {  // the block's rows of the partial [dVt | dZ]
        float* out = mem_part + (size_t(p) * G + gi) * size_t(K) * (dv + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + r0 + i;
            if (k >= K) continue;
            if (m0 < dv)
#pragma unroll
                for (int j = 0; j < TW; ++j) out[size_t(k) * dv + m0 + j] = mv[i][j];
            if (m0 == 0) out[size_t(K) * dv + k] = mz[i];
        }
    }
}

// Key rows, grid (G, P): dV_j = gamma^K_j dVt (an output) and w_j = V_j . dV_j + gamma^K_j . dZ from
// the cached responsibilities and dmem = [dVt | dZ].
template <int KB>
__global__ void __launch_bounds__(kThreads)
    f32_bwd_kb_keyrows_kernel(const float* __restrict__ V, int64_t N, int dv, int K, int64_t seg,
                              const float* __restrict__ dmem, const float* __restrict__ gcache,
                              float* __restrict__ dV, float* __restrict__ roww) {
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int gi = blockIdx.x;
    const int tid = threadIdx.x, r0 = (tid >> 4) * 4, m0 = (tid & 15) * 4;
    const int LY = dv + 4;
    float* Gb = lds;               // [64][kLB]
    float* Mb = Gb + kBT * kLB;    // [kKB][dv + 4] a block of dVt
    float* Zb = Mb + kKB * LY;     // [kKB]
    const float* mp = dmem + size_t(p) * K * (dv + 1);
    const float* gc = gcache + size_t(p) * N * K;
    const int64_t lo = int64_t(gi) * seg, hi = min<int64_t>(lo + seg, N);
    for (int64_t n0 = lo; n0 < hi; n0 += kBT) {
        const int rows = int(min<int64_t>(kBT, hi - n0));
        float nv[4][4] = {}, ez[4] = {};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int k0 = kb * kKB;
            __syncthreads();  // the previous block is consumed
            load_gamma_block(gc, n0, rows, K, k0, Gb);
            for (int i = tid; i < kKB * (dv / 4); i += kThreads) {
                const int kl = i / (dv / 4), cc = (i - kl * (dv / 4)) * 4, k = k0 + kl;
                *reinterpret_cast<float4*>(Mb + kl * LY + cc) =
                    k < K ? *reinterpret_cast<const float4*>(mp + size_t(k) * dv + cc) : make_float4(0, 0, 0, 0);
            }
            for (int kl = tid; kl < kKB; kl += kThreads) Zb[kl] = k0 + kl < K ? mp[size_t(K) * dv + k0 + kl] : 0.0f;
            __syncthreads();
#pragma unroll 4
            for (int kl = 0; kl < kKB; ++kl) {
                float ga[4], va[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) ga[i] = Gb[(r0 + i) * kLB + kl];
                unpack(lds4(Mb + kl * LY + (m0 < dv ? m0 : 0)), va);
                const float z = Zb[kl];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ez[i] = fmaf(ga[i], z, ez[i]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) nv[i][j] = fmaf(ga[i], va[j], nv[i][j]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n = n0 + r0 + i;
            float dot = 0.0f;
            if (m0 < dv && r0 + i < rows) {
                const float4 v = *reinterpret_cast<const float4*>(V + (size_t(p) * N + n) * dv + m0);
                dot = v.x * nv[i][0] + v.y * nv[i][1] + v.z * nv[i][2] + v.w * nv[i][3];
                *reinterpret_cast<float4*>(dV + (size_t(p) * N + n) * dv + m0) =
                    make_float4(nv[i][0], nv[i][1], nv[i][2], nv[i][3]);
            }
            dot = sum16(dot);
            if ((tid & 15) == 0 && r0 + i < rows) roww[size_t(p) * N + n] = dot + ez[i];
        }
    }
}

// dX = sum over the component blocks of their shares, in block order.
__global__ void __launch_bounds__(kThreads) f32_bwd_kb_sum_kernel(const float* __restrict__ part, int KB, size_t n,
                                                                  float* __restrict__ dX) {
    const size_t i = (size_t(blockIdx.x) * kThreads + threadIdx.x) * 4;
    if (i >= n) return;
    float4 s = *reinterpret_cast<const float4*>(part + i);
    for (int kb = 1; kb < KB; ++kb) {
        const float4 v = *reinterpret_cast<const float4*>(part + size_t(kb) * n + i);
        s.x += v.x, s.y += v.y, s.z += v.z, s.w += v.w;
    }
    *reinterpret_cast<float4*>(dX + i) = s;
}

// The one-element-per-thread passes: FAST (tables and memory in LDS) with the largest tile (64
// down to 16 positions) that fits, else the general form with the largest tile that fits.
// With larger K the tables alone stay in LDS (the memory is read from the workspace) and the
// tiles shrink to 8 positions.
struct SideConfig {
    bool fast;
    int mem_lds;
    int T;
    size_t lds;
};
SideConfig side_config(int K, int dr, int dv) {
    const size_t tables = size_t(2 * K * (dr + 1) + K) * sizeof(float);
    const size_t memory = size_t(K * (dv + 1) + K) * sizeof(float);
    for (int t = kTile; t >= 16; t /= 2)
        if (bwd_lds_bytes(t, dr, dv, K) + tables + memory <= kMaxLds)
            return {true, 1, t, bwd_lds_bytes(t, dr, dv, K) + tables + memory};
    for (int t = kTile; t >= 8; t /= 2)
        if (bwd_lds_bytes(t, dr, dv, K) + tables <= kMaxLds) return {true, 0, t, bwd_lds_bytes(t, dr, dv, K) + tables};
    int T = kTile;
    while (T > 8 && bwd_lds_bytes(T, dr, dv, K) > kMaxLds) T /= 2;
    return {false, 0, T, bwd_lds_bytes(T, dr, dv, K)};
}

hipError_t bwd_allow_lds() {
    static const hipError_t e = [] {
        const void* fns[] = {(const void*)f32_write_kernel, (const void*)f32_bwd_side_kernel<true, false>,
                             (const void*)f32_bwd_side_kernel<false, false>, (const void*)f32_bwd_side_kernel<true, true>,
                             (const void*)f32_bwd_side_kernel<false, true>,
                             (const void*)f32_bwd_tiled_kernel<BWD_WRITE, kTiledTW>, (const void*)f32_bwd_tiled_kernel<BWD_QUERY, kTiledTW>,
                             (const void*)f32_bwd_tiled_kernel<BWD_KEY, kTiledTW>, (const void*)f32_bwd_tiled_kernel<BWD_CQUERY, kTiledTW>,
                             (const void*)f32_bwd_tiled_kernel<BWD_CKEY, kTiledTW>,
                             (const void*)f32_bwd_kb_rows_kernel<2, KB_KEY, kRowsTW>, (const void*)f32_bwd_kb_rows_kernel<2, KB_QUERY, kRowsTW>,
                             (const void*)f32_bwd_kb_rows_kernel<3, KB_KEY, kRowsTW>, (const void*)f32_bwd_kb_rows_kernel<3, KB_QUERY, kRowsTW>,
                             (const void*)f32_bwd_kb_rows_kernel<4, KB_KEY, kRowsTW>, (const void*)f32_bwd_kb_rows_kernel<4, KB_QUERY, kRowsTW>,
                             (const void*)f32_bwd_kb_block_kernel<true, kBlockTW>, (const void*)f32_bwd_kb_block_kernel<false, kBlockTW>,
                             (const void*)f32_bwd_kb_keyrows_kernel<2>, (const void*)f32_bwd_kb_keyrows_kernel<3>,
                             (const void*)f32_bwd_kb_keyrows_kernel<4>};
        for (const void* f : fns) {
            hipError_t r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxLds));
            if (r != hipSuccess) return r;
        }
        return hipSuccess;
    }();
    return e;
}

}  // namespace

// Responsibilities of one side, [P][N][K] fp32 (the register-tiled passes keep them between passes).
size_t gamma_cache_bytes(const Plan& p) { return round_up(size_t(p.P * p.N) * size_t(p.K) * 4, 256); }

bool bwd_kb_applies(const Plan& p) {
    return p.K > 64 && p.K <= 256 && p.dr % 4 == 0 && p.dv % 4 == 0 && p.dr <= 64 && p.dv <= 64 && p.N > 0 &&
           p.Nq > 0;
}

// The K-blocked passes' buffers: the responsibilities of both sides ([P][Nq][K], [P][N][K]),
// (D, a') per query row, w per key row and the blocks' shares of dX ([KB][P][max(N, Nq)][dr]).
struct KbBuffers {
    float *gq, *gk, *rowq, *roww, *dxpart;
};
size_t kb_bytes(const Plan& p, KbBuffers* b, char* base) {
    const size_t P = size_t(p.P), K = size_t(p.K), nmax = size_t(std::max(p.N, p.Nq));
    const size_t sizes[5] = {round_up(P * size_t(p.Nq) * K * 4, 256), round_up(P * size_t(p.N) * K * 4, 256),
                             round_up(P * size_t(p.Nq) * 2 * 4, 256), round_up(P * size_t(p.N) * 4, 256),
                             round_up(size_t(kb_blocks(p.K)) * P * nmax * size_t(p.dr) * 4, 256)};
    size_t off = 0;
    float** outs[5] = {b ? &b->gq : nullptr, b ? &b->gk : nullptr, b ? &b->rowq : nullptr, b ? &b->roww : nullptr,
                       b ? &b->dxpart : nullptr};
    for (int i = 0; i < 5; ++i) {
        if (b) *outs[i] = reinterpret_cast<float*>(base + off);
        off += sizes[i];
    }
    return off;
}

size_t f32_backward_extra_bytes(const Plan& p) {
    const size_t E = size_t(p.K) * size_t(p.dv + 1);
    return round_up(size_t(p.P * p.G) * E * 4, 256) + round_up(size_t(p.P) * E * 4, 256) +
           round_up(2 * size_t(p.P * p.G) * size_t(2 * p.K * p.dr + p.K) * 4, 256) +
           (bwd_tiled_applies(p) ? gamma_cache_bytes(p) : 0) + (bwd_kb_applies(p) ? kb_bytes(p, nullptr, nullptr) : 0);
}

namespace {

// Splits of the K-blocked block passes.  Each workgroup walks its split's tiles for one component
// block; its prologue (the block's tables and memory) and its moment record are per workgroup,
// so the block passes take coarser splits than the row passes: about 256 workgroups in all
// (one round of one workgroup per CU; measured faster than 512, 1024 or 4096 at B8 H8 N1024).
// The moment records of the block passes and the memory-gradient partials then follow this
// split (the workspace holds the plan's finer one).
struct BlockSplit {
    int G;
    int64_t seg, seg_q;
};
BlockSplit block_split(const Plan& p, int KB) {
    const int64_t per = std::max<int64_t>(1, (256 + p.P * KB - 1) / (p.P * KB));
    const int64_t g = std::min<int64_t>(p.G, per);
    auto tiles = [&](int64_t n) { return int64_t(round_up(size_t((std::max<int64_t>(n, 1) + g - 1) / g), kBT)); };
    BlockSplit b{};
    b.seg = tiles(p.N);
    b.seg_q = tiles(p.Nq);
    b.G = int(std::max<int64_t>(1, std::max((p.N + b.seg - 1) / b.seg, (p.Nq + b.seg_q - 1) / b.seg_q)));
    return b;
}

// The parameter gradients from moment records of G splits per problem (query side, then key side
// after P G records).
hipError_t reduce_params_split(const Plan& p, int G, const float* part, const double* inv, const float* pi,
                               float* dmu, float* ds2, float* dpi, hipStream_t st) {
    Plan q = p;
    q.G = G;
    return reduce_params(q, part, int(p.B), inv, pi, dmu, ds2, dpi, st);
}

template <typename F>
hipError_t with_kb(int KB, F&& f) {
    if (KB == 2) return f(std::integral_constant<int, 2>());
    if (KB == 3) return f(std::integral_constant<int, 3>());
    if (KB == 4) return f(std::integral_constant<int, 4>());
    return hipErrorNotSupported;
}

// The bidirectional backward in K-blocked passes (see f32_bwd_kb_rows_kernel).
hipError_t f32_backward_bidir_kb(const Plan& p, const float* XQ, const float* XK, const float* V, const float* mu,
                                 const float* pi, float eps, const float* dO, float* dXQ, float* dXK, float* dV,
                                 float* dmu, float* ds2, float* dpi, const F32Params& v, float* partials, float* memory,
                                 float* dpart, float* dmem, float* ppart, float* ppart_key, char* kbase, hipStream_t st) {
    KbBuffers b{};
    kb_bytes(p, &b, kbase);
    const int H = int(p.H), dr = int(p.dr), dv = int(p.dv), K = int(p.K), G = int(p.G), KB = kb_blocks(p.K);
    const BlockSplit bs = block_split(p, KB);
    const int Ei = int(size_t(p.K) * size_t(p.dv + 1));
    const dim3 grid(unsigned(p.G), unsigned(p.P)), bgrid(unsigned(bs.G), unsigned(p.P), unsigned(KB));
    const dim3 cgrid(unsigned((Ei + kThreads - 1) / kThreads), unsigned(p.P));
    const float* cnone = nullptr;
    float* none = nullptr;
    const size_t blds = kb_block_lds_bytes(dr, dv);
    // the key side's moment records follow the query side's P bs.G ones
    ppart_key = ppart + size_t(p.P) * size_t(bs.G) * size_t(2 * p.K * p.dr + p.K);
    auto sum_dx = [&](int64_t N, float* dX) {
        const size_t n = size_t(p.P) * size_t(N) * size_t(dr);
        if (n == 0) return hipSuccess;  // an empty side of cross-attention: no rows, no launch
        GMA_LAUNCH("f32_bwd_dx_sum", f32_bwd_kb_sum_kernel, dim3(unsigned((n / 4 + kThreads - 1) / kThreads)),
                   dim3(kThreads), 0, st, static_cast<const float*>(b.dxpart), KB, n, dX);
        return hipGetLastError();
    };
    return with_kb(KB, [&](auto KBc) -> hipError_t {
        constexpr int KBT = decltype(KBc)::value;
        const size_t rlds = kb_rows_lds_bytes<KBT>(dr, dv);
        hipError_t e;
        GMA_LAUNCH("f32_bwd_kb_write", (f32_bwd_kb_rows_kernel<KBT, KB_KEY, kRowsTW>), grid, dim3(1024 / kRowsTW), rlds, st, XK, V, p.N, H,
                   dr, dv, K, p.seg, G, v.c, v.inv, mu, cnone, eps, b.gk, partials, none);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        GMA_LAUNCH("f32_bwd_combine", f32_combine_kernel, cgrid, dim3(kThreads), 0, st, partials, G, Ei, memory);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        GMA_LAUNCH("f32_bwd_kb_query_rows", (f32_bwd_kb_rows_kernel<KBT, KB_QUERY, kRowsTW>), grid, dim3(1024 / kRowsTW), rlds, st, XQ, dO,
                   p.Nq, H, dr, dv, K, p.seg_q, G, v.c, v.inv, mu, static_cast<const float*>(memory), eps, b.gq, none,
                   b.rowq);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        GMA_LAUNCH("f32_bwd_kb_query", (f32_bwd_kb_block_kernel<true, kBlockTW>), bgrid, dim3(1024 / kBlockTW), blds, st, XQ, dO, p.Nq, H,
                   dr, dv, K, bs.seg_q, bs.G, v.inv, mu, static_cast<const float*>(memory), eps,
                   static_cast<const float*>(b.gq), static_cast<const float*>(b.rowq), dpart, ppart, b.dxpart);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = sum_dx(p.Nq, dXQ)) != hipSuccess) return e;
        GMA_LAUNCH("f32_bwd_combine", f32_combine_kernel, cgrid, dim3(kThreads), 0, st, dpart, bs.G, Ei, dmem);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        GMA_LAUNCH("f32_bwd_kb_key_rows", f32_bwd_kb_keyrows_kernel<KBT>, grid, dim3(kThreads),
                   size_t(kBT * kLB + kKB * (dv + 4) + kKB) * sizeof(float), st, V, p.N, dv, K, p.seg,
                   static_cast<const float*>(dmem), static_cast<const float*>(b.gk), dV, b.roww);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        GMA_LAUNCH("f32_bwd_kb_key", (f32_bwd_kb_block_kernel<false, kBlockTW>), bgrid, dim3(1024 / kBlockTW), blds, st, XK, V, p.N, H, dr,
                   dv, K, bs.seg, bs.G, v.inv, mu, static_cast<const float*>(dmem), eps, static_cast<const float*>(b.gk),
                   static_cast<const float*>(b.roww), none, ppart_key, b.dxpart);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = sum_dx(p.N, dXK)) != hipSuccess) return e;
        return reduce_params_split(p, bs.G, ppart, v.inv, pi, dmu, ds2, dpi, st);
    });
}

}  // namespace

hipError_t f32_backward_bidir(const Plan& p, const float* XQ, const float* XK, const float* V, const float* mu,
                              const float* s2, const float* pi, float eps, const float* dO, float* dXQ, float* dXK,
                              float* dV, float* dmu, float* ds2, float* dpi, char* ws, hipStream_t st) {
    if (p.H == 0) return hipSuccess;
    // no rows on either side: zero parameter gradients (one empty side of cross-attention runs the
    // passes, which give the zeros of that case: an empty context leaves O = 0)
    if (p.P == 0 || (p.N == 0 && p.Nq == 0)) return reduce_params(p, nullptr, 0, nullptr, pi, dmu, ds2, dpi, st);
    hipError_t e = bwd_allow_lds();
    if (e != hipSuccess) return e;
    if ((e = launch_param_tables(p, s2, pi, ws, st)) != hipSuccess) return e;
    F32Params v = f32_params_view(p, ws);
    float* partials = reinterpret_cast<float*>(ws + p.off_partials);
    float* memory = reinterpret_cast<float*>(ws + p.off_memory);
    const size_t E = size_t(p.K) * size_t(p.dv + 1);
    char* extra = ws + p.off_stage - f32_backward_extra_bytes(p);
    float* dpart = reinterpret_cast<float*>(extra);
    float* dmem = reinterpret_cast<float*>(extra + round_up(size_t(p.P * p.G) * E * 4, 256));
    float* ppart = reinterpret_cast<float*>(extra + round_up(size_t(p.P * p.G) * E * 4, 256) + round_up(size_t(p.P) * E * 4, 256));
    float* ppart_key = ppart + size_t(p.P * p.G) * size_t(2 * p.K * p.dr + p.K);
    // Gamma_K from the write pass, read back by the key pass (tiled passes only)
    float* gk_cache = reinterpret_cast<float*>(reinterpret_cast<char*>(ppart) +
                                               round_up(2 * size_t(p.P * p.G) * size_t(2 * p.K * p.dr + p.K) * 4, 256));
    float* none = nullptr;
    const float* cnone = nullptr;
    if (bwd_kb_applies(p))
        return f32_backward_bidir_kb(p, XQ, XK, V, mu, pi, eps, dO, dXQ, dXK, dV, dmu, ds2, dpi, v, partials, memory,
                                     dpart, dmem, ppart, ppart_key,
                                     reinterpret_cast<char*>(ppart) +
                                         round_up(2 * size_t(p.P * p.G) * size_t(2 * p.K * p.dr + p.K) * 4, 256),
                                     st);
    const dim3 grid(unsigned(p.G), unsigned(p.P));
    const int Ei = int(E);
    const dim3 cgrid(unsigned((Ei + kThreads - 1) / kThreads), unsigned(p.P));
    const int H = int(p.H), dr = int(p.dr), dv = int(p.dv), K = int(p.K), G = int(p.G);
    const SideConfig side = side_config(K, dr, dv);
    if (bwd_tiled_applies(p)) {
        GMA_LAUNCH("f32_bwd_write", (f32_bwd_tiled_kernel<BWD_WRITE, kTiledTW>), grid, dim3(1024 / kTiledTW),
                   bwd_tiled_lds_bytes(BWD_WRITE, K, dr, dv), st, XK, V, p.N, H, dr, dv, K, p.seg, G, v.c, v.inv, mu,
                   cnone, eps, none, none, partials, none, cnone, cnone, none, gk_cache, cnone, cnone);
    } else {
        const size_t lds_w = size_t(kTile) * (p.dr + p.K + p.dv) * sizeof(float);
        GMA_LAUNCH("f32_bwd_write", f32_write_kernel, grid, dim3(kThreads), lds_w, st, XK, V, p.N, H, dr, dv, K,
                   p.seg, G, v.c, v.inv, mu, partials);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GMA_LAUNCH("f32_bwd_combine", f32_combine_kernel, cgrid, dim3(kThreads), 0, st, partials, G, Ei, memory);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (bwd_tiled_applies(p)) {
        GMA_LAUNCH("f32_bwd_query", (f32_bwd_tiled_kernel<BWD_QUERY, kTiledTW>), grid, dim3(1024 / kTiledTW),
                   bwd_tiled_lds_bytes(BWD_QUERY, K, dr, dv), st, XQ, dO, p.Nq, H, dr, dv, K, p.seg_q, G, v.c, v.inv, mu,
                   static_cast<const float*>(memory), eps, dXQ, none, dpart, ppart, cnone, cnone, none, none, cnone,
                   cnone);
    } else if (side.fast) {
        GMA_LAUNCH("f32_bwd_query", (f32_bwd_side_kernel<true, true>), grid, dim3(kThreads), side.lds, st, XQ, dO, p.Nq,
                   H, dr, dv, K, p.seg_q, G, side.T, v.c, v.inv, mu, static_cast<const float*>(memory), eps, dXQ, none,
                   dpart, ppart, side.mem_lds);
    } else {
        GMA_LAUNCH("f32_bwd_query", (f32_bwd_side_kernel<true, false>), grid, dim3(kThreads), side.lds, st, XQ, dO,
                   p.Nq, H, dr, dv, K, p.seg_q, G, side.T, v.c, v.inv, mu, static_cast<const float*>(memory), eps, dXQ,
                   none, dpart, ppart, side.mem_lds);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GMA_LAUNCH("f32_bwd_combine", f32_combine_kernel, cgrid, dim3(kThreads), 0, st, dpart, G, Ei, dmem);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (bwd_tiled_applies(p)) {
        GMA_LAUNCH("f32_bwd_key", (f32_bwd_tiled_kernel<BWD_KEY, kTiledTW>), grid, dim3(1024 / kTiledTW),
                   bwd_tiled_lds_bytes(BWD_KEY, K, dr, dv), st, XK, V, p.N, H, dr, dv, K, p.seg, G, v.c, v.inv, mu,
                   static_cast<const float*>(dmem), eps, dXK, dV, none, ppart_key, cnone, cnone, none, none,
                   static_cast<const float*>(gk_cache), cnone);
    } else if (side.fast) {
        GMA_LAUNCH("f32_bwd_key", (f32_bwd_side_kernel<false, true>), grid, dim3(kThreads), side.lds, st, XK, V, p.N, H,
                   dr, dv, K, p.seg, G, side.T, v.c, v.inv, mu, static_cast<const float*>(dmem), eps, dXK, dV, none,
                   ppart_key, side.mem_lds);
    } else {
        GMA_LAUNCH("f32_bwd_key", (f32_bwd_side_kernel<false, false>), grid, dim3(kThreads), side.lds, st, XK, V, p.N,
                   H, dr, dv, K, p.seg, G, side.T, v.c, v.inv, mu, static_cast<const float*>(dmem), eps, dXK, dV, none,
                   ppart_key, side.mem_lds);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return reduce_params(p, ppart, int(p.B), v.inv, pi, dmu, ds2, dpi, st);
}

// ---------------------------------------------------------------------------- causal backward
// Gradients of <dO, O> for the causal forward (Eq. 6b, 8b).  Position i reads the prefix memory
// Vt^(i), Z^(i) over j <= i, so with D_i = gamma^Q_i . Z^(i) + eps and a_i = dO_i . O_i
//   g^Q_ik = (dO_i . Vt^(i)_k - a_i Z^(i)_k) / D_i,
// and key position j receives the suffix sums of what every later (or equal) query position
// sends to its memory:
//   dVt_j = sum_{i>=j} gamma^Q_i dO_i^T / D_i,  dZ_j = -sum_{i>=j} gamma^Q_i a_i / D_i,
//   dV_j = sum_k gamma^K_jk dVt_j[k],            g^K_jk = dVt_j[k] . V_j + dZ_j[k];
// Eq. 18-20 follow as for the bidirectional backward.  Within a tile of T positions the prefix
// (suffix) splits into the memory at the tile's start (end) and the masked T x T products
// C_ij = gamma^Q_i . gamma^K_j and A_ij = (dO_i . V_j - a_i) / D_i for j <= i.
namespace {

size_t bwdc_lds_bytes(int T, int dr, int dv, int K) {
    return size_t(T) * (dr + 3 * K + 2 * dv + 2 * T + 2) * sizeof(float);
}

// Causal: exclusive suffix over segments in place; segment g then holds the sum over the
// segments after it, starting from the gradient of the memory after the call (dstate_out,
// [P][K][dv+1], or zero when NULL).  The total, the gradient of the memory before the call, goes
// to dstate_in ([P][K][dv+1]) when it is not NULL.
__global__ void __launch_bounds__(kThreads) f32_suffix_kernel(float* __restrict__ partials, int G, int E,
                                                              const float* __restrict__ dstate_out,
                                                              float* __restrict__ dstate_in, int K, int dv) {
    const int64_t p = blockIdx.y;
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= E) return;
    float* src = partials + size_t(p) * G * E + e;
    float run = dstate_out ? dstate_out[size_t(p) * E + state_index(e, K, dv)] : 0.0f;
    for (int g = G - 1; g >= 0; --g) {
        const float a = src[size_t(g) * E];
        src[size_t(g) * E] = run;
        run += a;
    }
    if (dstate_in) dstate_in[size_t(p) * E + state_index(e, K, dv)] = run;
}

// ---- K-blocked passes of the causal backward (K <= 256; d_r, d_v <= 64, multiples of 4) where
// the register-tiled causal passes do not fit.  The tile of 64 positions is the unit of the
// prefix and suffix: a row pass over the key side gives every tile's aggregate gamma_K^T [V | 1]
// (then an exclusive prefix from state_in: the memory before each tile); the causal query rows
// give D_i and a'_i from that memory and the masked in-tile products C_ij = gamma^Q_i . gamma^K_j
// (j <= i, all components), keep C, and give every tile's aggregate of what its queries send,
// gamma^Q_i [dO'_i | -a'_i] (then an exclusive suffix from dstate_out: what the later tiles'
// queries send).  Block passes then need, per tile, only the memory block and
// A_ij = dO'_i . V_j - a'_i (j <= i):
//   query: g_ik = dO'_i . Vt_k - a'_i Z_k + sum_{j <= i} A_ij gamma^K_jk  (memory before the tile),
//   key:   g_jk = V_j . dVt_k + dZ_k + sum_{i >= j} A_ij gamma^Q_ik     (what later tiles send);
// the closed forms of the bidirectional passes give w (eps a'_i on the query side).

// Causal query rows, grid (G, P): per tile of rows [g seg, (g + 1) seg) of problem p: C (into
// cbuf [P][NT][64][64]), D_i and a'_i (into rowq), and the tile's aggregate of what its queries
// send (into tsend [P][NT][K (dv + 1)]).  tmem [P][NT][K (dv + 1)]: the memory before each tile.
template <int KB>
__global__ void __launch_bounds__(kThreads)
    f32_bwdc_kb_qrows_kernel(const float* __restrict__ V, const float* __restrict__ dO, int64_t N, int dv, int K,
                             int64_t seg, const float* __restrict__ gq, const float* __restrict__ gk,
                             const float* __restrict__ tmem, float eps, float* __restrict__ cbuf,
                             float* __restrict__ rowq, float* __restrict__ tsend) {
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int gi = blockIdx.x;
    const int tid = threadIdx.x, r0 = (tid >> 4) * 4, m0 = (tid & 15) * 4;
    const int LY = dv + 4, NT = int((N + kBT - 1) / kBT);
    const size_t E = size_t(K) * (dv + 1);
    // C and the V rows take the places of gamma^K and the memory block once the blocks are
    // done (kBT = kKB), which keeps the workgroup within 80 KB: two per CU
    float* Gq = lds;                // [64][kLB] gamma^Q of a block, rows i
    float* GkT = Gq + kBT * kLB;    // [kKB][kLB] gamma^K of a block, transposed: [k][j]
    float* Cm = GkT;                // [64][kLB] C (rows i, columns j), after the blocks
    float* Mb = GkT + kKB * kLB;    // [kKB][dv + 4] a block of the memory before the tile
    float* Vr = Mb;                 // [64][dv + 4] V rows, after the blocks
    float* Zb = Mb + kKB * LY;      // [kKB]
    float* Yr = Zb + kKB;           // [64][dv + 4] dO rows
    float* Dv = Yr + kBT * LY;      // [64] D
    float* Av = Dv + kBT;           // [64] a'
    static_assert(kBT == kKB, "C and the V rows reuse the block arrays");
    constexpr int VPT = kBT * 16 / kThreads;  // float4 pieces of the V rows per thread (d_v <= 64)
    float4 vreg[VPT];
    const float* gqp = gq + size_t(p) * N * K;
    const float* gkp = gk + size_t(p) * N * K;
    const int64_t lo = int64_t(gi) * seg, hi = min<int64_t>(lo + seg, N);
    for (int64_t n0 = lo; n0 < hi; n0 += kBT) {
        const int rows = int(min<int64_t>(kBT, hi - n0)), tile = int(n0 / kBT);
        const float* mp = tmem + (size_t(p) * NT + tile) * E;
        __syncthreads();  // the previous tile's reads are done
        for (int i = tid; i < kBT * (dv / 4); i += kThreads) {
            const int t = i / (dv / 4), cc = (i - t * (dv / 4)) * 4;
            const bool ok = t < rows;
            const size_t off = (size_t(p) * N + n0 + t) * dv + cc;
            *reinterpret_cast<float4*>(Yr + t * LY + cc) = ok ? *reinterpret_cast<const float4*>(dO + off) : make_float4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {  // V rows into registers, into LDS after the blocks
            const int i = tid + u * kThreads, t = i / (dv / 4), cc = (i - t * (dv / 4)) * 4;
            vreg[u] = (i < kBT * (dv / 4) && t < rows)
                          ? *reinterpret_cast<const float4*>(V + (size_t(p) * N + n0 + t) * dv + cc)
                          : make_float4(0, 0, 0, 0);
        }
        float cc4[4][4] = {}, nv[4][4] = {}, dz[4] = {};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int k0 = kb * kKB;
            __syncthreads();  // the previous block is consumed
            load_gamma_block(gqp, n0, rows, K, k0, Gq);
            if ((K & 3) == 0) {  // gamma^K rows j, transposed; 16-byte rows
                for (int i = tid; i < kBT * (kKB / 4); i += kThreads) {
                    const int t = i / (kKB / 4), kq = (i - t * (kKB / 4)) * 4;
                    const float4 v = (t < rows && k0 + kq < K) ? *reinterpret_cast<const float4*>(gkp + (n0 + t) * K + k0 + kq)
                                                             : make_float4(0, 0, 0, 0);
                    GkT[(kq + 0) * kLB + t] = v.x;
                    GkT[(kq + 1) * kLB + t] = v.y;
                    GkT[(kq + 2) * kLB + t] = v.z;
                    GkT[(kq + 3) * kLB + t] = v.w;
                }
            } else {
                for (int i = tid; i < kBT * kKB; i += kThreads) {
                    const int t = i / kKB, kl = i - t * kKB;
                    GkT[kl * kLB + t] = (t < rows && k0 + kl < K) ? gkp[(n0 + t) * K + k0 + kl] : 0.0f;
                }
            }
            for (int i = tid; i < kKB * (dv / 4); i += kThreads) {
                const int kl = i / (dv / 4), cc = (i - kl * (dv / 4)) * 4, k = k0 + kl;
                *reinterpret_cast<float4*>(Mb + kl * LY + cc) =
                    k < K ? *reinterpret_cast<const float4*>(mp + size_t(k) * dv + cc) : make_float4(0, 0, 0, 0);
            }
            for (int kl = tid; kl < kKB; kl += kThreads) Zb[kl] = k0 + kl < K ? mp[size_t(K) * dv + k0 + kl] : 0.0f;
            __syncthreads();
#pragma unroll 4
            for (int kl = 0; kl < kKB; ++kl) {
                float qa[4], ka[4], ma[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) qa[i] = Gq[(r0 + i) * kLB + kl];
                unpack(lds4(GkT + kl * kLB + m0), ka);
                unpack(lds4(Mb + kl * LY + (m0 < dv ? m0 : 0)), ma);
                const float z = Zb[kl];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dz[i] = fmaf(qa[i], z, dz[i]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        cc4[i][j] = fmaf(qa[i], ka[j], cc4[i][j]);
                        nv[i][j] = fmaf(qa[i], ma[j], nv[i][j]);
                    }
                }
            }
        }
        __syncthreads();  // gamma^K and the memory block are consumed: C and V take their places
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int i = tid + u * kThreads, t = i / (dv / 4), cc = (i - t * (dv / 4)) * 4;
            if (i < kBT * (dv / 4)) *reinterpret_cast<float4*>(Vr + t * LY + cc) = vreg[u];
        }
        // C masked to j <= i; its row sums join D
        float cs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float rsum = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (m0 + j > r0 + i) cc4[i][j] = 0.0f;
                rsum += cc4[i][j];
            }
            cs[i] = sum16(rsum);
            put4(Cm + (r0 + i) * kLB + m0, cc4[i][0], cc4[i][1], cc4[i][2], cc4[i][3]);
            if (r0 + i < rows)
                *reinterpret_cast<float4*>(cbuf + ((size_t(p) * NT + tile) * kBT + r0 + i) * kBT + m0) =
                    make_float4(cc4[i][0], cc4[i][1], cc4[i][2], cc4[i][3]);
        }
        __syncthreads();  // C in LDS
        if (m0 < dv)  // N_i += sum_{j <= i} C_ij V_j
#pragma unroll 4
            for (int jj = 0; jj < rows; ++jj) {
                float ca[4], va[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) ca[i] = Cm[(r0 + i) * kLB + jj];
                unpack(lds4(Vr + jj * LY + m0), va);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) nv[i][j] = fmaf(ca[i], va[j], nv[i][j]);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float dot = 0.0f;
            if (m0 < dv) {
                float oa[4];
                unpack(lds4(Yr + (r0 + i) * LY + m0), oa);
#pragma unroll
                for (int j = 0; j < 4; ++j) dot = fmaf(oa[j], nv[i][j], dot);
            }
            dot = sum16(dot);
            const float D = dz[i] + cs[i] + eps, a = dot / (D * D);
            if ((tid & 15) == 0) {
                Dv[r0 + i] = D;
                Av[r0 + i] = r0 + i < rows ? a : 0.0f;
                if (r0 + i < rows) {
                    rowq[(size_t(p) * N + n0 + r0 + i) * 2] = D;
                    rowq[(size_t(p) * N + n0 + r0 + i) * 2 + 1] = a;
                }
            }
        }
        // what the tile's queries send: gamma^Q_i dO_i / D_i and -gamma^Q_i a'_i (rows k, columns c)
        float* out = tsend + (size_t(p) * NT + tile) * E;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int k0 = kb * kKB;
            __syncthreads();  // Dv, Av visible; the previous block is consumed
            load_gamma_block(gqp, n0, rows, K, k0, Gq);
            __syncthreads();
            float bv[4][4] = {}, bz[4] = {};
#pragma unroll 4
            for (int t = 0; t < rows; ++t) {
                float ga[4], ya[4];
                unpack(lds4(Gq + t * kLB + r0), ga);
                unpack(lds4(Yr + t * LY + (m0 < dv ? m0 : 0)), ya);
                const float rD = 1.0f / Dv[t], a = Av[t];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bz[i] = fmaf(-ga[i], a, bz[i]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) bv[i][j] = fmaf(ga[i], ya[j] * rD, bv[i][j]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = k0 + r0 + i;
                if (k >= K) continue;
                if (m0 < dv)
#pragma unroll
                    for (int j = 0; j < 4; ++j) out[size_t(k) * dv + m0 + j] = bv[i][j];
                if (m0 == 0) out[size_t(K) * dv + k] = bz[i];
            }
        }
    }
}

template <int KB>
size_t kbc_qrows_lds_bytes(int dv) {
    return size_t(kBT * kLB + kKB * kLB + kKB * (dv + 4) + kKB + kBT * (dv + 4) + 2 * kBT) * sizeof(float);
}

// Causal key rows, grid (G, P): dV_j = gamma^K_j . S + sum_{i >= j} C_ij dO'_i (an output) and
// w_j = V_j . dV_j + gamma^K_j . S_Z - sum_{i >= j} C_ij a'_i, S = tsend of the tile (what the
// later tiles' queries send).
template <int KB>
__global__ void __launch_bounds__(kThreads)
    f32_bwdc_kb_krows_kernel(const float* __restrict__ V, const float* __restrict__ dO, int64_t N, int dv, int K,
                             int64_t seg, const float* __restrict__ gk, const float* __restrict__ tsend,
                             const float* __restrict__ cbuf, const float* __restrict__ rowq, float* __restrict__ dV,
                             float* __restrict__ roww) {
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int gi = blockIdx.x;
    const int tid = threadIdx.x, r0 = (tid >> 4) * 4, m0 = (tid & 15) * 4;
    const int LY = dv + 4, NT = int((N + kBT - 1) / kBT);
    const size_t E = size_t(K) * (dv + 1);
    float* Gk = lds;                // [64][kLB] gamma^K of a block, rows j
    float* Sb = Gk + kBT * kLB;     // [kKB][dv + 4] a block of S
    float* Zb = Sb + kKB * LY;      // [kKB]
    float* Cm = Zb + kKB;           // [64][kLB] C of the tile (rows i, columns j)
    float* Yr = Cm + kBT * kLB;     // [64][dv + 4] dO' rows
    float* Av = Yr + kBT * LY;      // [64] a'
    const float* gkp = gk + size_t(p) * N * K;
    const int64_t lo = int64_t(gi) * seg, hi = min<int64_t>(lo + seg, N);
    for (int64_t n0 = lo; n0 < hi; n0 += kBT) {
        const int rows = int(min<int64_t>(kBT, hi - n0)), tile = int(n0 / kBT);
        const float* sp = tsend + (size_t(p) * NT + tile) * E;
        __syncthreads();
        for (int i = tid; i < kBT * (kBT / 4); i += kThreads) {
            const int t = i / (kBT / 4), jq = (i - t * (kBT / 4)) * 4;
            *reinterpret_cast<float4*>(Cm + t * kLB + jq) =
                t < rows ? *reinterpret_cast<const float4*>(cbuf + ((size_t(p) * NT + tile) * kBT + t) * kBT + jq)
                         : make_float4(0, 0, 0, 0);
        }
        for (int t = tid; t < kBT; t += kThreads) Av[t] = t < rows ? rowq[(size_t(p) * N + n0 + t) * 2 + 1] : 0.0f;
        for (int i = tid; i < kBT * (dv / 4); i += kThreads) {
            const int t = i / (dv / 4), cc = (i - t * (dv / 4)) * 4;
            float4 v = make_float4(0, 0, 0, 0);
            if (t < rows) {
                v = *reinterpret_cast<const float4*>(dO + (size_t(p) * N + n0 + t) * dv + cc);
                const float rD = 1.0f / rowq[(size_t(p) * N + n0 + t) * 2];
                v.x *= rD, v.y *= rD, v.z *= rD, v.w *= rD;
            }
            *reinterpret_cast<float4*>(Yr + t * LY + cc) = v;
        }
        float nv[4][4] = {}, ez[4] = {};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int k0 = kb * kKB;
            __syncthreads();  // the previous block is consumed (and the tile's rows are in place)
            load_gamma_block(gkp, n0, rows, K, k0, Gk);
            for (int i = tid; i < kKB * (dv / 4); i += kThreads) {
                const int kl = i / (dv / 4), cc = (i - kl * (dv / 4)) * 4, k = k0 + kl;
                *reinterpret_cast<float4*>(Sb + kl * LY + cc) =
                    k < K ? *reinterpret_cast<const float4*>(sp + size_t(k) * dv + cc) : make_float4(0, 0, 0, 0);
            }
            for (int kl = tid; kl < kKB; kl += kThreads) Zb[kl] = k0 + kl < K ? sp[size_t(K) * dv + k0 + kl] : 0.0f;
            __syncthreads();
#pragma unroll 4
            for (int kl = 0; kl < kKB; ++kl) {
                float ga[4], sa[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) ga[i] = Gk[(r0 + i) * kLB + kl];
                unpack(lds4(Sb + kl * LY + (m0 < dv ? m0 : 0)), sa);
                const float z = Zb[kl];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ez[i] = fmaf(ga[i], z, ez[i]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) nv[i][j] = fmaf(ga[i], sa[j], nv[i][j]);
                }
            }
        }
        // the tile's own queries (i >= j): rows j = r0.. of C's columns
#pragma unroll 4
        for (int i = 0; i < rows; ++i) {
            float ca[4], ya[4];
            unpack(lds4(Cm + i * kLB + r0), ca);
            unpack(lds4(Yr + i * LY + (m0 < dv ? m0 : 0)), ya);
            const float a = Av[i];
#pragma unroll
            for (int jr = 0; jr < 4; ++jr) {
                ez[jr] = fmaf(-ca[jr], a, ez[jr]);
#pragma unroll
                for (int c = 0; c < 4; ++c) nv[jr][c] = fmaf(ca[jr], ya[c], nv[jr][c]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n = n0 + r0 + i;
            float dot = 0.0f;
            if (m0 < dv && r0 + i < rows) {
                const float4 v = *reinterpret_cast<const float4*>(V + (size_t(p) * N + n) * dv + m0);
                dot = v.x * nv[i][0] + v.y * nv[i][1] + v.z * nv[i][2] + v.w * nv[i][3];
                *reinterpret_cast<float4*>(dV + (size_t(p) * N + n) * dv + m0) =
                    make_float4(nv[i][0], nv[i][1], nv[i][2], nv[i][3]);
            }
            dot = sum16(dot);
            if ((tid & 15) == 0 && r0 + i < rows) roww[size_t(p) * N + n] = dot + ez[i];
        }
    }
}

template <int KB>
size_t kbc_krows_lds_bytes(int dv) {
    return size_t(kBT * kLB + kKB * (dv + 4) + kKB + kBT * kLB + kBT * (dv + 4) + kBT) * sizeof(float);
}

size_t kbc_block_lds_bytes(int dr, int dv) {
    return size_t(2 * kBT * kLB + kBT * (dv + 4) + kBT * kLB + kBT * kLB + dv * kLB + kKB + kBT * (dr + 4) +
                  2 * kKB * (dr + 4) + 3 * kBT) *
           sizeof(float);
}

// Causal block passes, grid (G, P, KB): component block kb = blockIdx.z of split g of problem p.
//   QUERY: X = X_Q; own responsibilities gown = gamma^Q, other = gamma^K; tstate: the memory before
//     each tile; w = eps a';
//   key: X = X_K; gown = gamma^K, other = gamma^Q; tstate: what the later tiles' queries send;
//     w = roww.
// Both: the block's entries of the moment record and its share of dX (as the bidirectional pass).
// 4 x TW register tiles over 1024 / TW threads, as the bidirectional block passes.
template <bool QUERY, int TW>
__global__ void __launch_bounds__(1024 / TW)
    f32_bwdc_kb_block_kernel(const float* __restrict__ X, const float* __restrict__ V, const float* __restrict__ dO,
                             int64_t N, int H, int dr, int dv, int K, int64_t seg, int G, const double* __restrict__ inv,
                             const float* __restrict__ mu, const float* __restrict__ tstate, float eps,
                             const float* __restrict__ gown, const float* __restrict__ gother,
                             const float* __restrict__ rowq, const float* __restrict__ roww,
                             float* __restrict__ param_part, float* __restrict__ dX_part) {
    constexpr int NTH = 1024 / TW, CG = 64 / TW;  // threads; column groups of a row group
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int gi = blockIdx.x, kb = blockIdx.z, h = int(p % H);
    const int tid = threadIdx.x, r0 = (tid / CG) * 4, m0 = (tid % CG) * TW;
    const int LY = dv + 4, LX = dr + 4, k0 = kb * kKB, NT = int((N + kBT - 1) / kBT);
    const size_t E = size_t(K) * (dv + 1);
    float* Gb = lds;                  // [64][kLB] own responsibilities of the block
    float* Go = Gb + kBT * kLB;       // [64][kLB] the other side's, same positions
    float* Yr = Go + kBT * kLB;       // [64][dv + 4] dO' rows
    float* VD = Yr + kBT * LY;        // [64][kLB]: V^T ([dv][.]) until g is formed, then ds
    float* Am = VD + kBT * kLB;       // [64][kLB] A (rows i, columns j)
    float* MT = Am + kBT * kLB;       // [dv][kLB] the tile's state block, transposed
    float* Zb = MT + dv * kLB;        // [kKB]
    float* Xr = Zb + kKB;             // [64][dr + 4] x rows
    float* muR = Xr + kBT * LX;       // [kKB][dr + 4] mu of the block
    float* ivR = muR + kKB * LX;      // [kKB][dr + 4] 1 / sigma2 of the block
    float* Av = ivR + kKB * LX;       // [64] a'
    float* Wv = Av + kBT;             // [64] w
    float* Dv = Wv + kBT;             // [64] D
    const double* ih = inv + size_t(h) * K * dr;
    const float* mh = mu + size_t(h) * K * dr;
    for (int i = tid; i < kKB * dr; i += NTH) {
        const int kl = i / dr, d = i - kl * dr, k = k0 + kl;
        muR[kl * LX + d] = k < K ? mh[size_t(k) * dr + d] : 0.0f;
        ivR[kl * LX + d] = k < K ? float(ih[size_t(k) * dr + d]) : 0.0f;
    }
    __syncthreads();
    const bool mom = r0 < dr;
    float mreg[4][TW], s1[4][TW] = {}, s2[4][TW] = {}, s0[TW] = {};
    if (mom)
#pragma unroll
        for (int j = 0; j < TW; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) mreg[i][j] = muR[(m0 + j) * LX + r0 + i];
    const int64_t lo = int64_t(gi) * seg, hi = min<int64_t>(lo + seg, N);
    const float* Xp = X + size_t(p) * N * dr;
    const float* gop = gown + size_t(p) * N * K;
    const float* gtp = gother + size_t(p) * N * K;
    float* dXp = dX_part + (size_t(kb) * gridDim.y + p) * N * dr;
    for (int64_t n0 = lo; n0 < hi; n0 += kBT) {
        const int rows = int(min<int64_t>(kBT, hi - n0)), tile = int(n0 / kBT);
        const float* mp = tstate + (size_t(p) * NT + tile) * E;
        __syncthreads();  // the previous tile's reads are done
        load_gamma_block_n<NTH>(gop, n0, rows, K, k0, Gb);
        load_gamma_block_n<NTH>(gtp, n0, rows, K, k0, Go);
        for (int t = tid; t < kBT; t += NTH) {
            const float D = t < rows ? rowq[(size_t(p) * N + n0 + t) * 2] : 1.0f;
            const float a = t < rows ? rowq[(size_t(p) * N + n0 + t) * 2 + 1] : 0.0f;
            Dv[t] = D;
            Av[t] = a;
            Wv[t] = QUERY ? eps * a : (t < rows ? roww[size_t(p) * N + n0 + t] : 0.0f);
        }
        for (int i = tid; i < kBT * (dr / 4); i += NTH) {
            const int t = i / (dr / 4), d = (i - t * (dr / 4)) * 4;
            *reinterpret_cast<float4*>(Xr + t * LX + d) =
                t < rows ? *reinterpret_cast<const float4*>(Xp + (n0 + t) * dr + d) : make_float4(0, 0, 0, 0);
        }
        load_mem_block_t<NTH>(mp, K, dv, k0, MT);
        for (int kl = tid; kl < kKB; kl += NTH) Zb[kl] = k0 + kl < K ? mp[size_t(K) * dv + k0 + kl] : 0.0f;
        __syncthreads();  // Dv before the scaled rows
        for (int i = tid; i < kBT * (dv / 4); i += NTH) {
            const int t = i / (dv / 4), cc = (i - t * (dv / 4)) * 4;
            float4 o = make_float4(0, 0, 0, 0), v = o;
            if (t < rows) {
                const size_t off = (size_t(p) * N + n0 + t) * dv + cc;
                o = *reinterpret_cast<const float4*>(dO + off);
                v = *reinterpret_cast<const float4*>(V + off);
                const float rD = 1.0f / Dv[t];
                o.x *= rD, o.y *= rD, o.z *= rD, o.w *= rD;
            }
            *reinterpret_cast<float4*>(Yr + t * LY + cc) = o;
            VD[(cc + 0) * kLB + t] = v.x;
            VD[(cc + 1) * kLB + t] = v.y;
            VD[(cc + 2) * kLB + t] = v.z;
            VD[(cc + 3) * kLB + t] = v.w;
        }
        __syncthreads();
        {   // A_ij = dO'_i . V_j - a'_i for j <= i (rows i = r0.., columns j = m0..)
            float aa[4][TW] = {};
#pragma unroll 4
            for (int cc = 0; cc < dv; ++cc) {
                float ya[4], va[TW];
#pragma unroll
                for (int i = 0; i < 4; ++i) ya[i] = Yr[(r0 + i) * LY + cc];
                ldsw<TW>(VD + cc * kLB + m0, va);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) aa[i][j] = fmaf(ya[i], va[j], aa[i][j]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float o[TW];
#pragma unroll
                for (int j = 0; j < TW; ++j)
                    o[j] = (m0 + j <= r0 + i && r0 + i < rows && m0 + j < rows) ? aa[i][j] - Av[r0 + i] : 0.0f;
                stsw<TW>(Am + (r0 + i) * kLB + m0, o);
            }
        }
        __syncthreads();  // A in LDS
        float gg[4][TW] = {};
        if (QUERY) {  // rows i = r0.., components k = m0..
#pragma unroll 4
            for (int cc = 0; cc < dv; ++cc) {
                float ya[4], ma[TW];
#pragma unroll
                for (int i = 0; i < 4; ++i) ya[i] = Yr[(r0 + i) * LY + cc];
                ldsw<TW>(MT + cc * kLB + m0, ma);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) gg[i][j] = fmaf(ya[i], ma[j], gg[i][j]);
            }
#pragma unroll 4
            for (int jj = 0; jj < rows; ++jj) {  // sum_{j <= i} A_ij gamma^K_jk
                float aa[4], ka[TW];
#pragma unroll
                for (int i = 0; i < 4; ++i) aa[i] = Am[(r0 + i) * kLB + jj];
                ldsw<TW>(Go + jj * kLB + m0, ka);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) gg[i][j] = fmaf(aa[i], ka[j], gg[i][j]);
            }
        } else {  // rows j = r0.., components k = m0..
#pragma unroll 4
            for (int cc = 0; cc < dv; ++cc) {
                float va[4], ma[TW];
                unpack(lds4(VD + cc * kLB + r0), va);
                ldsw<TW>(MT + cc * kLB + m0, ma);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) gg[i][j] = fmaf(va[i], ma[j], gg[i][j]);
            }
#pragma unroll 4
            for (int ii = 0; ii < rows; ++ii) {  // sum_{i >= j} A_ij gamma^Q_ik
                float aa[4], qa[TW];
                unpack(lds4(Am + ii * kLB + r0), aa);
                ldsw<TW>(Go + ii * kLB + m0, qa);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) gg[i][j] = fmaf(aa[i], qa[j], gg[i][j]);
            }
        }
        float za[TW];
        ldsw<TW>(Zb + m0, za);
        float ds[4][TW];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float ga[TW];
            ldsw<TW>(Gb + (r0 + i) * kLB + m0, ga);
            const float w = Wv[r0 + i];
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                const float g = QUERY ? gg[i][j] - Av[r0 + i] * za[j] : gg[i][j] + za[j];
                ds[i][j] = ga[j] * (g - w);
            }
        }
        __syncthreads();  // V^T is consumed: ds takes its place
#pragma unroll
        for (int i = 0; i < 4; ++i) stsw<TW>(VD + (r0 + i) * kLB + m0, ds[i]);
        __syncthreads();  // ds in LDS
        if (mom)  // moments (rows d = r0.., columns k = m0..), direct (centred) form
#pragma unroll 4
            for (int t = 0; t < rows; ++t) {
                float xa[4], da[TW];
                unpack(lds4(Xr + t * LX + r0), xa);
                ldsw<TW>(VD + t * kLB + m0, da);
#pragma unroll
                for (int j = 0; j < TW; ++j) {
                    s0[j] += da[j];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float df = xa[i] - mreg[i][j], w = da[j] * df;
                        s1[i][j] += w;
                        s2[i][j] = fmaf(w, df, s2[i][j]);
                    }
                }
            }
        if (m0 < dr) {  // this block's share of dX (rows t = r0.., columns d = m0..)
            float xa[4][TW], acc[4][TW] = {};
#pragma unroll
            for (int i = 0; i < 4; ++i) ldsw<TW>(Xr + (r0 + i) * LX + m0, xa[i]);
            const int kn = min(kKB, K - k0);
#pragma unroll 4
            for (int kl = 0; kl < kn; ++kl) {
                float ma[TW], ia[TW], da[4];
                ldsw<TW>(muR + kl * LX + m0, ma);
                ldsw<TW>(ivR + kl * LX + m0, ia);
#pragma unroll
                for (int i = 0; i < 4; ++i) da[i] = VD[(r0 + i) * kLB + kl];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) acc[i][j] = fmaf(da[i] * ia[j], xa[i][j] - ma[j], acc[i][j]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (r0 + i < rows) {
                    float o[TW];
#pragma unroll
                    for (int j = 0; j < TW; ++j) o[j] = -acc[i][j];
                    stsw<TW>(dXp + (n0 + r0 + i) * dr + m0, o);
                }
        }
    }
    float* pp = param_part + (size_t(p) * G + gi) * size_t(2 * K * dr + K);
    if (mom)
#pragma unroll
        for (int j = 0; j < TW; ++j) {
            const int k = k0 + m0 + j;
            if (k >= K) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pp[size_t(k) * dr + r0 + i] = s1[i][j];
                pp[size_t(K) * dr + size_t(k) * dr + r0 + i] = s2[i][j];
            }
            if (r0 == 0) pp[2 * size_t(K) * dr + k] = s0[j];
        }
}

// Grid (G segments, P).  QUERY walks the segment's tiles forward from the memory before the
// segment (state: [Vt (K dv) | Z (K)]), writes dX_Q, D_i and a_i of every row (rowda), the
// segment's total of what its queries send to the memory (seg_part) and its moments.  KEY walks
// the tiles backward from what the later segments' queries sent (state), writes dX_K, dV and its
// moments.  FAST: the per-head tables (fp32) live in LDS (rows padded by one element), and the
// running memory too when mem_lds is set; the scores, dX and moments are fp32.  Otherwise the
// tables are the fp64 ones, and a memory outside LDS is advanced in place in the workspace.
template <bool QUERY, bool FAST>
__global__ void __launch_bounds__(kThreads)
    f32_bwdc_kernel(const float* __restrict__ XQ, const float* __restrict__ XK, const float* __restrict__ V,
                    const float* __restrict__ dO, int64_t N, int H, int dr, int dv, int K, int64_t seg, int G, int T,
                    const double* c, const double* inv, const float* mu, float* state, float eps,
                    float* __restrict__ rowda, float* __restrict__ dX, float* __restrict__ dV,
                    float* __restrict__ seg_part, float* __restrict__ param_part, int mem_lds) {
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int gi = blockIdx.x, h = int(p % H);
    float* xs = lds;          // T*dr: scratch of gamma_tile; left holding this side's rows
    float* gq = xs + T * dr;  // T*K
    float* gk = gq + T * K;   // T*K
    float* gg = gk + T * K;   // T*K: upstream gradient, then ds
    float* ys = gg + T * K;   // T*dv: dO
    float* vs = ys + T * dv;  // T*dv: V
    float* Cm = vs + T * dv;  // T*T
    float* Am = Cm + T * T;   // T*T
    float* dd = Am + T * T;   // T: D_i
    float* aa = dd + T;       // T: a_i
    const int LR = dr + 1, LV = dv + 1;
    float* mT = aa + T;             // FAST: [K][LR] mu
    float* iT = mT + K * LR;        // FAST: [K][LR] 1 / sigma2
    float* cT = iT + K * LR;        // FAST: [K] score constants
    float* Sm = cT + K;             // FAST: [K][LV] running memory (Vt or dVt)
    float* Sz = Sm + K * LV;        // FAST: [K] its Z (or dZ)
    const double *ch = c + size_t(h) * K, *ih = inv + size_t(h) * K * dr;
    const float* mh = mu + size_t(h) * K * dr;
    const int E = K * (dv + 1), PE = 2 * K * dr + K;
    float* Sg = state + (size_t(p) * G + gi) * E;  // [K][dv], then Z
    // the running memory: LDS rows of LV or the workspace record
    const bool ML = FAST && mem_lds;
    float* St = ML ? Sm : Sg;
    float* Zs = ML ? Sz : Sg + size_t(K) * dv;
    const int SL = ML ? LV : dv;
    if (FAST) {
        for (int i = threadIdx.x; i < K * dr; i += kThreads) {
            const int k = i / dr, d = i - k * dr;
            mT[k * LR + d] = mh[i];
            iT[k * LR + d] = float(ih[i]);
        }
        for (int k = threadIdx.x; k < K; k += kThreads) {
            cT[k] = float(ch[k]);
            if (ML) Sz[k] = Sg[K * dv + k];
        }
        if (ML)
            for (int i = threadIdx.x; i < K * dv; i += kThreads) Sm[(i / dv) * LV + i % dv] = Sg[i];
        __syncthreads();
    }
    float* sp = QUERY ? seg_part + (size_t(p) * G + gi) * E : nullptr;
    float* pp = param_part + (size_t(p) * G + gi) * PE;
    const int64_t lo = int64_t(gi) * seg, hi = min<int64_t>(lo + seg, N);
    const int ntiles = int((hi - lo + T - 1) / T);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    bool first = true;
    for (int it = 0; it < ntiles; ++it) {
        const int64_t n0 = lo + int64_t(QUERY ? it : ntiles - 1 - it) * T;
        const int rows = int(min<int64_t>(T, hi - n0));
        // responsibilities; the side's own rows are left in xs
        if (FAST) {
            gamma_tile_lds(QUERY ? XK + p * N * dr : XQ + p * N * dr, n0, rows, T, dr, K, cT, iT, mT, xs,
                           QUERY ? gk : gq);
            gamma_tile_lds(QUERY ? XQ + p * N * dr : XK + p * N * dr, n0, rows, T, dr, K, cT, iT, mT, xs,
                           QUERY ? gq : gk);
        } else if (QUERY) {
            gamma_tile(XK + p * N * dr, n0, rows, T, dr, K, ch, ih, mh, xs, gk);
            gamma_tile(XQ + p * N * dr, n0, rows, T, dr, K, ch, ih, mh, xs, gq);
        } else {
            gamma_tile(XQ + p * N * dr, n0, rows, T, dr, K, ch, ih, mh, xs, gq);
            gamma_tile(XK + p * N * dr, n0, rows, T, dr, K, ch, ih, mh, xs, gk);
        }
        for (int i = threadIdx.x; i < T * dv; i += kThreads) {
            const int t = i / dv;
            ys[i] = t < rows ? dO[(p * N + n0) * dv + i] : 0.0f;
            vs[i] = t < rows ? V[(p * N + n0) * dv + i] : 0.0f;
        }
        if (!QUERY)
            for (int t = threadIdx.x; t < T; t += kThreads) {
                dd[t] = t < rows ? rowda[(p * N + n0 + t) * 2 + 0] : 1.0f;
                aa[t] = t < rows ? rowda[(p * N + n0 + t) * 2 + 1] : 0.0f;
            }
        // C_ij = gamma^Q_i . gamma^K_j (j <= i)
        for (int e = threadIdx.x; e < T * T; e += kThreads) {
            const int i = e / T, j = e - i * T;
            float acc = 0.0f;
            if (j <= i && i < rows)
                for (int k = 0; k < K; ++k) acc = fmaf(gq[i * K + k], gk[j * K + k], acc);
            Cm[e] = acc;
        }
        __syncthreads();
        if (QUERY) {  // D_i and a_i from the memory at the tile's start and the tile's own keys
            for (int t = wave; t < rows; t += kThreads / kWave) {
                float d = 0.0f;
                for (int k = lane; k < K; k += kWave) d = fmaf(gq[t * K + k], Zs[k], d);
                for (int j = lane; j <= t; j += kWave) d += Cm[t * T + j];
                d = wave_sum(d) + eps;
                float a = 0.0f;
                for (int cc = lane; cc < dv; cc += kWave) {
                    float nn = 0.0f;
                    for (int k = 0; k < K; ++k) nn = fmaf(gq[t * K + k], St[size_t(k) * SL + cc], nn);
                    for (int j = 0; j <= t; ++j) nn = fmaf(Cm[t * T + j], vs[j * dv + cc], nn);
                    a = fmaf(ys[t * dv + cc], nn / d, a);
                }
                a = wave_sum(a);
                if (lane == 0) {
                    dd[t] = d;
                    aa[t] = a;
                    rowda[(p * N + n0 + t) * 2 + 0] = d;
                    rowda[(p * N + n0 + t) * 2 + 1] = a;
                }
            }
            __syncthreads();
        }
        // A_ij = (dO_i . V_j - a_i) / D_i (j <= i)
        for (int e = threadIdx.x; e < T * T; e += kThreads) {
            const int i = e / T, j = e - i * T;
            float acc = 0.0f;
            if (j <= i && i < rows) {
                for (int cc = 0; cc < dv; ++cc) acc = fmaf(ys[i * dv + cc], vs[j * dv + cc], acc);
                acc = (acc - aa[i]) / dd[i];
            }
            Am[e] = acc;
        }
        __syncthreads();
        if (QUERY) {  // g^Q
            for (int e = threadIdx.x; e < T * K; e += kThreads) {
                const int t = e / K, k = e - t * K;
                float acc = 0.0f;
                if (t < rows) {
                    for (int cc = 0; cc < dv; ++cc) acc = fmaf(ys[t * dv + cc], St[size_t(k) * SL + cc], acc);
                    acc = (acc - aa[t] * Zs[k]) / dd[t];
                    for (int j = 0; j <= t; ++j) acc = fmaf(Am[t * T + j], gk[j * K + k], acc);
                }
                gg[e] = acc;
            }
        } else {  // dV and g^K from the memory gradient after the tile and the tile's own queries
            for (int e = threadIdx.x; e < rows * dv; e += kThreads) {
                const int j = e / dv, cc = e - j * dv;
                float acc = 0.0f;
                for (int k = 0; k < K; ++k) acc = fmaf(gk[j * K + k], St[size_t(k) * SL + cc], acc);
                for (int i = j; i < rows; ++i) acc = fmaf(Cm[i * T + j], ys[i * dv + cc] / dd[i], acc);
                dV[(p * N + n0) * dv + e] = acc;
            }
            for (int e = threadIdx.x; e < T * K; e += kThreads) {
                const int j = e / K, k = e - j * K;
                float acc = 0.0f;
                if (j < rows) {
                    for (int cc = 0; cc < dv; ++cc) acc = fmaf(vs[j * dv + cc], St[size_t(k) * SL + cc], acc);
                    acc += Zs[k];
                    for (int i = j; i < rows; ++i) acc = fmaf(Am[i * T + j], gq[i * K + k], acc);
                }
                gg[e] = acc;
            }
        }
        __syncthreads();
        // Eq. 18 with this side's responsibilities, one wave per row
        const float* gm = QUERY ? gq : gk;
        for (int t = wave; t < T; t += kThreads / kWave) {
            float w = 0.0f;
            for (int k = lane; k < K; k += kWave) w = fmaf(gm[t * K + k], gg[t * K + k], w);
            w = wave_sum(w);
            for (int k = lane; k < K; k += kWave) gg[t * K + k] = gm[t * K + k] * (gg[t * K + k] - w);
        }
        __syncthreads();
        // routing-vector gradient
        for (int i = threadIdx.x; i < rows * dr; i += kThreads) {
            const int t = i / dr, d = i - t * dr;
            float acc = 0.0f;
            if (FAST) {
                const float x = xs[t * dr + d];
                for (int k = 0; k < K; ++k) acc = fmaf(gg[t * K + k] * iT[k * LR + d], x - mT[k * LR + d], acc);
            } else {
                for (int k = 0; k < K; ++k)
                    acc = fmaf(gg[t * K + k], float((double(xs[t * dr + d]) - double(mh[size_t(k) * dr + d])) * ih[size_t(k) * dr + d]), acc);
            }
            dX[(p * N + n0) * dr + i] = -acc;
        }
        // moments of these rows
        for (int e = threadIdx.x; e < K * dr; e += kThreads) {
            const int k = e / dr, d = e - k * dr;
            float a1, a2;
            if (FAST) {
                const float m = mT[k * LR + d];
                a1 = 0.0f, a2 = 0.0f;
                for (int t = 0; t < rows; ++t) {
                    const float df = xs[t * dr + d] - m, w = gg[t * K + k] * df;
                    a1 += w;
                    a2 = fmaf(w, df, a2);
                }
            } else {
                const double m = double(mh[e]);
                double b1 = 0.0, b2 = 0.0;
                for (int t = 0; t < rows; ++t) {
                    const double df = double(xs[t * dr + d]) - m, w = double(gg[t * K + k]) * df;
                    b1 += w;
                    b2 += w * df;
                }
                a1 = float(b1), a2 = float(b2);
            }
            pp[e] = first ? a1 : pp[e] + a1;
            pp[K * dr + e] = first ? a2 : pp[K * dr + e] + a2;
        }
        for (int k = threadIdx.x; k < K; k += kThreads) {
            float acc = 0.0f;
            for (int t = 0; t < rows; ++t) acc += gg[t * K + k];
            pp[2 * K * dr + k] = first ? acc : pp[2 * K * dr + k] + acc;
        }
        __syncthreads();  // every read of the memory for this tile is done
        // advance the memory past the tile: QUERY adds the tile's keys (Eq. 6b) and totals what
        // its queries send; KEY adds what the tile's queries send
        for (int e = threadIdx.x; e < E; e += kThreads) {
            float qsum = 0.0f, ksum = 0.0f;
            if (e < K * dv) {
                const int k = e / dv, cc = e - k * dv;
                for (int t = 0; t < rows; ++t) {
                    qsum = fmaf(gq[t * K + k], ys[t * dv + cc] / dd[t], qsum);
                    if (QUERY) ksum = fmaf(gk[t * K + k], vs[t * dv + cc], ksum);
                }
            } else {
                const int k = e - K * dv;
                for (int t = 0; t < rows; ++t) {
                    qsum -= gq[t * K + k] * aa[t] / dd[t];
                    if (QUERY) ksum += gk[t * K + k];
                }
            }
            // element e of the [Vt | Z] record in the running memory's layout
            float& m = e < K * dv ? St[(e / dv) * SL + e % dv] : Zs[e - K * dv];
            if (QUERY) {
                m += ksum;
                sp[e] = first ? qsum : sp[e] + qsum;
            } else {
                m += qsum;
            }
        }
        first = false;
        __syncthreads();  // the memory and the tile's LDS are ready for the next tile
    }
    if (first) {  // empty segment
        for (int e = threadIdx.x; e < PE; e += kThreads) pp[e] = 0.0f;
        if (QUERY)
            for (int e = threadIdx.x; e < E; e += kThreads) sp[e] = 0.0f;
    }
}

}  // namespace

// The causal passes take the register-tiled form where the LDS holds it.
bool bwdc_tiled_applies(const Plan& p) {
    const int K = int(p.K), dr = int(p.dr), dv = int(p.dv);
    return bwd_tiled_applies(p) && bwd_tiled_lds_bytes(BWD_CQUERY, K, dr, dv) <= kMaxLds &&
           bwd_tiled_lds_bytes(BWD_CKEY, K, dr, dv) <= kMaxLds;
}

// The K-blocked causal passes where the register-tiled ones do not fit.
bool bwdc_kb_applies(const Plan& p) {
    return !bwdc_tiled_applies(p) && p.K <= 256 && p.dr % 4 == 0 && p.dv % 4 == 0 && p.dr <= 64 && p.dv <= 64 &&
           p.N > 0;
}

namespace {

// The K-blocked causal passes' buffers: per tile of 64 positions the memory before it and what
// the later tiles' queries send ([P][NT][K (dv + 1)] each, NT = ceil(N / 64)) and C
// ([P][NT][64][64]); the responsibilities of both sides ([P][N][K]), (D, a') per row, w per key
// row and the blocks' shares of dX ([KB][P][N][dr]).
struct KbcBuffers {
    float *tmem, *tsend, *cbuf, *gq, *gk, *rowq, *roww, *dxpart;
};
size_t kbc_bytes(const Plan& p, KbcBuffers* b, char* base) {
    const size_t P = size_t(p.P), K = size_t(p.K), N = size_t(p.N), NT = (N + kBT - 1) / kBT;
    const size_t E = K * size_t(p.dv + 1);
    const size_t sizes[8] = {round_up(P * NT * E * 4, 256),         round_up(P * NT * E * 4, 256),
                             round_up(P * NT * kBT * kBT * 4, 256), round_up(P * N * K * 4, 256),
                             round_up(P * N * K * 4, 256),          round_up(P * N * 2 * 4, 256),
                             round_up(P * N * 4, 256),
                             round_up(size_t(kb_blocks(p.K)) * P * N * size_t(p.dr) * 4, 256)};
    float** outs[8] = {b ? &b->tmem : nullptr, b ? &b->tsend : nullptr, b ? &b->cbuf : nullptr,
                       b ? &b->gq : nullptr,   b ? &b->gk : nullptr,    b ? &b->rowq : nullptr,
                       b ? &b->roww : nullptr, b ? &b->dxpart : nullptr};
    size_t off = 0;
    for (int i = 0; i < 8; ++i) {
        if (b) *outs[i] = reinterpret_cast<float*>(base + off);
        off += sizes[i];
    }
    return off;
}

template <typename F>
hipError_t with_kbc(int KB, F&& f) {
    if (KB == 1) return f(std::integral_constant<int, 1>());
    return with_kb(KB, f);
}

template <int KB>
hipError_t kbc_allow_lds_for() {
    const void* fns[] = {(const void*)f32_bwd_kb_rows_kernel<KB, KB_KEY, kRowsTW>, (const void*)f32_bwd_kb_rows_kernel<KB, KB_GAMMA, kRowsTW>,
                         (const void*)f32_bwdc_kb_qrows_kernel<KB>, (const void*)f32_bwdc_kb_krows_kernel<KB>};
    for (const void* f : fns) {
        hipError_t r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxLds));
        if (r != hipSuccess) return r;
    }
    return hipSuccess;
}

hipError_t kbc_allow_lds() {
    static const hipError_t e = [] {
        hipError_t r;
        if ((r = kbc_allow_lds_for<1>()) != hipSuccess || (r = kbc_allow_lds_for<2>()) != hipSuccess ||
            (r = kbc_allow_lds_for<3>()) != hipSuccess || (r = kbc_allow_lds_for<4>()) != hipSuccess)
            return r;
        const void* fns[] = {(const void*)f32_bwdc_kb_block_kernel<true, kBlockTW>,
                             (const void*)f32_bwdc_kb_block_kernel<false, kBlockTW>};
        for (const void* f : fns)
            if ((r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxLds))) != hipSuccess)
                return r;
        return hipSuccess;
    }();
    return e;
}

// The causal backward in K-blocked passes: tile aggregates of the key side (and Gamma_K), their
// exclusive prefix from state_in, Gamma_Q, the causal query rows (C, D, a', what each tile's
// queries send), its exclusive suffix from dstate_out (the total into dstate_in), the query
// blocks, the key rows (dV, w) and the key blocks.
hipError_t f32_backward_causal_kb(const Plan& p, const float* XQ, const float* XK, const float* V, const float* mu,
                                  const float* pi, float eps, const float* dO, float* dXQ, float* dXK, float* dV,
                                  float* dmu, float* ds2, float* dpi, const F32Params& v, float* ppart,
                                  float* ppart_key, char* kbase, hipStream_t st, const float* state_in,
                                  const float* dstate_out, float* dstate_in) {
    hipError_t e = kbc_allow_lds();
    if (e != hipSuccess) return e;
    KbcBuffers b{};
    kbc_bytes(p, &b, kbase);
    const int H = int(p.H), dr = int(p.dr), dv = int(p.dv), K = int(p.K), KB = kb_blocks(p.K);
    const int NT = int((p.N + kBT - 1) / kBT), Ei = int(size_t(p.K) * size_t(p.dv + 1));
    const int64_t tseg = kBT;
    const BlockSplit bs = block_split(p, KB);
    const dim3 tgrid(unsigned(NT), unsigned(p.P)), bgrid(unsigned(bs.G), unsigned(p.P), unsigned(KB));
    // the key side's moment records follow the query side's P bs.G ones
    ppart_key = ppart + size_t(p.P) * size_t(bs.G) * size_t(2 * p.K * p.dr + p.K);
    const dim3 egrid(unsigned((Ei + kThreads - 1) / kThreads), unsigned(p.P));
    const float* cnone = nullptr;
    float* none = nullptr;
    const size_t blds = kbc_block_lds_bytes(dr, dv);
    auto sum_dx = [&](float* dX) {
        const size_t n = size_t(p.P) * size_t(p.N) * size_t(dr);
        GMA_LAUNCH("f32_bwd_dx_sum", f32_bwd_kb_sum_kernel, dim3(unsigned((n / 4 + kThreads - 1) / kThreads)),
                   dim3(kThreads), 0, st, static_cast<const float*>(b.dxpart), KB, n, dX);
        return hipGetLastError();
    };
    return with_kbc(KB, [&](auto KBc) -> hipError_t {
        constexpr int KBT = decltype(KBc)::value;
        const size_t rlds = kb_rows_lds_bytes<KBT>(dr, dv);
        hipError_t r;
        GMA_LAUNCH("f32_bwdc_kb_aggregate", (f32_bwd_kb_rows_kernel<KBT, KB_KEY, kRowsTW>), tgrid, dim3(1024 / kRowsTW), rlds, st, XK, V,
                   p.N, H, dr, dv, K, tseg, NT, v.c, v.inv, mu, cnone, eps, b.gk, b.tmem, none);
        if ((r = hipGetLastError()) != hipSuccess) return r;
        GMA_LAUNCH("f32_bwdc_prefix", f32_prefix_kernel, egrid, dim3(kThreads), 0, st, b.tmem, NT, Ei, state_in, K, dv);
        if ((r = hipGetLastError()) != hipSuccess) return r;
        GMA_LAUNCH("f32_bwdc_kb_query_gamma", (f32_bwd_kb_rows_kernel<KBT, KB_GAMMA, kRowsTW>), tgrid, dim3(1024 / kRowsTW), rlds, st,
                   XQ, cnone, p.N, H, dr, dv, K, tseg, NT, v.c, v.inv, mu, cnone, eps, b.gq, none, none);
        if ((r = hipGetLastError()) != hipSuccess) return r;
        GMA_LAUNCH("f32_bwdc_kb_query_rows", f32_bwdc_kb_qrows_kernel<KBT>, tgrid, dim3(kThreads),
                   kbc_qrows_lds_bytes<KBT>(dv), st, V, dO, p.N, dv, K, tseg, static_cast<const float*>(b.gq),
                   static_cast<const float*>(b.gk), static_cast<const float*>(b.tmem), eps, b.cbuf, b.rowq, b.tsend);
        if ((r = hipGetLastError()) != hipSuccess) return r;
        GMA_LAUNCH("f32_bwdc_suffix", f32_suffix_kernel, egrid, dim3(kThreads), 0, st, b.tsend, NT, Ei, dstate_out,
                   dstate_in, K, dv);
        if ((r = hipGetLastError()) != hipSuccess) return r;
        GMA_LAUNCH("f32_bwdc_kb_query", (f32_bwdc_kb_block_kernel<true, kBlockTW>), bgrid, dim3(1024 / kBlockTW), blds, st, XQ, V, dO, p.N,
                   H, dr, dv, K, bs.seg, bs.G, v.inv, mu, static_cast<const float*>(b.tmem), eps,
                   static_cast<const float*>(b.gq), static_cast<const float*>(b.gk), static_cast<const float*>(b.rowq),
                   cnone, ppart, b.dxpart);
        if ((r = hipGetLastError()) != hipSuccess) return r;
        if ((r = sum_dx(dXQ)) != hipSuccess) return r;
        GMA_LAUNCH("f32_bwdc_kb_key_rows", f32_bwdc_kb_krows_kernel<KBT>, tgrid, dim3(kThreads), kbc_krows_lds_bytes<KBT>(dv),
                   st, V, dO, p.N, dv, K, tseg, static_cast<const float*>(b.gk), static_cast<const float*>(b.tsend),
                   static_cast<const float*>(b.cbuf), static_cast<const float*>(b.rowq), dV, b.roww);
        if ((r = hipGetLastError()) != hipSuccess) return r;
        GMA_LAUNCH("f32_bwdc_kb_key", (f32_bwdc_kb_block_kernel<false, kBlockTW>), bgrid, dim3(1024 / kBlockTW), blds, st, XK, V, dO, p.N,
                   H, dr, dv, K, bs.seg, bs.G, v.inv, mu, static_cast<const float*>(b.tsend), eps,
                   static_cast<const float*>(b.gk), static_cast<const float*>(b.gq), static_cast<const float*>(b.rowq),
                   static_cast<const float*>(b.roww), ppart_key, b.dxpart);
        if ((r = hipGetLastError()) != hipSuccess) return r;
        if ((r = sum_dx(dXK)) != hipSuccess) return r;
        return reduce_params_split(p, bs.G, ppart, v.inv, pi, dmu, ds2, dpi, st);
    });
}

}  // namespace

size_t f32_backward_causal_extra_bytes(const Plan& p) {
    const size_t E = size_t(p.K) * size_t(p.dv + 1);
    return round_up(size_t(p.P * p.G) * E * 4, 256) + round_up(size_t(p.P * p.N) * 2 * 4, 256) +
           round_up(2 * size_t(p.P * p.G) * size_t(2 * p.K * p.dr + p.K) * 4, 256) +
           (bwdc_tiled_applies(p) ? 2 * gamma_cache_bytes(p) : 0) + (bwdc_kb_applies(p) ? kbc_bytes(p, nullptr, nullptr) : 0);
}

hipError_t f32_backward_causal(const Plan& p, const float* XQ, const float* XK, const float* V, const float* mu,
                               const float* s2, const float* pi, float eps, const float* dO, float* dXQ, float* dXK,
                               float* dV, float* dmu, float* ds2, float* dpi, char* ws, hipStream_t st,
                               const float* state_in, const float* dstate_out, float* dstate_in) {
    if (p.H == 0) return hipSuccess;
    if (p.P == 0) return reduce_params(p, nullptr, 0, nullptr, pi, dmu, ds2, dpi, st);
    if (p.N == 0) {  // no positions: zero parameter gradients, and the memory passes its gradient through
        hipError_t e0 = reduce_params(p, nullptr, 0, nullptr, pi, dmu, ds2, dpi, st);
        if (e0 != hipSuccess || !dstate_in) return e0;
        return copy_state(p, dstate_out, dstate_in, st);
    }
    static const hipError_t attr = [] {
        const void* fns[] = {(const void*)f32_bwdc_kernel<true, false>, (const void*)f32_bwdc_kernel<false, false>,
                             (const void*)f32_bwdc_kernel<true, true>, (const void*)f32_bwdc_kernel<false, true>};
        for (const void* f : fns) {
            hipError_t r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxLds));
            if (r != hipSuccess) return r;
        }
        return hipSuccess;
    }();
    if (attr != hipSuccess) return attr;
    hipError_t e = bwd_allow_lds();
    if (e != hipSuccess) return e;
    if ((e = launch_param_tables(p, s2, pi, ws, st)) != hipSuccess) return e;
    F32Params v = f32_params_view(p, ws);
    float* states = reinterpret_cast<float*>(ws + p.off_partials);  // segment aggregates, then running memories
    const size_t E = size_t(p.K) * size_t(p.dv + 1);
    char* extra = ws + p.off_stage - f32_backward_causal_extra_bytes(p);
    float* seg_part = reinterpret_cast<float*>(extra);
    float* rowda = reinterpret_cast<float*>(extra + round_up(size_t(p.P * p.G) * E * 4, 256));
    float* ppart = reinterpret_cast<float*>(extra + round_up(size_t(p.P * p.G) * E * 4, 256) +
                                            round_up(size_t(p.P * p.N) * 2 * 4, 256));
    float* ppart_key = ppart + size_t(p.P * p.G) * size_t(2 * p.K * p.dr + p.K);
    // Gamma_K (from the aggregate pass) and Gamma_Q (from the query pass) for the tiled passes
    float* gk_cache = reinterpret_cast<float*>(reinterpret_cast<char*>(ppart) +
                                               round_up(2 * size_t(p.P * p.G) * size_t(2 * p.K * p.dr + p.K) * 4, 256));
    float* gq_cache = reinterpret_cast<float*>(reinterpret_cast<char*>(gk_cache) + gamma_cache_bytes(p));
    if (bwdc_kb_applies(p))
        return f32_backward_causal_kb(p, XQ, XK, V, mu, pi, eps, dO, dXQ, dXK, dV, dmu, ds2, dpi, v, ppart, ppart_key,
                                      reinterpret_cast<char*>(gk_cache), st, state_in, dstate_out, dstate_in);
    float* none = nullptr;
    const float* cnone = nullptr;
    const bool tiled = bwdc_tiled_applies(p);
    const dim3 grid(unsigned(p.G), unsigned(p.P));
    const int Ei = int(E);
    const dim3 egrid(unsigned((Ei + kThreads - 1) / kThreads), unsigned(p.P));
    const int H = int(p.H), dr = int(p.dr), dv = int(p.dv), K = int(p.K), G = int(p.G);
    // segment aggregates of the forward memory (one segment: the prefix writes zeros); the tiled
    // passes also take Gamma_K from this pass, so it runs for one segment too
    if (tiled || (p.G > 1 && bwd_tiled_applies(p))) {
        GMA_LAUNCH("f32_bwdc_aggregate", (f32_bwd_tiled_kernel<BWD_WRITE, kTiledTW>), grid, dim3(1024 / kTiledTW),
                   bwd_tiled_lds_bytes(BWD_WRITE, K, dr, dv), st, XK, V, p.N, H, dr, dv, K, p.seg, G, v.c, v.inv, mu,
                   cnone, eps, none, none, states, none, cnone, cnone, none, tiled ? gk_cache : none, cnone, cnone);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (p.G > 1) {
        const size_t lds_w = size_t(kTile) * (p.dr + p.K + p.dv) * sizeof(float);
        GMA_LAUNCH("f32_bwdc_aggregate", f32_write_kernel, grid, dim3(kThreads), lds_w, st, XK, V, p.N, H, dr, dv, K,
                   p.seg, G, v.c, v.inv, mu, states);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    GMA_LAUNCH("f32_bwdc_prefix", f32_prefix_kernel, egrid, dim3(kThreads), 0, st, states, G, Ei, state_in, K, dv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (tiled) {  // register-tiled passes with the running memory in LDS
        GMA_LAUNCH("f32_bwdc_query", (f32_bwd_tiled_kernel<BWD_CQUERY, kTiledTW>), grid, dim3(1024 / kTiledTW),
                   bwd_tiled_lds_bytes(BWD_CQUERY, K, dr, dv), st, XQ, dO, p.N, H, dr, dv, K, p.seg, G, v.c, v.inv, mu,
                   static_cast<const float*>(states), eps, dXQ, none, seg_part, ppart, XK, V, rowda, gq_cache, cnone,
                   static_cast<const float*>(gk_cache));
        if ((e = hipGetLastError()) != hipSuccess) return e;
        GMA_LAUNCH("f32_bwdc_suffix", f32_suffix_kernel, egrid, dim3(kThreads), 0, st, seg_part, G, Ei, dstate_out,
                   dstate_in, K, dv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        GMA_LAUNCH("f32_bwdc_key", (f32_bwd_tiled_kernel<BWD_CKEY, kTiledTW>), grid, dim3(1024 / kTiledTW),
                   bwd_tiled_lds_bytes(BWD_CKEY, K, dr, dv), st, XK, V, p.N, H, dr, dv, K, p.seg, G, v.c, v.inv, mu,
                   static_cast<const float*>(seg_part), eps, dXK, dV, none, ppart_key, XQ, dO, rowda, none,
                   static_cast<const float*>(gk_cache), static_cast<const float*>(gq_cache));
        if ((e = hipGetLastError()) != hipSuccess) return e;
        return reduce_params(p, ppart, int(p.B), v.inv, pi, dmu, ds2, dpi, st);
    }
    // one element per thread: FAST (tables and running memory in LDS) with 64- or 32-position
    // tiles when two workgroups still fit a CU, else with the largest tile (down to 16) that fits
    // one; else the tables alone in LDS (tiles down to 4: K = 256 at d_r = 64 fits with 4);
    // otherwise the general form: 64-position tiles when two fit, else the largest tile that lets
    // two fit (down to 32), else the largest that fits
    const size_t tables = size_t(2 * K * (dr + 1) + K) * sizeof(float);
    const size_t memory = size_t(K * (dv + 1) + K) * sizeof(float);
    int T = kTile, mem_lds = 1;
    bool fast = false;
    for (int t = kTile; t >= 32 && !fast; t /= 2)
        if (bwdc_lds_bytes(t, dr, dv, K) + tables + memory <= kMaxLds / 2) fast = true, T = t;
    for (int t = kTile; t >= 16 && !fast; t /= 2)
        if (bwdc_lds_bytes(t, dr, dv, K) + tables + memory <= kMaxLds) fast = true, T = t;
    for (int t = kTile; t >= 4 && !fast; t /= 2)
        if (bwdc_lds_bytes(t, dr, dv, K) + tables <= kMaxLds) fast = true, T = t, mem_lds = 0;
    if (!fast) {
        mem_lds = 0;
        while (T > 32 && bwdc_lds_bytes(T, dr, dv, K) > kMaxLds / 2) T /= 2;
        while (T > 8 && bwdc_lds_bytes(T, dr, dv, K) > kMaxLds) T /= 2;
    }
    const size_t lds = bwdc_lds_bytes(T, dr, dv, K) + (fast ? tables + (mem_lds ? memory : 0) : 0);
    if (fast)
        GMA_LAUNCH("f32_bwdc_query", (f32_bwdc_kernel<true, true>), grid, dim3(kThreads), lds, st, XQ, XK, V, dO, p.N,
                   H, dr, dv, K, p.seg, G, T, v.c, v.inv, mu, states, eps, rowda, dXQ, none, seg_part, ppart, mem_lds);
    else
        GMA_LAUNCH("f32_bwdc_query", (f32_bwdc_kernel<true, false>), grid, dim3(kThreads), lds, st, XQ, XK, V, dO, p.N,
                   H, dr, dv, K, p.seg, G, T, v.c, v.inv, mu, states, eps, rowda, dXQ, none, seg_part, ppart, mem_lds);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GMA_LAUNCH("f32_bwdc_suffix", f32_suffix_kernel, egrid, dim3(kThreads), 0, st, seg_part, G, Ei, dstate_out, dstate_in,
               K, dv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (fast)
        GMA_LAUNCH("f32_bwdc_key", (f32_bwdc_kernel<false, true>), grid, dim3(kThreads), lds, st, XQ, XK, V, dO, p.N, H,
                   dr, dv, K, p.seg, G, T, v.c, v.inv, mu, seg_part, eps, rowda, dXK, dV, none, ppart_key, mem_lds);
    else
        GMA_LAUNCH("f32_bwdc_key", (f32_bwdc_kernel<false, false>), grid, dim3(kThreads), lds, st, XQ, XK, V, dO, p.N,
                   H, dr, dv, K, p.seg, G, T, v.c, v.inv, mu, seg_part, eps, rowda, dXK, dV, none, ppart_key, mem_lds);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return reduce_params(p, ppart, int(p.B), v.inv, pi, dmu, ds2, dpi, st);
}

// ---------------------------------------------------------------------------- bf16 staging
namespace {
__global__ void __launch_bounds__(kThreads) widen_bf16_kernel(const uint16_t* __restrict__ src,
                                                              float* __restrict__ dst, size_t n) {
    for (size_t i = size_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += size_t(gridDim.x) * kThreads)
        dst[i] = bf16_bits_to_f32(src[i]);
}
__global__ void __launch_bounds__(kThreads) narrow_bf16_kernel(const float* __restrict__ src,
                                                               uint16_t* __restrict__ dst, size_t n) {
    for (size_t i = size_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += size_t(gridDim.x) * kThreads)
        dst[i] = f32_to_bf16_bits(src[i]);
}
unsigned cast_blocks(size_t n) { return unsigned(std::min<size_t>((n + kThreads - 1) / kThreads, 8192)); }
}  // namespace

hipError_t widen_bf16(const void* src, float* dst, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    GMA_LAUNCH("widen_bf16", widen_bf16_kernel, dim3(cast_blocks(n)), dim3(kThreads), 0, st,
               static_cast<const uint16_t*>(src), dst, n);
    return hipGetLastError();
}

hipError_t narrow_to_bf16(const float* src, void* dst, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    GMA_LAUNCH("narrow_bf16", narrow_bf16_kernel, dim3(cast_blocks(n)), dim3(kThreads), 0, st, src,
               static_cast<uint16_t*>(dst), n);
    return hipGetLastError();
}

}  // namespace gma
