// Responsibility diagnostics (Sec. 5.4 of "Gaussian Mixture Attention", Eq. 24-29) of
// routing vectors X [B,H,N,d_r]: B sequences of N positions, H heads with their own mixtures.
//   1. Gamma [B,H,N,K] fp32 into the workspace by the responsibilities kernels (Eq. 3); with
//      bf16 input one fused kernel instead accumulates the head sums of Gamma in LDS (below)
//   2. token kernel, per block of 64 positions of one sequence: gbar = head mean of Gamma
//      (Eq. 24, heads in order), each position's entropy -sum_k gbar log gbar, maximum and
//      argmax (Eq. 27-29; the lowest k among equal maxima), and the block's fp64 partial sums of
//      gbar (usage, Eq. 25), of the entropies and of the maxima
//   3. column kernel: each of the K + 2 partial columns summed over the blocks in a fixed order;
//      final kernel: usage p_k = sum / T, H_usage = -sum p log p / log K (Eq. 26), H_token and
//      R_max the means over the T = B N positions
// Every sum runs in a fixed order, so results are bitwise reproducible.  0 log 0 is 0; with
// K = 1 both normalised entropies are reported as 0.
#include <cmath>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "gma_bf16_common.h"
#include "gma_bf16_phases.h"
#include "gma_device.h"
#include "gma_internal.h"

namespace gma {
namespace diag {

constexpr int kThreads = 256;
constexpr int kTokens = 64;   // positions per block of the token kernel (16 per wave)
constexpr int kMaxKPL = 4;    // components per lane (K <= 256)

// (value, index) pair reduction over the wave: the larger value, the lower index on ties.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(v, o, kWave);
        const int oi = __shfl_xor(i, o, kWave);
        if (ov > v || (ov == v && oi < i)) {
            v = ov;
            i = oi;
        }
    }
}

// Grid (blocks of kTokens positions, B).  Gamma: [B][H][N][K] fp32.  partials: per block
// (b-major), K + 2 doubles: sum of gbar per component, sum of entropies, sum of maxima.
__global__ void __launch_bounds__(kThreads)
    diag_tokens_kernel(const float* __restrict__ Gamma, int64_t N, int H, int K, int32_t* __restrict__ argmax,
                       float* __restrict__ gbar, double* __restrict__ partials) {
    __shared__ double red[kThreads / 64][kMaxKPL * 64 + 2];
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t b = blockIdx.y;
    const int64_t blk = int64_t(blockIdx.y) * gridDim.x + blockIdx.x;
    // lane l holds components l KPL .. l KPL + KPL - 1 (consecutive: one vector load per row
    // when KPL is 2 or 4 and divides K)
    const int KPL = (K + 63) / 64;
    const bool v2 = KPL == 2 && (K & 1) == 0, v4 = KPL == 4 && (K & 3) == 0;
    const float invH = 1.0f / float(H);
    double acc[kMaxKPL] = {0.0, 0.0, 0.0, 0.0};
    double ent_sum = 0.0, max_sum = 0.0;
    for (int q = 0; q < kTokens / (kThreads / 64); ++q) {
        const int64_t n = int64_t(blockIdx.x) * kTokens + w * (kTokens / (kThreads / 64)) + q;
        if (n >= N) break;  // uniform over the wave
        float g[kMaxKPL];
#pragma unroll
        for (int u = 0; u < kMaxKPL; ++u) g[u] = 0.0f;
        for (int h = 0; h < H; ++h) {  // Eq. 24, heads in order
            const float* row = Gamma + ((size_t(b) * H + h) * N + n) * K + l * KPL;
            if (v4) {
                if (l * 4 < K) {
                    const float4 x = *reinterpret_cast<const float4*>(row);
                    g[0] += x.x; g[1] += x.y; g[2] += x.z; g[3] += x.w;
                }
            } else if (v2) {
                if (l * 2 < K) {
                    const float2 x = *reinterpret_cast<const float2*>(row);
                    g[0] += x.x; g[1] += x.y;
                }
            } else {
#pragma unroll
                for (int u = 0; u < kMaxKPL; ++u)
                    if (u < KPL && l * KPL + u < K) g[u] += row[u];
            }
        }
        float ent = 0.0f, best = -1.0f;
        int bi = 0;
#pragma unroll
        for (int u = 0; u < kMaxKPL; ++u) {
            if (u < KPL && l * KPL + u < K) {
                const float v = g[u] * invH;
                g[u] = v;
                // natural log; values below the smallest normal float (where the hardware log
                // flushes to -inf) contribute less than 1e-35 and are skipped
                if (v >= 1.17549435e-38f) ent -= v * (__builtin_amdgcn_logf(v) * 0.69314718055994530942f);
                if (v > best) {  // k ascending within the lane: equal values keep the lower k
                    best = v;
                    bi = l * KPL + u;
                }
                acc[u] += double(v);
                if (gbar) gbar[(size_t(b) * N + n) * K + l * KPL + u] = v;
            }
        }
        for (int o = 32; o >= 1; o >>= 1) ent += __shfl_xor(ent, o, kWave);
        wave_argmax(best, bi);
        if (l == 0) {
            if (argmax) argmax[size_t(b) * N + n] = bi;
            ent_sum += double(ent);
            max_sum += double(best);
        }
    }
    // the block's partial sums: waves combined in wave order
#pragma unroll
    for (int u = 0; u < kMaxKPL; ++u) red[w][l * kMaxKPL + u] = acc[u];
    if (l == 0) {
        red[w][kMaxKPL * 64] = ent_sum;
        red[w][kMaxKPL * 64 + 1] = max_sum;
    }
    __syncthreads();
    double* out = partials + size_t(blk) * (K + 2);
    for (int k = threadIdx.x; k < K + 2; k += kThreads) {
        const int src = k < K ? (k / KPL) * kMaxKPL + k % KPL : kMaxKPL * 64 + (k - K);
        double s = 0.0;
        for (int ww = 0; ww < kThreads / 64; ++ww) s += red[ww][src];
        out[k] = s;
    }
}

// Grid (K + 2): column c of the block partials summed over the nblk blocks, each thread a
// fixed strided subset in order, then a fixed-shape tree over the threads.
__global__ void __launch_bounds__(kThreads)
    diag_columns_kernel(const double* __restrict__ partials, int64_t nblk, int K, double* __restrict__ cols) {
    __shared__ double red[kThreads];
    const int c = blockIdx.x, t = threadIdx.x;
    double s = 0.0;
    for (int64_t i = t; i < nblk; i += kThreads) s += partials[size_t(i) * (K + 2) + c];
    red[t] = s;
    __syncthreads();
    for (int o = kThreads / 2; o >= 1; o >>= 1) {
        if (t < o) red[t] += red[t + o];
        __syncthreads();
    }
    if (t == 0) cols[c] = red[0];
}

// One block: usage [K], stats [3] = H_usage, H_token, R_max from the K + 2 column sums
// (T = 0 gives zeros).
__global__ void __launch_bounds__(kThreads)
    diag_final_kernel(const double* __restrict__ cols, int K, int64_t T, float* __restrict__ usage,
                      float* __restrict__ stats) {
    __shared__ double red[kThreads / 64];
    const int t = threadIdx.x, l = t & 63, w = t >> 6;
    double plogp = 0.0;
    for (int k = t; k < K; k += kThreads) {
        const double p = T > 0 ? cols[k] / double(T) : 0.0;
        usage[k] = float(p);
        if (p > 0.0) plogp += p * log(p);
    }
    for (int o = 32; o >= 1; o >>= 1) plogp += __shfl_xor(plogp, o, kWave);
    if (l == 0) red[w] = plogp;
    __syncthreads();
    if (t == 0) {
        double pl = 0.0;
        for (int ww = 0; ww < kThreads / 64; ++ww) pl += red[ww];
        const double es = T > 0 ? cols[K] : 0.0, ms = T > 0 ? cols[K + 1] : 0.0;
        const double logk = log(double(K));
        stats[0] = (K > 1) ? float(-pl / logk) : 0.0f;
        stats[1] = (K > 1 && T > 0) ? float(es / double(T) / logk) : 0.0f;
        stats[2] = T > 0 ? float(ms / double(T)) : 0.0f;
    }
}

// ---- bf16 input: one fused kernel, Gamma never leaves the chip --------------------------
// Per-head operand planes, built once per call into the workspace (the PlaneBuilder layout).
template <int DR, int KT>
__global__ void __launch_bounds__((bf::Split<DR, KT>::NW * 64)) plane_table_kernel(bf::Mixture mx, char* __restrict__ table) {
    using PB = bf::PlaneBuilder<DR, KT * 32, bf::Split<DR, KT>::NW * 64>;
    PB pb;
    pb.load(mx, blockIdx.x);
    pb.build(table + size_t(blockIdx.x) * PB::LDS_BYTES, mx.K);
}

// Tokens per workgroup: rounds of the score tile until the fp32 tile of head sums is 64 KiB.
template <int DR, int KT>
constexpr int fused_tokens() {
    constexpr int round = bf::Split<DR, KT>::ROUND, per = 65536 / (KT * 32 * 4);
    return per >= round ? (per / round) * round : round;
}

// Grid (token tiles, B).  For each head in order: the head's planes from the table, then the
// responsibilities of the tile's tokens (split-operand MFMA scores and softmax, as in the
// responsibilities kernel) added, times 1/H, into the tile's sums in LDS (each (token,
// component) owned by one lane for every head).  Then, per token, the statistics of the
// token kernel above, and the workgroup's partial sums.
template <int DR, int KT>
__global__ void __launch_bounds__((bf::Split<DR, KT>::NW * 64))
    diag_fused_kernel(const uint16_t* __restrict__ X, int64_t N, int H, int K, const char* __restrict__ table,
                      int32_t* __restrict__ argmax, float* __restrict__ gbar, double* __restrict__ partials) {
    using S = bf::Split<DR, KT>;
    constexpr int NT = S::NW * 64, Kp = KT * 32, TT = fused_tokens<DR, KT>(), NW = S::NW;
    constexpr int LDT = Kp + 4;  // row pitch of the tile of sums: rows of one subtile fall in different banks
    constexpr size_t TBL = bf::PlaneBuilder<DR, Kp, NT>::LDS_BYTES;
    __shared__ __attribute__((aligned(16))) float gs[TT * LDT];
    __shared__ bf::Stats st[S::TS * S::CS * 32];
    __shared__ double red[NW][kMaxKPL * 64 + 2];
    const int wave = bf::wave_id(), l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const int cs = wave % S::CS, ts = wave / S::CS;
    const int64_t b = blockIdx.y, t0 = int64_t(blockIdx.x) * TT;
    const float invH = 1.0f / float(H);
    for (int i = threadIdx.x; i < TT * LDT / 4; i += NT) reinterpret_cast<float4*>(gs)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();  // zeroed by every thread, accumulated by each entry's owner lane
    bf::WaveParams<DR, S::CTW> P;
    // rounds it = (head h, round r) in order
    const int RR = TT / S::ROUND;
    int64_t rr_valid = (N - t0 + S::ROUND - 1) / S::ROUND;  // rounds of this tile that hold tokens
    const int RV = int(rr_valid < RR ? rr_valid : RR);
    auto fetch = [&](int it, bf::bf16x8 (&xs)[DR / 16]) {
        const int h = it / RV, r = it - h * RV;
        const int64_t n0 = t0 + r * S::ROUND + ts * 32;
        const int valid = it < H * RV ? int(max<int64_t>(0, min<int64_t>(32, N - n0))) : 0;
        bf::load_x<DR>(X + (size_t(b) * H + (h < H ? h : 0)) * N * DR, n0, valid, xs);
    };
    // software pipeline: round it + 1's score MFMAs are issued before round it's softmax, and
    // x fragments are fetched two rounds ahead of their scores
    const int total = H * RV;
    bf::bf16x8 xa[DR / 16], xb[DR / 16];
    fetch(0, xa);
    fetch(1, xb);
    P.template read_planes<Kp>(table, cs * S::CTW);
    bf::f32x16 cur[S::CTW], nxt[S::CTW];
    bf::scores_x<DR, S::CTW>(P, xa, cur);
    fetch(2, xa);
    for (int it = 0; it < total; ++it) {  // Eq. 24, heads in order
        const int r = it % RV;
        if (it + 1 < total) {
            if ((it + 1) % RV == 0) P.template read_planes<Kp>(table + size_t((it + 1) / RV) * TBL, cs * S::CTW);
            bf::scores_x<DR, S::CTW>(P, xb, nxt);
#pragma unroll
            for (int ks = 0; ks < DR / 16; ++ks) xb[ks] = xa[ks];
            fetch(it + 3, xa);
        }
        const int tl = r * S::ROUND + ts * 32;  // first token of this wave's subtile in the tile
        const int valid = int(max<int64_t>(0, min<int64_t>(32, N - (t0 + tl))));
        float m, L, D, zr[S::CTW][16];
        bf::local_softmax<S::CTW, false>(cur, zr, m, L, D);
        if (S::CS > 1) {
            __syncthreads();  // the previous round's statistics are read
            if (lh == 0) st[(ts * S::CS + cs) * 32 + j] = bf::Stats{m, L, 0.0f};
            __syncthreads();
        }
        float dl;
        const float scale = bf::combine_stats<S::CS>(st, ts, cs, j, m, L, 0.0f, dl) * invH;
        if (j < valid) {
            float* row = gs + (tl + j) * LDT;
#pragma unroll
            for (int ct = 0; ct < S::CTW; ++ct)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float4* g4 = reinterpret_cast<float4*>(row + (cs * S::CTW + ct) * 32 + 8 * q + 4 * lh);
                    float4 v = *g4;
                    v.x += cur[ct][4 * q] * scale;
                    v.y += cur[ct][4 * q + 1] * scale;
                    v.z += cur[ct][4 * q + 2] * scale;
                    v.w += cur[ct][4 * q + 3] * scale;
                    *g4 = v;
                }
        }
#pragma unroll
        for (int ct = 0; ct < S::CTW; ++ct) cur[ct] = nxt[ct];
    }
    __syncthreads();
    // per-token statistics (Eq. 27-29) and partial sums, as in diag_tokens_kernel
    const int KPL = (K + 63) / 64;
    double accu[kMaxKPL] = {0.0, 0.0, 0.0, 0.0};
    double ent_sum = 0.0, max_sum = 0.0;
    for (int tt = wave; tt < TT; tt += NW) {
        const int64_t n = t0 + tt;
        if (n >= N) break;
        float ent = 0.0f, best = -1.0f;
        int bi = 0;
#pragma unroll
        for (int u = 0; u < kMaxKPL; ++u) {
            const int k = l * KPL + u;
            if (u < KPL && k < K) {
                const float v = gs[tt * LDT + k];
                if (v >= 1.17549435e-38f) ent -= v * (__builtin_amdgcn_logf(v) * 0.69314718055994530942f);
                if (v > best) {
                    best = v;
                    bi = k;
                }
                accu[u] += double(v);
                if (gbar) gbar[(size_t(b) * N + n) * K + k] = v;
            }
        }
        for (int o = 32; o >= 1; o >>= 1) ent += __shfl_xor(ent, o, kWave);
        wave_argmax(best, bi);
        if (l == 0) {
            if (argmax) argmax[size_t(b) * N + n] = bi;
            ent_sum += double(ent);
            max_sum += double(best);
        }
    }
#pragma unroll
    for (int u = 0; u < kMaxKPL; ++u) red[wave][l * kMaxKPL + u] = accu[u];
    if (l == 0) {
        red[wave][kMaxKPL * 64] = ent_sum;
        red[wave][kMaxKPL * 64 + 1] = max_sum;
    }
    __syncthreads();
    double* out = partials + (size_t(blockIdx.y) * gridDim.x + blockIdx.x) * (K + 2);
    for (int k = threadIdx.x; k < K + 2; k += NT) {
        const int src = k < K ? (k / KPL) * kMaxKPL + k % KPL : kMaxKPL * 64 + (k - K);
        double s = 0.0;
        for (int ww = 0; ww < NW; ++ww) s += red[ww][src];
        out[k] = s;
    }
}

template <typename F>
hipError_t with_dr_kt(int dr, int kt, F&& f) {
#define GMA_DIAG_CASE(D, T) \
    if (dr == D && kt == T) return f(std::integral_constant<int, D>(), std::integral_constant<int, T>());
#define GMA_DIAG_DR(D) GMA_DIAG_CASE(D, 1) GMA_DIAG_CASE(D, 2) GMA_DIAG_CASE(D, 4) GMA_DIAG_CASE(D, 8)
    GMA_DIAG_DR(16) GMA_DIAG_DR(32) GMA_DIAG_DR(64) GMA_DIAG_DR(128)
#undef GMA_DIAG_DR
#undef GMA_DIAG_CASE
    return hipErrorNotSupported;
}

// The fused path applies where one head's plane table fits a workgroup's reads comfortably and
// the tile of sums fits LDS next to the kernel's other arrays.
template <int DR, int KT>
constexpr bool fused_ok() {
    return bf::PlaneBuilder<DR, KT * 32, bf::Split<DR, KT>::NW * 64>::LDS_BYTES <= 160 * 1024;
}

}  // namespace diag

namespace {

// bf16 input with a fused variant: (tokens per workgroup, plane table bytes per head); (0, 0) if none
std::pair<int64_t, size_t> fused_geometry(const Plan& p) {
    std::pair<int64_t, size_t> g{0, 0};
    if (p.io != GMA_BF16) return g;
    (void)diag::with_dr_kt(int(p.dr), int(p.Kp / 32), [&](auto D, auto T) {
        constexpr int DR = decltype(D)::value, KT = decltype(T)::value;
        if constexpr (diag::fused_ok<DR, KT>())
            g = {diag::fused_tokens<DR, KT>(),
                 bf::PlaneBuilder<DR, KT * 32, bf::Split<DR, KT>::NW * 64>::LDS_BYTES};
        return hipSuccess;
    });
    return g;
}

}  // namespace

size_t diag_gamma_bytes(const Plan& p) {
    const auto fg = fused_geometry(p);
    if (fg.first > 0) return round_up(size_t(p.H) * fg.second, 256);  // the per-head plane table
    return round_up(size_t(p.P) * size_t(p.N) * size_t(p.K) * 4, 256);  // every head's Gamma
}
int64_t diag_blocks(const Plan& p) {
    const auto fg = fused_geometry(p);
    const int64_t tt = fg.first > 0 ? fg.first : diag::kTokens;
    return p.B * ((p.N + tt - 1) / tt);
}
size_t diag_partials_bytes(const Plan& p) {  // block partials, then the K + 2 column sums
    return round_up(size_t(diag_blocks(p)) * size_t(p.K + 2) * 8, 256) + round_up(size_t(p.K + 2) * 8, 256);
}

hipError_t diagnostics(const Plan& p, const Plan& resp, const void* X, const float* mu, const float* s2,
                       const float* pi, float* usage, float* stats, int32_t* argmax, float* gbar, char* ws,
                       hipStream_t st) {
    float* gamma = reinterpret_cast<float*>(ws);
    double* partials = reinterpret_cast<double*>(ws + diag_gamma_bytes(p));
    double* cols = reinterpret_cast<double*>(ws + diag_gamma_bytes(p) +
                                             round_up(size_t(diag_blocks(p)) * size_t(p.K + 2) * 8, 256));
    char* rws = ws + diag_gamma_bytes(p) + diag_partials_bytes(p);
    const int64_t nblk = (p.P > 0 && p.N > 0) ? diag_blocks(p) : 0;
    const auto fg = fused_geometry(p);
    if (nblk > 0 && fg.first > 0) {
        const bf::Mixture mx{mu, s2, pi, int(p.K)};
        hipError_t e = diag::with_dr_kt(int(p.dr), int(p.Kp / 32), [&](auto D, auto T) {
            constexpr int DR = decltype(D)::value, KT = decltype(T)::value;
            if constexpr (diag::fused_ok<DR, KT>()) {
                constexpr int NT = bf::Split<DR, KT>::NW * 64;
                GMA_LAUNCH("diag_planes", (diag::plane_table_kernel<DR, KT>), dim3(unsigned(p.H)), dim3(NT), 0, st, mx,
                           ws);
                hipError_t e2 = hipGetLastError();
                if (e2 != hipSuccess) return e2;
                GMA_LAUNCH("bf16_diag", (diag::diag_fused_kernel<DR, KT>),
                           dim3(unsigned((p.N + fg.first - 1) / fg.first), unsigned(p.B)), dim3(NT), 0, st,
                           static_cast<const uint16_t*>(X), p.N, int(p.H), int(p.K), ws, argmax, gbar, partials);
            }
            return hipGetLastError();
        });
        if (e != hipSuccess) return e;
        GMA_LAUNCH("diag_columns", diag::diag_columns_kernel, dim3(unsigned(p.K + 2)), dim3(diag::kThreads), 0, st,
                   partials, nblk, int(p.K), cols);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (nblk > 0) {
        hipError_t e = p.io == GMA_F32
                           ? f32_responsibilities(resp, static_cast<const float*>(X), mu, s2, pi, gamma, GMA_F32, rws, st)
                           : bf16_responsibilities(resp, X, mu, s2, pi, gamma, GMA_F32, rws, st);
        if (e != hipSuccess) return e;
        GMA_LAUNCH("diag_tokens", diag::diag_tokens_kernel,
                   dim3(unsigned((p.N + diag::kTokens - 1) / diag::kTokens), unsigned(p.B)), dim3(diag::kThreads), 0,
                   st, gamma, p.N, int(p.H), int(p.K), argmax, gbar, partials);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        GMA_LAUNCH("diag_columns", diag::diag_columns_kernel, dim3(unsigned(p.K + 2)), dim3(diag::kThreads), 0, st,
                   partials, nblk, int(p.K), cols);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    GMA_LAUNCH("diag_final", diag::diag_final_kernel, dim3(1), dim3(diag::kThreads), 0, st, cols, int(p.K),
               nblk > 0 ? p.B * p.N : int64_t(0), usage, stats);
    return hipGetLastError();
}

}  // namespace gma
