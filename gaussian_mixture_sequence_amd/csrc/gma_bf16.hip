// bf16 I/O path of the GMA forward: MFMA kernels for gfx950.
//
// Kernel sequence on the caller's stream:
//   write     per (problem, split): partial [Vt | Z] = Gamma_K^T [V | 1] over the split
//             (Sec. 3.3 Eq. 5-6 of "Gaussian Mixture Attention"); Gamma_K never leaves
//             the chip: scores -> softmax in registers -> bf16 tile in LDS -> MFMA
//   combine   bidirectional: fixed-order sum of the partials, then Vt split into hi + lo
//             bf16 planes stored transposed (the A operand of the read) and Z in fp32
//   read      O = Gamma_Q Vt / (Gamma_Q Z + eps) (Eq. 7-8): computed as O^T = Vt^T Gamma_Q^T
//             with hi + lo Vt, the denominator in fp32 on the VALU during the softmax
//   aggregate causal: the write kernel over segments 0 .. G-2 (segment aggregates)
//   scan      causal chunked scan (gma_bf16_scan.hip); segment s starts from the sum of
//             the aggregates of segments 0 .. s-1
// Every kernel builds the score operands of its own component tiles from mu, sigma2 and
// pi in registers (WaveParams::compute), so no launch is spent on the parameters.
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "gma_bf16_common.h"
#include "gma_internal.h"

namespace gma {
namespace bf {

// ---------------------------------------------------------------------------- softmax across waves

// Per-round softmax statistics shared by the CS waves of one token subtile.
struct Stats {
    float m, L, D;
};

// Combines this wave's (m, L, D) with those of the other component groups of its
// token subtile (published in `st` before the barrier).  Returns the factor that turns
// this wave's exp2(s - m_w) into probabilities, and the full D / L.
template <int CS>
__device__ __forceinline__ float combine_stats(const Stats* st, int ts, int cs, int j, float m, float L, float D,
                                               float& DoverL) {
    if (CS == 1) {
        const float r = __builtin_amdgcn_rcpf(L);
        DoverL = D * r;
        return r;
    }
    float mm = -INFINITY;
#pragma unroll
    for (int c = 0; c < CS; ++c) mm = fmaxf(mm, st[(ts * CS + c) * 32 + j].m);
    float Lt = 0.0f, Dt = 0.0f;
#pragma unroll
    for (int c = 0; c < CS; ++c) {
        const Stats s = st[(ts * CS + c) * 32 + j];
        const float f = __builtin_amdgcn_exp2f(s.m - mm);
        Lt = fmaf(s.L, f, Lt);
        Dt = fmaf(s.D, f, Dt);
    }
    (void)cs;
    const float r = __builtin_amdgcn_rcpf(Lt);
    DoverL = Dt * r;
    return __builtin_amdgcn_exp2f(m - mm) * r;
}

// ---------------------------------------------------------------------------- responsibilities

template <int DR, int KT>
__global__ void __launch_bounds__((Split<DR, KT>::NW * 64)) resp_kernel(const uint16_t* __restrict__ X, int64_t N,
                                                                       int H, Mixture mx, void* Gamma,
                                                                       int gamma_bf16) {
    using S = Split<DR, KT>;
    __shared__ Stats st[S::TS * S::CS * 32];
    const int wave = wave_id(), l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const int cs = wave % S::CS, ts = wave / S::CS;
    const int64_t p = blockIdx.y;
    const int h = int(p % H), K = mx.K;
    WaveParams<DR, S::CTW> P;
    P.compute(mx, h, cs * S::CTW);
    const uint16_t* Xp = X + size_t(p) * N * DR;
    const int64_t n0 = int64_t(blockIdx.x) * S::ROUND + ts * 32;
    const int valid = int(max<int64_t>(0, min<int64_t>(32, N - n0)));
    f32x16 acc[S::CTW];
    scores<DR, S::CTW>(P, Xp, n0, valid, acc);
    float m, L, D;
    float zr[S::CTW][16];
    local_softmax<S::CTW, false>(acc, zr, m, L, D);
    if (S::CS > 1) {
        if (lh == 0) st[(ts * S::CS + cs) * 32 + j] = Stats{m, L, 0.0f};
        __syncthreads();
    }
    float dl;
    const float scale = combine_stats<S::CS>(st, ts, cs, j, m, L, 0.0f, dl);
    if (j >= valid) return;
    const size_t rowoff = (size_t(p) * N + n0 + j) * K;
#pragma unroll
    for (int ct = 0; ct < S::CTW; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int comp = (cs * S::CTW + ct) * 32 + 8 * q + 4 * lh;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (comp + e < K) {
                    const float g = acc[ct][4 * q + e] * scale;
                    if (gamma_bf16)
                        static_cast<uint16_t*>(Gamma)[rowoff + comp + e] = f32_to_bf16_bits(g);
                    else
                        static_cast<float*>(Gamma)[rowoff + comp + e] = g;
                }
            }
        }
}

// ---------------------------------------------------------------------------- write (Gamma_K^T [V | 1])

// Rows [lo, hi) of one problem, in rounds of ROUND tokens, software-pipelined so that
// every wave keeps the matrix cores and the vector ALU busy at the same time.
// Iteration r, region A (one basic block, MFMA and VALU interleaved):
//   MFMAs of round r+1's scores (x tile r+1, in LDS) and of round r-1's accumulation
//   Vt^T += V^T Gamma_K, Z += Gamma_K^T 1 (Gamma_K and V tiles r-1, in LDS);
//   VALU: softmax statistics of round r (scores issued in iteration r-1) and, with a
//   double-buffered x tile, the split of x tile r+2 into its free buffer  -> B1
// Region B: Gamma_K of round r (bf16) and V tile r into LDS (single x buffer: x tile r+2
//   too); loads of V r+1 and x r+3 issued  -> B2
// Every LDS overwrite follows a barrier that all reads of the old contents precede (a
// wave's LDS reads complete before the MFMAs that use them issue).  Gamma_K and V start
// zeroed, so round -1's accumulation adds nothing; round R's scores (x past the end
// reads zero) are computed and discarded.  No branch splits region A.
constexpr int gcd_i(int a, int b) { return b == 0 ? a : gcd_i(b, a % b); }

template <int DR, int KT, int VT>
__global__ void __launch_bounds__((Split<DR, KT>::NW * 64)) write_kernel(const uint16_t* __restrict__ XK,
                                                                        const uint16_t* __restrict__ V, int64_t N,
                                                                        int H, int64_t seg, int G,
                                                                        Mixture mx, float* __restrict__ partials) {
    using S = Split<DR, KT>;
    constexpr int NW = S::NW, NT = NW * 64;
    constexpr int Kp = KT * 32, DV = VT * 32;
    constexpr int LDG = Kp + 8, LDV = DV + 8;
    using XT = XTile<DR, S::ROUND, NT>;
    constexpr int VCHUNKS = S::ROUND * DV / 8;
    constexpr int VCH = (VCHUNKS + NT - 1) / NT;
    constexpr bool VEVEN = VCHUNKS % NT == 0;
    // accumulation work, identical for every wave: V units are (component tile, value
    // tile) pairs, split along the round's k-steps when there are fewer pairs than waves;
    // Z units are component tiles times an all-ones operand, split the same way
    constexpr int KSR = S::ROUND / 16;
    constexpr int VPAIRS = KT * VT;
    constexpr int VSPLIT = NW / gcd_i(VPAIRS, NW), VU = VPAIRS * VSPLIT / NW, VKS = KSR / VSPLIT;
    constexpr int ZSPLIT = NW / gcd_i(KT, NW), ZU = KT * ZSPLIT / NW, ZKS = KSR / ZSPLIT;
    static_assert(KSR % VSPLIT == 0 && KSR % ZSPLIT == 0, "round too short for the accumulation split");
    constexpr int MF_A = 5 * S::CTW * S::KS + VU * VKS + ZU * ZKS;  // MFMAs of region A
    constexpr int BASE_LDS = S::TS * S::CS * 32 * 12 + S::ROUND * (LDG + LDV) * 2;
    constexpr int XB = (BASE_LDS + 2 * XT::LDS_BYTES <= 80 * 1024) ? 2 : 1;  // keep two workgroups per CU
    __shared__ Stats st[S::TS * S::CS * 32];
    __shared__ __attribute__((aligned(16))) u32x4 Xt[XB][XT::LDS_BYTES / 16];
    __shared__ __attribute__((aligned(16))) uint16_t Gs[S::ROUND * LDG];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[S::ROUND * LDV];
    __shared__ float Zred[KT * ZSPLIT * 32];

    const int wave = wave_id(), l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const int cs = wave % S::CS, ts = wave / S::CS;
    const int64_t p = blockIdx.y;
    const int g_idx = blockIdx.x;
    const int h = int(p % H);
    const int64_t lo = int64_t(g_idx) * seg, hi = min<int64_t>(lo + seg, N);
    const int64_t rows = hi - lo;
    const int64_t R = (rows + S::ROUND - 1) / S::ROUND;  // rounds of this split
    // mixture parameters staged through the x tile buffer when it is large enough
    using MS = MixtureStage<DR, Kp, NT>;
    constexpr bool STAGE = sizeof(Xt) >= MS::LDS_BYTES;
    WaveParams<DR, S::CTW> P;
    typename WaveParams<DR, S::CTW>::Raw praw;
    MS mstage;
    if constexpr (STAGE) {
        mstage.load(mx, h);
        P.fetch_pi(mx, h, cs * S::CTW, praw);
    } else {
        P.fetch(mx, h, cs * S::CTW, praw);
    }
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(XK + (size_t(p) * N + lo) * DR, rows * DR * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + (size_t(p) * N + lo) * DV, rows * DV * 2);

    XT xt;
    u32x4 vr[VCH];
    auto load_v = [&](int64_t row0) {
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = threadIdx.x + u * NT;
            vr[u] = (VEVEN || c < VCHUNKS) ? buf_load16(rv, uint32_t((row0 * DV + int64_t(c) * 8) * 2))
                                           : u32x4{0u, 0u, 0u, 0u};
        }
    };
    f32x16 vacc[VU], zacc[ZU];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int i = 0; i < VU; ++i) vacc[i][r] = 0.0f;
#pragma unroll
        for (int i = 0; i < ZU; ++i) zacc[i][r] = 0.0f;
    }
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    float zr[S::CTW][16];
    f32x16 acc_a_init[S::CTW];  // round 0's scores when the x tile is single-buffered
    auto accumulate = [&]() __attribute__((always_inline)) {  // Vt^T += V^T Gamma_K, Z += Gamma_K^T 1
#pragma unroll
        for (int i = 0; i < VU; ++i) {
            const int q = wave + i * NW, pair = q / VSPLIT, part = q - pair * VSPLIT;
            const int ct = pair / VT, vt = pair - ct * VT;
#pragma unroll
            for (int kk = 0; kk < VKS; ++kk) {
                const int ks = part * VKS + kk;
                vacc[i] = mfma(read_colfrag(Gs, LDG, 16 * ks, ct * 32), read_colfrag(Vs, LDV, 16 * ks, vt * 32), vacc[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < ZU; ++i) {
            const int q = wave + i * NW, ct = q / ZSPLIT, part = q - ct * ZSPLIT;
#pragma unroll
            for (int kk = 0; kk < ZKS; ++kk)
                zacc[i] = mfma(read_colfrag(Gs, LDG, 16 * (part * ZKS + kk), ct * 32), ones, zacc[i]);
        }
    };

    // prologue: Gamma_K and V tiles zeroed; x tiles 0 and 1 fetched together (one memory
    // round trip), 0 (and 1) split into LDS; scores of round 0 issued; V 0 and x tile 2
    // in flight
    {
        XT xt1;
        xt.load(rx, 0);
        xt1.load(rx, S::ROUND);
        load_v(0);
        for (int c = threadIdx.x; c < S::ROUND * LDG / 8; c += NT) reinterpret_cast<u32x4*>(Gs)[c] = u32x4{0u, 0u, 0u, 0u};
        for (int c = threadIdx.x; c < S::ROUND * LDV / 8; c += NT) reinterpret_cast<u32x4*>(Vs)[c] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (STAGE) {  // while the tiles are in flight
            mstage.commit(reinterpret_cast<float*>(&Xt[0][0]));
            __syncthreads();
            P.template read_staged<Kp>(reinterpret_cast<const float*>(&Xt[0][0]), cs * S::CTW, praw);
            P.build(praw, mx.K, cs * S::CTW);
            __syncthreads();  // staging area free for the x tiles
        } else {
            P.build(praw, mx.K, cs * S::CTW);
        }
        xt.commit(Xt[0]);
        xt.load(rx, 2 * S::ROUND);
        if (XB == 2) xt1.commit(Xt[XB - 1]);
        __syncthreads();
        if (XB == 1) {
            scores_lds<DR, S::CTW>(P, Xt[0], ts, acc_a_init);
            __syncthreads();  // x tile 0 consumed by every wave
            xt1.commit(Xt[0]);
            __syncthreads();
        }
    }
    f32x16 acc_a[S::CTW], acc_b[S::CTW];
    if (XB == 2) scores_lds<DR, S::CTW>(P, Xt[0], ts, acc_a);
    else
#pragma unroll
        for (int ct = 0; ct < S::CTW; ++ct) acc_a[ct] = acc_a_init[ct];

    // one pipelined iteration; `cur` holds round r's scores, `nxt` receives round r+1's
    auto iteration = [&](const int64_t r, f32x16 (&cur)[S::CTW], f32x16 (&nxt)[S::CTW]) __attribute__((always_inline)) {
        const int64_t r0 = r * S::ROUND;
        const int xb1 = int((r + 1) % XB);
        // ---- region A (the accumulation first: its transposing LDS reads bound the
        // scheduling region, so everything after them can be interleaved)
        accumulate();
        scores_lds<DR, S::CTW>(P, Xt[xb1], ts, nxt);
        if (XB == 2) {
            xt.commit(Xt[xb1 ^ 1]);  // x tile r+2 into the buffer x tile r left
            xt.load(rx, r0 + 3 * S::ROUND);
        }
        float m, L, D;
        local_softmax<S::CTW, false>(cur, zr, m, L, D);
        if (S::CS > 1) st[(ts * S::CS + cs) * 32 + j] = Stats{m, L, 0.0f};  // both lane halves hold the same
#pragma unroll
        for (int i = 0; i < MF_A; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // then up to five VALU
        }
        __syncthreads();  // B1: statistics published; x tile r+1 and tiles r-1 consumed
        // ---- region B
        const int valid = int(max<int64_t>(0, min<int64_t>(32, rows - r0 - ts * 32)));
        float dl;
        float scale = combine_stats<S::CS>(st, ts, cs, j, m, L, 0.0f, dl);
        if (j >= valid) scale = 0.0f;
        store_gamma_lds<S::CTW>(cur, scale, Gs, LDG, ts * 32 + j, cs * S::CTW);
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = threadIdx.x + u * NT;
            if (VEVEN || c < VCHUNKS) {
                const int row = c / (DV / 8), col = (c - row * (DV / 8)) * 8;
                *reinterpret_cast<u32x4*>(Vs + row * LDV + col) = vr[u];
            }
        }
        load_v(r0 + S::ROUND);
        if (XB == 1) {
            xt.commit(Xt[0]);
            xt.load(rx, r0 + 3 * S::ROUND);
        }
        __syncthreads();  // B2: Gamma_K r, V r and x tile r+2 are in LDS
    };
    // rounds in pairs (static accumulator roles, no register copies on the back-edge); a
    // round past the end only exists for an odd count and is skipped
    for (int64_t r = 0; r < R; r += 2) {
        iteration(r, acc_a, acc_b);
        if (r + 1 < R) iteration(r + 1, acc_b, acc_a);
    }
    accumulate();  // the last round

    // ---- partial of this split: VtT [DV][Kp] (Vt transposed) then Z [Kp].  Parts of a
    // split unit are summed through LDS in increasing part order (the x tile area is free).
    float* mem = partials + (size_t(p) * G + g_idx) * size_t(Kp) * (DV + 1);
    float* red = reinterpret_cast<float*>(&Xt[0][0]);
    static_assert(VSPLIT == 1 || VPAIRS * 1024 * 4 <= XB * XT::LDS_BYTES, "x tile area too small for the reduction");
    __syncthreads();  // every wave is done with the x tiles
#pragma unroll
    for (int i = 0; i < VU; ++i) {
        const int q = wave + i * NW, pair = q / VSPLIT, part = q - pair * VSPLIT;
        const int ct = pair / VT, vt = pair - ct * VT;
#pragma unroll
        for (int pp = 0; pp < VSPLIT; ++pp) {
            if (VSPLIT > 1) {
                if (part == pp && pp > 0)
#pragma unroll
                    for (int r = 0; r < 16; ++r) vacc[i][r] += red[pair * 1024 + r * 64 + l];
                if (part == pp && pp < VSPLIT - 1)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[pair * 1024 + r * 64 + l] = vacc[i][r];
                __syncthreads();
            }
        }
        if (part == VSPLIT - 1) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int comp = ct * 32 + 8 * qq + 4 * lh;
                *reinterpret_cast<float4*>(mem + size_t(vt * 32 + j) * Kp + comp) =
                    make_float4(vacc[i][4 * qq + 0], vacc[i][4 * qq + 1], vacc[i][4 * qq + 2], vacc[i][4 * qq + 3]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < ZU; ++i) {
        const int q = wave + i * NW, ct = q / ZSPLIT, part = q - ct * ZSPLIT;
        if (j == 0)  // every column of the ones-operand tile holds the same sums
#pragma unroll
            for (int r = 0; r < 16; ++r) Zred[(ct * ZSPLIT + part) * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)] = zacc[i][r];
    }
    __syncthreads();
    for (int k = threadIdx.x; k < Kp; k += NT) {
        const int ct = k >> 5, i = k & 31;
        float z = 0.0f;
#pragma unroll
        for (int pp = 0; pp < ZSPLIT; ++pp) z += Zred[(ct * ZSPLIT + pp) * 32 + i];
        mem[size_t(Kp) * DV + k] = z;
    }
}

// ---------------------------------------------------------------------------- combine / prefix

// Bidirectional: memory = sum_g partial_g (increasing g), then the read operands:
// VtT_hi, VtT_lo [DV][Kp] bf16 (Vt transposed, hi + lo split) and Z [Kp] fp32.  The
// partials use the same [DV][Kp] + [Kp] order, so every access is coalesced.
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ partials, int G, int Kp, int DV,
                                                      uint16_t* __restrict__ memory) {
    // four consecutive elements per thread (Kp * DV is a multiple of 4, so a group never
    // straddles the VtT / Z boundary); the G loads are independent and issued together
    const int64_t p = blockIdx.y;
    const int E = Kp * (DV + 1);
    const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= E) return;
    const float* src = partials + size_t(p) * G * E + e;
    float4 acc = *reinterpret_cast<const float4*>(src);
#pragma unroll 8
    for (int g = 1; g < G; ++g) {
        const float4 v = *reinterpret_cast<const float4*>(src + size_t(g) * E);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    uint16_t* base = memory + size_t(p) * E * 2;  // E floats of room per problem
    if (e < Kp * DV) {
        const uint32_t h01 = pack_bf16x2(acc.x, acc.y), h23 = pack_bf16x2(acc.z, acc.w);
        const uint32_t l01 = pack_bf16x2(acc.x - __uint_as_float(h01 << 16), acc.y - __uint_as_float(h01 & 0xffff0000u));
        const uint32_t l23 = pack_bf16x2(acc.z - __uint_as_float(h23 << 16), acc.w - __uint_as_float(h23 & 0xffff0000u));
        *reinterpret_cast<u32x2*>(base + e) = u32x2{h01, h23};
        *reinterpret_cast<u32x2*>(base + size_t(DV) * Kp + e) = u32x2{l01, l23};
    } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(base + size_t(2) * DV * Kp) + (e - Kp * DV)) = acc;
    }
}

// ---------------------------------------------------------------------------- read

// Rows [lo, hi) of one problem.  The softmax normalisation cancels between numerator
// and denominator of Eq. 7: with e_k = exp2(s_k - m) and L = sum_k e_k,
//   O = sum_k e_k Vt_k / (sum_k e_k Z_k + eps L),
// so the MFMA takes e (bf16) directly and the denominator D + eps L is formed in fp32.
// Software-pipelined like the write kernel.  Iteration r, region A (one basic block,
// MFMA and VALU interleaved): MFMAs of round r-1's output O^T = Vt^T e^T (e of round r-1
// in LDS, Vt hi + lo in LDS) and of round r+1's scores; VALU: softmax statistics of round
// r (and, with a double-buffered x tile, the split of x tile r+2)  -> B1
// Region B: round r-1's output scaled by 1 / den and stored; e of round r and its
// denominator into LDS (single x buffer: x tile r+2 too)  -> B2
template <int DR, int KT, int VT>
__global__ void __launch_bounds__((Split<DR, KT>::NW * 64)) read_kernel(const uint16_t* __restrict__ XQ, int64_t N,
                                                                       int H, int64_t rows_per_block,
                                                                       Mixture mx, const uint16_t* __restrict__ memory,
                                                                       float eps,
                                                                       uint16_t* __restrict__ O) {
    using S = Split<DR, KT>;
    constexpr int NW = S::NW, NT = NW * 64;
    constexpr int Kp = KT * 32, DV = VT * 32;
    constexpr int LDG = Kp + 8, LDM = Kp + 8;
    constexpr int PAIRS = S::TS * VT;  // (token subtile, value tile) output tiles per round
    constexpr int PW = (PAIRS + NW - 1) / NW;
    constexpr bool PEVEN = PAIRS % NW == 0;
    using XT = XTile<DR, S::ROUND, NT>;
    // VtT hi/lo staged in LDS when it fits; otherwise read from L2
    constexpr bool MS_LDS = (2 * DV * LDM + S::ROUND * LDG) * 2 + XT::LDS_BYTES <= 150 * 1024;
    constexpr int BASE_LDS = S::TS * S::CS * 32 * 12 + S::ROUND * LDG * 2 + (MS_LDS ? 2 * DV * LDM * 2 : 0) +
                             2 * S::ROUND * 4;
    constexpr int XB = (BASE_LDS + 2 * XT::LDS_BYTES <= 80 * 1024) ? 2 : 1;  // keep two workgroups per CU
    constexpr int MF_A = 5 * S::CTW * S::KS + PW * 2 * (Kp / 16);
    __shared__ Stats st[S::TS * S::CS * 32];
    __shared__ __attribute__((aligned(16))) u32x4 Xt[XB][XT::LDS_BYTES / 16];
    __shared__ __attribute__((aligned(16))) uint16_t Gs[S::ROUND * LDG];
    __shared__ __attribute__((aligned(16))) uint16_t Ms[MS_LDS ? 2 * DV * LDM : 8];
    __shared__ float den_s[2][S::ROUND];

    const int wave = wave_id(), l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const int cs = wave % S::CS, ts = wave / S::CS;
    const int64_t p = blockIdx.y;
    const int h = int(p % H);
    const int64_t lo = int64_t(blockIdx.x) * rows_per_block, hi = min<int64_t>(lo + rows_per_block, N);
    const int64_t rows = hi - lo;
    const int64_t R = (rows + S::ROUND - 1) / S::ROUND;
    using MS = MixtureStage<DR, Kp, NT>;
    constexpr bool STAGE = sizeof(Xt) >= MS::LDS_BYTES;
    WaveParams<DR, S::CTW> P;
    typename WaveParams<DR, S::CTW>::Raw praw;
    MS mstage;
    if constexpr (STAGE) {
        mstage.load(mx, h);
        P.fetch_pi(mx, h, cs * S::CTW, praw);
    } else {
        P.fetch(mx, h, cs * S::CTW, praw);
    }
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(XQ + (size_t(p) * N + lo) * DR, rows * DR * 2);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + (size_t(p) * N + lo) * DV, rows * DV * 2);
    // latent memory of this problem: Z -> registers in score-row order (loaded before the
    // x tiles, so their wait covers it), VtT hi/lo -> LDS
    const uint16_t* mp = memory + size_t(p) * Kp * (DV + 1) * 2;
    const float* Zp = reinterpret_cast<const float*>(mp + size_t(2) * DV * Kp);
    float zr[S::CTW][16];
#pragma unroll
    for (int ct = 0; ct < S::CTW; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) zr[ct][r] = Zp[(cs * S::CTW + ct) * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)];
    const uint16_t* Msrc = MS_LDS ? Ms : mp;
    constexpr int LDMS = MS_LDS ? LDM : Kp;

    XT xt;
    f32x16 acc_a[S::CTW], acc_b[S::CTW], acc_a_init[S::CTW];
    {
        XT xt1;
        xt.load(rx, 0);
        xt1.load(rx, S::ROUND);
        if constexpr (STAGE) {  // while the tiles are in flight
            mstage.commit(reinterpret_cast<float*>(&Xt[0][0]));
            __syncthreads();
            P.template read_staged<Kp>(reinterpret_cast<const float*>(&Xt[0][0]), cs * S::CTW, praw);
            P.build(praw, mx.K, cs * S::CTW);
            __syncthreads();  // staging area free for the x tiles
        } else {
            P.build(praw, mx.K, cs * S::CTW);
        }
        if (MS_LDS)
            for (int c = threadIdx.x; c < 2 * DV * Kp / 8; c += NT) {
                const int row = c / (Kp / 8), col = (c - row * (Kp / 8)) * 8;
                *reinterpret_cast<u32x4*>(Ms + row * LDM + col) =
                    *reinterpret_cast<const u32x4*>(mp + size_t(row) * Kp + col);
            }
        xt.commit(Xt[0]);
        xt.load(rx, 2 * S::ROUND);
        if (XB == 2) xt1.commit(Xt[XB - 1]);
        __syncthreads();
        if (XB == 1) {
            scores_lds<DR, S::CTW>(P, Xt[0], ts, acc_a_init);
            __syncthreads();  // x tile 0 consumed by every wave
            xt1.commit(Xt[0]);
            __syncthreads();
        }
    }
    if (XB == 2) scores_lds<DR, S::CTW>(P, Xt[0], ts, acc_a);
    else
#pragma unroll
        for (int ct = 0; ct < S::CTW; ++ct) acc_a[ct] = acc_a_init[ct];

    f32x16 o[PW];
    auto out_mfma = [&]() __attribute__((always_inline)) {  // O^T tiles of the round whose e is in LDS
#pragma unroll
        for (int q = 0; q < PW; ++q) {
            const int pair = wave + q * NW;
            if (PEVEN || pair < PAIRS) {
                const int tsub = pair / VT, vt = pair - tsub * VT;
#pragma unroll
                for (int r = 0; r < 16; ++r) o[q][r] = 0.0f;
#pragma unroll
                for (int ks = 0; ks < Kp / 16; ++ks) {
                    const bf16x8 b = read_rowfrag(Gs, LDG, tsub * 32 + j, 16 * ks);
                    const bf16x8 ah = read_rowfrag(Msrc, LDMS, vt * 32 + j, 16 * ks);
                    const bf16x8 al = read_rowfrag(Msrc + DV * LDMS, LDMS, vt * 32 + j, 16 * ks);
                    o[q] = mfma(ah, b, o[q]);
                    o[q] = mfma(al, b, o[q]);
                }
            }
        }
    };
    auto out_store = [&](const int64_t rr) __attribute__((always_inline)) {  // round rr's outputs
#pragma unroll
        for (int q = 0; q < PW; ++q) {
            const int pair = wave + q * NW;
            if (PEVEN || pair < PAIRS) {
                const int tsub = pair / VT, vt = pair - tsub * VT;
                const float rden = __builtin_amdgcn_rcpf(den_s[rr & 1][tsub * 32 + j]);
                const uint32_t off = uint32_t(((rr * S::ROUND + tsub * 32 + j) * DV + vt * 32 + 4 * lh) * 2);
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    u32x2 v;
                    v[0] = pack_bf16x2(o[q][4 * qq + 0] * rden, o[q][4 * qq + 1] * rden);
                    v[1] = pack_bf16x2(o[q][4 * qq + 2] * rden, o[q][4 * qq + 3] * rden);
                    buf_store8(ro, off + 16 * qq, v);  // rows past hi are dropped by the range check
                }
            }
        }
    };

    auto iteration = [&](const int64_t r, f32x16 (&cur)[S::CTW], f32x16 (&nxt)[S::CTW]) __attribute__((always_inline)) {
        const int xb1 = int((r + 1) % XB);
        // ---- region A
        out_mfma();  // round r-1 (on zero-padded or stale e for r = 0: never stored)
        scores_lds<DR, S::CTW>(P, Xt[xb1], ts, nxt);
        if (XB == 2) {
            xt.commit(Xt[xb1 ^ 1]);
            xt.load(rx, (r + 3) * S::ROUND);
        }
        float m, L, D;
        local_softmax<S::CTW, true>(cur, zr, m, L, D);
        if (S::CS > 1) st[(ts * S::CS + cs) * 32 + j] = Stats{m, L, D};  // both lane halves hold the same
#pragma unroll
        for (int i = 0; i < MF_A; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
        __syncthreads();  // B1
        // ---- region B
        if (r > 0) out_store(r - 1);
        float scale = 1.0f, den = D + eps * L;
        if (S::CS > 1) {
            float mm = -INFINITY;
#pragma unroll
            for (int c = 0; c < S::CS; ++c) mm = fmaxf(mm, st[(ts * S::CS + c) * 32 + j].m);
            float Lt = 0.0f, Dt = 0.0f;
#pragma unroll
            for (int c = 0; c < S::CS; ++c) {
                const Stats sc = st[(ts * S::CS + c) * 32 + j];
                const float f = __builtin_amdgcn_exp2f(sc.m - mm);
                Lt = fmaf(sc.L, f, Lt);
                Dt = fmaf(sc.D, f, Dt);
            }
            scale = __builtin_amdgcn_exp2f(m - mm);
            den = Dt + eps * Lt;
        }
        store_gamma_lds<S::CTW>(cur, scale, Gs, LDG, ts * 32 + j, cs * S::CTW);
        if (cs == 0 && lh == 0) den_s[r & 1][ts * 32 + j] = den;
        if (XB == 1) {
            xt.commit(Xt[0]);
            xt.load(rx, (r + 3) * S::ROUND);
        }
        __syncthreads();  // B2
    };
    for (int64_t r = 0; r < R; r += 2) {
        iteration(r, acc_a, acc_b);
        if (r + 1 < R) iteration(r + 1, acc_b, acc_a);
    }
    out_mfma();
    out_store(R - 1);
}

// ---------------------------------------------------------------------------- dispatch

template <typename F>
hipError_t with_dr_kt(int dr, int kt, F&& f) {
#define GMA_CASE(D, T) \
    if (dr == D && kt == T) return f(std::integral_constant<int, D>(), std::integral_constant<int, T>());
#define GMA_DR(D) GMA_CASE(D, 1) GMA_CASE(D, 2) GMA_CASE(D, 4) GMA_CASE(D, 8)
    GMA_DR(16) GMA_DR(32) GMA_DR(64) GMA_DR(128)
#undef GMA_DR
#undef GMA_CASE
    return hipErrorNotSupported;
}

template <typename F>
hipError_t with_vt(int vt, F&& f) {
    if (vt == 1) return f(std::integral_constant<int, 1>());
    if (vt == 2) return f(std::integral_constant<int, 2>());
    if (vt == 4) return f(std::integral_constant<int, 4>());
    return hipErrorNotSupported;
}

}  // namespace bf

namespace {

int kt_of(const Plan& p) { return int(p.Kp / 32); }

}  // namespace

int64_t bf16_round_tokens(int dr, int64_t Kp) {
    int64_t out = 0;
    (void)bf::with_dr_kt(dr, int(Kp / 32), [&](auto D, auto T) {
        out = bf::Split<decltype(D)::value, decltype(T)::value>::ROUND;
        return hipSuccess;
    });
    return out;
}

hipError_t bf16_responsibilities(const Plan& p, const void* X, const float* mu, const float* s2, const float* pi,
                                 void* Gamma, gma_dtype_t gamma_dtype, char* ws, hipStream_t st) {
    (void)ws;
    const bf::Mixture mx{mu, s2, pi, int(p.K)};
    return bf::with_dr_kt(int(p.dr), kt_of(p), [&](auto D, auto T) {
        constexpr int DR = decltype(D)::value, KT = decltype(T)::value;
        using S = bf::Split<DR, KT>;
        dim3 grid(unsigned((p.N + S::ROUND - 1) / S::ROUND), unsigned(p.P));
        GMA_LAUNCH("bf16_resp", (bf::resp_kernel<DR, KT>), grid, dim3(S::NW * 64), 0, st,
                           static_cast<const uint16_t*>(X), p.N, int(p.H), mx, Gamma,
                           gamma_dtype == GMA_BF16 ? 1 : 0);
        return hipGetLastError();
    });
}

hipError_t bf16_write_partials(const Plan& p, const void* XK, const void* V, const bf::Mixture& mx, char* ws,
                               hipStream_t st, int64_t splits) {
    float* partials = reinterpret_cast<float*>(ws + p.off_partials);
    return bf::with_dr_kt(int(p.dr), kt_of(p), [&](auto D, auto T) {
        constexpr int DR = decltype(D)::value, KT = decltype(T)::value;
        return bf::with_vt(int(p.dv / 32), [&](auto VV) {
            constexpr int VT = decltype(VV)::value;
            using S = bf::Split<DR, KT>;
            GMA_LAUNCH(p.op == GMA_OP_CAUSAL ? "bf16_causal_aggregate" : "bf16_write", (bf::write_kernel<DR, KT, VT>), dim3(unsigned(splits), unsigned(p.P)), dim3(S::NW * 64), 0,
                               st, static_cast<const uint16_t*>(XK), static_cast<const uint16_t*>(V), p.N, int(p.H),
                               p.seg, int(p.G), mx, partials);
            return hipGetLastError();
        });
    });
}

hipError_t bf16_bidir(const Plan& p, const void* XQ, const void* XK, const void* V, const float* mu, const float* s2,
                      const float* pi, float eps, void* O, char* ws, hipStream_t st) {
    const bf::Mixture mx{mu, s2, pi, int(p.K)};
    hipError_t e = bf16_write_partials(p, XK, V, mx, ws, st, p.G);
    if (e != hipSuccess) return e;
    float* partials = reinterpret_cast<float*>(ws + p.off_partials);
    uint16_t* memory = reinterpret_cast<uint16_t*>(ws + p.off_memory);
    const int E = int(p.Kp * (p.dv + 1));
    GMA_LAUNCH("bf16_combine", bf::combine_kernel, dim3(unsigned((E / 4 + 255) / 256), unsigned(p.P)), dim3(256), 0, st, partials,
                       int(p.G), int(p.Kp), int(p.dv), memory);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return bf::with_dr_kt(int(p.dr), kt_of(p), [&](auto D, auto T) {
        constexpr int DR = decltype(D)::value, KT = decltype(T)::value;
        return bf::with_vt(int(p.dv / 32), [&](auto VV) {
            constexpr int VT = decltype(VV)::value;
            using S = bf::Split<DR, KT>;
            dim3 grid(unsigned((p.N + p.read_rows - 1) / p.read_rows), unsigned(p.P));
            GMA_LAUNCH("bf16_read", (bf::read_kernel<DR, KT, VT>), grid, dim3(S::NW * 64), 0, st,
                               static_cast<const uint16_t*>(XQ), p.N, int(p.H), p.read_rows, mx, memory,
                               eps, static_cast<uint16_t*>(O));
            return hipGetLastError();
        });
    });
}

hipError_t bf16_causal(const Plan& p, const void* XQ, const void* XK, const void* V, const float* mu, const float* s2,
                       const float* pi, float eps, void* O, char* ws, hipStream_t st) {
    const bf::Mixture mx{mu, s2, pi, int(p.K)};
    hipError_t e = hipSuccess;
    // aggregates of segments 0 .. G-2 (the last segment's aggregate is never read); the
    // scan workgroup of segment s sums aggregates 0 .. s-1 itself
    if (p.G > 1 && (e = bf16_write_partials(p, XK, V, mx, ws, st, p.G - 1)) != hipSuccess) return e;
    return bf16_scan(p, XQ, XK, V, mu, s2, pi, eps, O, ws, st);
}

}  // namespace gma
