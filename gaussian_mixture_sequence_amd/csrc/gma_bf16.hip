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
// Every kernel builds the score operands from mu, sigma2 and pi itself (PlaneBuilder: each
// (component, dim) pair once per workgroup, through LDS; WaveParams::compute per wave where
// the planes do not fit), so no launch is spent on the parameters.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "gma_bf16_common.h"
#include "gma_bf16_phases.h"
#include "gma_internal.h"

namespace gma {
namespace bf {

// ---------------------------------------------------------------------------- responsibilities

// Grid (G, P): workgroup (g, p) computes Gamma for rounds [g RPW, (g + 1) RPW) of problem p
// (ROUND tokens each), so the operand planes, built once per workgroup, serve RPW rounds.
template <int DR, int KT>
constexpr size_t resp_plane_bytes() {
    return PlaneBuilder<DR, KT * 32, Split<DR, KT>::NW * 64>::LDS_BYTES <= 96 * 1024
               ? PlaneBuilder<DR, KT * 32, Split<DR, KT>::NW * 64>::LDS_BYTES
               : 16;
}

template <int DR, int KT>
__global__ void __launch_bounds__((Split<DR, KT>::NW * 64)) resp_kernel(const uint16_t* __restrict__ X, int64_t N,
                                                                       int H, int RPW, Mixture mx, void* Gamma,
                                                                       int gamma_bf16) {
    using S = Split<DR, KT>;
    constexpr int NT = S::NW * 64, Kp = KT * 32;
    using PB = PlaneBuilder<DR, Kp, NT>;
    constexpr bool COOP = resp_plane_bytes<DR, KT>() > 16;
    __shared__ Stats st[S::TS * S::CS * 32];
    __shared__ __attribute__((aligned(16))) char planes[resp_plane_bytes<DR, KT>()];
    const int wave = wave_id(), l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const int cs = wave % S::CS, ts = wave / S::CS;
    const int64_t p = blockIdx.y;
    const int h = int(p % H), K = mx.K;
    WaveParams<DR, S::CTW> P;
    if constexpr (COOP) {  // each (component, dim) pair once per workgroup
        PB pb;
        pb.load(mx, h);
        pb.build(planes, K);
        __syncthreads();
        P.template read_planes<Kp>(planes, cs * S::CTW);
    } else {
        P.compute(mx, h, cs * S::CTW);
    }
    const uint16_t* Xp = X + size_t(p) * N * DR;
    const bool vec = (K & 3) == 0;  // whole groups of 4 components: 16- or 8-byte stores
    // the wave's x fragments are loaded one round ahead of their scores
    auto first_row = [&](int r) { return (int64_t(blockIdx.x) * RPW + r) * S::ROUND + ts * 32; };
    auto rows_of = [&](int64_t n0) { return int(max<int64_t>(0, min<int64_t>(32, N - n0))); };
    bf16x8 xs[DR / 16];
    load_x<DR>(Xp, first_row(0), rows_of(first_row(0)), xs);
    for (int r = 0; r < RPW; ++r) {
        const int64_t n0 = first_row(r);
        if (n0 - ts * 32 >= N) break;  // uniform over the workgroup
        const int valid = rows_of(n0);
        bf16x8 xn[DR / 16];
        load_x<DR>(Xp, first_row(r + 1), r + 1 < RPW ? rows_of(first_row(r + 1)) : 0, xn);
        f32x16 acc[S::CTW];
        scores_x<DR, S::CTW>(P, xs, acc);
#pragma unroll
        for (int ks = 0; ks < DR / 16; ++ks) xs[ks] = xn[ks];
        float m, L, D;
        float zr[S::CTW][16];
        local_softmax<S::CTW, false>(acc, zr, m, L, D);
        if (S::CS > 1) {
            __syncthreads();  // the previous round's statistics are read
            if (lh == 0) st[(ts * S::CS + cs) * 32 + j] = Stats{m, L, 0.0f};
            __syncthreads();
        }
        float dl;
        const float scale = combine_stats<S::CS>(st, ts, cs, j, m, L, 0.0f, dl);
        if (j >= valid) continue;
        const size_t rowoff = (size_t(p) * N + n0 + j) * K;
#pragma unroll
        for (int ct = 0; ct < S::CTW; ++ct)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int comp = (cs * S::CTW + ct) * 32 + 8 * q + 4 * lh;
                const float g0 = acc[ct][4 * q] * scale, g1 = acc[ct][4 * q + 1] * scale;
                const float g2 = acc[ct][4 * q + 2] * scale, g3 = acc[ct][4 * q + 3] * scale;
                if (vec) {
                    if (comp < K) {
                        if (gamma_bf16)
                            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(Gamma) + rowoff + comp) =
                                u32x2{pack_bf16x2(g0, g1), pack_bf16x2(g2, g3)};
                        else
                            *reinterpret_cast<float4*>(static_cast<float*>(Gamma) + rowoff + comp) =
                                make_float4(g0, g1, g2, g3);
                    }
                } else {
                    const float gg[4] = {g0, g1, g2, g3};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (comp + e < K) {
                            if (gamma_bf16)
                                static_cast<uint16_t*>(Gamma)[rowoff + comp + e] = f32_to_bf16_bits(gg[e]);
                            else
                                static_cast<float*>(Gamma)[rowoff + comp + e] = gg[e];
                        }
                    }
                }
            }
    }
}

// ---------------------------------------------------------------------------- write (standalone)

// Grid (G, P): split g of problem p into its partial.
template <int DR, int KT, int VT>
__global__ void __launch_bounds__((Split<DR, KT>::NW * 64))
__attribute__((amdgpu_waves_per_eu(waves_for_lds(WriteLds<DR, KT, VT>::bytes)))) write_kernel(const uint16_t* __restrict__ XK,
                                                                        const uint16_t* __restrict__ V, int64_t N,
                                                                        int H, int64_t seg, int G,
                                                                        Mixture mx, float* __restrict__ partials) {
    __shared__ __attribute__((aligned(16))) char smem[WriteLds<DR, KT, VT>::bytes];
    constexpr int Kp = KT * 32, DV = VT * 32;
    const int64_t p = blockIdx.y;
    const int g = blockIdx.x;
    const int64_t lo = min<int64_t>(int64_t(g) * seg, N), hi = min<int64_t>(lo + seg, N);
    WaveParams<DR, Split<DR, KT>::CTW> P;
    write_body<DR, KT, VT, true>(smem, XK, V, N, p, int(p % H), lo, hi, mx, P,
                                 partials + (size_t(p) * G + g) * size_t(Kp) * (DV + 1));
}

// ---------------------------------------------------------------------------- combine

// Bidirectional: memory = sum_g partial_g (increasing g), then the read operands:
// VtT_hi, VtT_lo [DV][Kp] bf16 (Vt transposed, hi + lo split) and Z [Kp] fp32.  The
// partials use the same [DV][Kp] + [Kp] order, so every access is coalesced.
//
// 16-byte groups [c0, c1) of one problem's memory: the G partials summed in increasing
// order, VtT split into hi + lo bf16 planes, Z kept in fp32, all through device-coherent
// accesses.  Kp * DV is a multiple of 4, so a group never straddles the VtT / Z boundary.
// part: the problem's G partials of E floats; base: its memory (E floats of room).
__device__ __forceinline__ void combine_range(const float* __restrict__ part, int G, int E, int Kp, int DV, int c0,
                                              int c1, uint16_t* __restrict__ base, int stride) {
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(part, int64_t(G) * E * 4);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(base, int64_t(E) * 4);
    constexpr int GB = 8;  // partials loaded together (one memory round trip per batch)
    for (int c = c0 + int(threadIdx.x); c < c1; c += stride) {
        const int e = 4 * c;
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int g0 = 0; g0 < G; g0 += GB) {
            u32x4 v[GB];
#pragma unroll
            for (int u = 0; u < GB; ++u)  // past the last partial: a repeat of it, not added
                v[u] = buf_load16_dev(rp, uint32_t((size_t(min(g0 + u, G - 1)) * E + e) * 4));
#pragma unroll
            for (int u = 0; u < GB; ++u) {
                if (g0 + u < G) {
                    acc.x = g0 + u == 0 ? __uint_as_float(v[u][0]) : acc.x + __uint_as_float(v[u][0]);
                    acc.y = g0 + u == 0 ? __uint_as_float(v[u][1]) : acc.y + __uint_as_float(v[u][1]);
                    acc.z = g0 + u == 0 ? __uint_as_float(v[u][2]) : acc.z + __uint_as_float(v[u][2]);
                    acc.w = g0 + u == 0 ? __uint_as_float(v[u][3]) : acc.w + __uint_as_float(v[u][3]);
                }
            }
        }
        if (e < Kp * DV) {
            const uint32_t h01 = pack_bf16x2(acc.x, acc.y), h23 = pack_bf16x2(acc.z, acc.w);
            const uint32_t l01 = pack_bf16x2(acc.x - __uint_as_float(h01 << 16), acc.y - __uint_as_float(h01 & 0xffff0000u));
            const uint32_t l23 = pack_bf16x2(acc.z - __uint_as_float(h23 << 16), acc.w - __uint_as_float(h23 & 0xffff0000u));
            buf_store8_dev(rb, uint32_t(e * 2), u32x2{h01, h23});
            buf_store8_dev(rb, uint32_t((Kp * DV + e) * 2), u32x2{l01, l23});
        } else {
            buf_store16_dev(rb, uint32_t(4 * Kp * DV + (e - Kp * DV) * 4),
                            u32x4{__float_as_uint(acc.x), __float_as_uint(acc.y), __float_as_uint(acc.z),
                                  __float_as_uint(acc.w)});
        }
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
// LDS of read_body, carved in this order out of one workgroup buffer.
template <int DR, int KT, int VT>
struct ReadLds {
    using S = Split<DR, KT, true>;
    static constexpr int NT = S::NW * 64, Kp = KT * 32, DV = VT * 32, LDG = Kp + 8, LDM = Kp + 8;
    using XT = XTile<DR, S::ROUND, NT>;
    // VtT hi/lo staged in LDS when it fits; otherwise read from L2
    static constexpr bool MS_LDS = (2 * DV * LDM + S::ROUND * LDG) * 2 + XT::LDS_BYTES <= 150 * 1024;
    using st_t = Stats[S::CS > 1 ? S::TS * S::CS * 32 : 1];  // unused with one component group
    using gs_t = uint16_t[S::ROUND * LDG];
    using ms_t = uint16_t[MS_LDS ? 2 * DV * LDM : 8];
    using dn_t = float[2][S::ROUND];
    using vote_t = int[S::NW];  // per-wave votes of the fused kernel's hand-off (workgroup_all)
    // everything but the x tiles, as laid out below; two x buffers only if the whole still
    // keeps two workgroups per CU
    static constexpr size_t REST = lds_align(sizeof(st_t)) + lds_align(sizeof(gs_t)) + lds_align(sizeof(ms_t)) +
                                   lds_align(sizeof(dn_t)) + lds_align(sizeof(vote_t));
    static constexpr int XB = (REST + 2 * size_t(XT::LDS_BYTES) <= 80 * 1024) ? 2 : 1;
    using xt_t = u32x4[XB][XT::LDS_BYTES / 16];
    static constexpr size_t o_st = 0, o_xt = lds_align(o_st + sizeof(st_t)), o_gs = lds_align(o_xt + sizeof(xt_t)),
                            o_ms = lds_align(o_gs + sizeof(gs_t)), o_dn = lds_align(o_ms + sizeof(ms_t)),
                            o_vote = lds_align(o_dn + sizeof(dn_t)), bytes = lds_align(o_vote + sizeof(vote_t));
};

// Rows [lo, hi) of problem p (head h): O = Gamma_Q Vt / (Gamma_Q Z + eps) from the problem's
// latent memory `mp` (VtT hi, VtT lo [DV][Kp] bf16, then Z [Kp] fp32; read device-coherent,
// as another workgroup of the launch writes it).  BUILD as in write_body.  wait() runs
// after the first x tiles are committed and round 0's scores issued, before `mp` is read:
// a fused kernel completes the memory there, behind that work.
template <int DR, int KT, int VT, bool BUILD, typename WaitF>
__device__ __forceinline__ void read_body(char* __restrict__ smem, const uint16_t* __restrict__ XQ, int64_t N,
                                          int64_t p, int h, int64_t lo, int64_t hi, const Mixture& mx,
                                          WaveParams<DR, Split<DR, KT, true>::CTW>& P, const uint16_t* mp, float eps,
                                          uint16_t* __restrict__ O, WaitF&& wait) {
    using S = Split<DR, KT, true>;
    using LY = ReadLds<DR, KT, VT>;
    constexpr int NW = S::NW, NT = NW * 64;
    constexpr int Kp = KT * 32, DV = VT * 32;
    constexpr int LDG = Kp + 8, LDM = Kp + 8;
    constexpr int PAIRS = S::TS * VT;  // (token subtile, value tile) output tiles per round
    constexpr int PW = (PAIRS + NW - 1) / NW;
    constexpr bool PEVEN = PAIRS % NW == 0;
    using XT = XTile<DR, S::ROUND, NT>;
    constexpr bool MS_LDS = LY::MS_LDS;
    constexpr int XB = LY::XB;
    constexpr int MF_A = 5 * S::CTW * S::KS + PW * 2 * (Kp / 16);
    typename LY::st_t& st = *reinterpret_cast<typename LY::st_t*>(smem + LY::o_st);
    typename LY::xt_t& Xt = *reinterpret_cast<typename LY::xt_t*>(smem + LY::o_xt);
    typename LY::gs_t& Gs = *reinterpret_cast<typename LY::gs_t*>(smem + LY::o_gs);
    typename LY::ms_t& Ms = *reinterpret_cast<typename LY::ms_t*>(smem + LY::o_ms);
    typename LY::dn_t& den_s = *reinterpret_cast<typename LY::dn_t*>(smem + LY::o_dn);

    const int wave = wave_id(), l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const int cs = wave % S::CS, ts = wave / S::CS;
    const int64_t rows = hi - lo;
    const int64_t R = (rows + S::ROUND - 1) / S::ROUND;
    using PB = PlaneBuilder<DR, Kp, NT>;
    constexpr bool COOP = sizeof(Xt) >= PB::LDS_BYTES;
    typename WaveParams<DR, S::CTW>::Raw praw;
    PB pb;
    if constexpr (BUILD) {
        if constexpr (COOP) pb.load(mx, h);
        else P.fetch(mx, h, cs * S::CTW, praw);
    }
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(XQ + (size_t(p) * N + lo) * DR, rows * DR * 2);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + (size_t(p) * N + lo) * DV, rows * DV * 2);
    // latent memory of this problem (read after wait()): Z -> registers in score-row order,
    // VtT hi/lo -> LDS
    const __amdgpu_buffer_rsrc_t rmp = make_rsrc(mp, int64_t(Kp) * (DV + 1) * 4);
    float zr[S::CTW][16];
    const uint16_t* Msrc = MS_LDS ? Ms : mp;
    constexpr int LDMS = MS_LDS ? LDM : Kp;

    XT xt;
    f32x16 acc_a[S::CTW], acc_b[S::CTW], acc_a_init[S::CTW];
    {
        XT xt1;
        xt.load(rx, 0);
        xt1.load(rx, S::ROUND);
        if constexpr (BUILD && COOP) {  // while the tiles are in flight
            pb.build(reinterpret_cast<char*>(&Xt[0][0]), mx.K);
            __syncthreads();
            P.template read_planes<Kp>(reinterpret_cast<const char*>(&Xt[0][0]), cs * S::CTW);
            __syncthreads();  // staging area free for the x tiles
        } else if constexpr (BUILD) {
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
    if (XB == 2) scores_lds<DR, S::CTW>(P, Xt[0], ts, acc_a);
    else
#pragma unroll
        for (int ct = 0; ct < S::CTW; ++ct) acc_a[ct] = acc_a_init[ct];

    // the latent memory: only now (a fused kernel waits here for it to be complete)
    wait();
#pragma unroll
    for (int ct = 0; ct < S::CTW; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 zv = buf_load16_dev(rmp, uint32_t(4 * Kp * DV + ((cs * S::CTW + ct) * 32 + 8 * q + 4 * lh) * 4));
#pragma unroll
            for (int i = 0; i < 4; ++i) zr[ct][4 * q + i] = __uint_as_float(zv[i]);
        }
    if constexpr (MS_LDS) {  // VtT hi/lo: all loads in flight before the first LDS store
        constexpr int MCH = 2 * DV * Kp / 8, MPER = (MCH + NT - 1) / NT;
        u32x4 mv[MPER];
#pragma unroll
        for (int u = 0; u < MPER; ++u) {
            const int c = threadIdx.x + u * NT;
            const int row = c / (Kp / 8), col = (c - row * (Kp / 8)) * 8;
            if (MCH % NT == 0 || c < MCH) mv[u] = buf_load16_dev(rmp, uint32_t((row * Kp + col) * 2));
        }
#pragma unroll
        for (int u = 0; u < MPER; ++u) {
            const int c = threadIdx.x + u * NT;
            const int row = c / (Kp / 8), col = (c - row * (Kp / 8)) * 8;
            if (MCH % NT == 0 || c < MCH) *reinterpret_cast<u32x4*>(Ms + row * LDM + col) = mv[u];
        }
        __syncthreads();  // VtT in LDS for every wave
    }

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
        // ---- region A (raised priority while feeding the matrix cores, as in write_body)
        __builtin_amdgcn_s_setprio(1);
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
        __builtin_amdgcn_s_setprio(0);
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

// ---------------------------------------------------------------------------- bidirectional forward

// One launch for the whole bidirectional forward.  Grid (G, P); workgroup (g, p) owns key
// rows [g seg, (g + 1) seg) and query rows [g seg_q, (g + 1) seg_q) of problem p (the same
// rows unless the queries come from another sequence than the keys, as in cross-attention;
// either range may then be empty):
//   1. write: the partial [Vt^T | Z] of its rows (write_body, operand planes built once);
//   2. read phase (read_body, same planes): its first x tiles committed and round 0's
//      scores issued, which need no memory;
//   3. after all G partials of p are published: combine 1/G of p's memory (fixed order);
//   4. after all G slices are published: the rest of the read phase.
// Steps 3 and 4 wait on every workgroup of the problem, so the host launches this kernel
// only when its whole grid can be resident at once (otherwise the three phases run as
// separate launches: write_kernel, combine_kernel, read_kernel).
// flags: [P][2][G] words (partials ready, memory slice ready), compared with `token`.  A
// workgroup whose first wait times out neither combines nor publishes its slice, so no
// workgroup ever reads a memory summed from incomplete partials; every workgroup of the
// problem then times out in turn, writes NaN over its output rows and raises
// kDevErrTimeout in `err`.
template <int DR, int KT, int VT>
constexpr size_t bidir_lds_bytes() {
    return WriteLds<DR, KT, VT>::bytes > ReadLds<DR, KT, VT>::bytes ? WriteLds<DR, KT, VT>::bytes
                                                                     : ReadLds<DR, KT, VT>::bytes;
}

template <int DR, int KT, int VT>
__global__ void __launch_bounds__((Split<DR, KT>::NW * 64))
__attribute__((amdgpu_waves_per_eu(waves_for_lds(bidir_lds_bytes<DR, KT, VT>()))))
    bidir_kernel(const uint16_t* __restrict__ XQ, const uint16_t* __restrict__ XK, const uint16_t* __restrict__ V,
                 int64_t N, int64_t Nq, int H, int64_t seg, int64_t seg_q, int G, Mixture mx, float* __restrict__ partials,
                 uint16_t* __restrict__ memory, uint64_t* __restrict__ flags, uint64_t token,
                 uint32_t wait_limit, float eps, uint16_t* __restrict__ O, uint32_t* __restrict__ err) {
    using RL = ReadLds<DR, KT, VT>;
    __shared__ __attribute__((aligned(16))) char smem[bidir_lds_bytes<DR, KT, VT>()];
    constexpr int Kp = KT * 32, DV = VT * 32, E = Kp * (DV + 1), NT = Split<DR, KT>::NW * 64;
    const int64_t p = blockIdx.y;
    const int g = blockIdx.x, h = int(p % H);
    const int64_t lo = min<int64_t>(int64_t(g) * seg, N), hi = min<int64_t>(lo + seg, N);
    const int64_t lo_q = min<int64_t>(int64_t(g) * seg_q, Nq), hi_q = min<int64_t>(lo_q + seg_q, Nq);
    float* part = partials + size_t(p) * G * E;
    uint16_t* mem = memory + size_t(p) * E * 2;
    uint64_t* fl = flags + size_t(p) * 2 * G;

    WaveParams<DR, Split<DR, KT>::CTW> P;
    write_body<DR, KT, VT, true>(smem, XK, V, N, p, h, lo, hi, mx, P, part + size_t(g) * E);
    publish_token(fl + g, token);  // its barrier also frees the write phase's LDS
    bool ok = true;
    auto complete = [&] {
        // behind the read phase's first tiles and scores: complete the memory.  The waves
        // poll on their own and agree before the combine, which needs every wave.
        ok = workgroup_all(wait_tokens(fl, G, token, wait_limit), reinterpret_cast<int*>(smem + RL::o_vote));
        if (ok) {
            const int per = (E / 4 + G - 1) / G;  // 16-byte groups per slice
            combine_range(part, G, E, Kp, DV, min(g * per, E / 4), min((g + 1) * per, E / 4), mem, NT);
            publish_token(fl + G + g, token);
            ok = wait_tokens(fl + G, G, token, wait_limit);
        }
    };
    if constexpr (Split<DR, KT, true>::CTW == Split<DR, KT>::CTW) {  // the write phase's planes serve
        read_body<DR, KT, VT, false>(smem, XQ, Nq, p, h, lo_q, hi_q, mx, P, mem, eps, O, complete);
    } else {  // the read phase's own split: its planes are built again
        WaveParams<DR, Split<DR, KT, true>::CTW> PR;
        read_body<DR, KT, VT, true>(smem, XQ, Nq, p, h, lo_q, hi_q, mx, PR, mem, eps, O, complete);
    }
    ok = workgroup_all(ok, reinterpret_cast<int*>(smem));
    if (!ok) {  // the memory was never complete: make that visible in the output and to the host
        __builtin_amdgcn_s_waitcnt(0);  // the phase's own stores of these rows land first
        __syncthreads();
        uint16_t* op = O + (size_t(p) * Nq + lo_q) * DV;
        for (int64_t e = threadIdx.x; e < (hi_q - lo_q) * DV; e += NT) op[e] = 0x7fc0u;
        if (threadIdx.x == 0) atomicOr(err, kDevErrTimeout);
    }
}

// The bidirectional forward as three launches with no waits between workgroups (used when
// the single launch's grid cannot be resident at once, or when the caller asks for it):
// write_kernel (partials), combine_kernel (the memory, slice g of problem p per workgroup,
// the same fixed order as the single launch), read_kernel.
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ partials, int G, int Kp, int DV,
                                                      uint16_t* __restrict__ memory) {
    const int E = Kp * (DV + 1);
    const int64_t p = blockIdx.y;
    const int g = blockIdx.x;
    const int per = (E / 4 + G - 1) / G;
    combine_range(partials + size_t(p) * G * E, G, E, Kp, DV, min(g * per, E / 4), min((g + 1) * per, E / 4),
                  memory + size_t(p) * E * 2, 256);
}

template <int DR, int KT, int VT>
__global__ void __launch_bounds__((Split<DR, KT>::NW * 64))
__attribute__((amdgpu_waves_per_eu(waves_for_lds(ReadLds<DR, KT, VT>::bytes))))
    read_kernel(const uint16_t* __restrict__ XQ, int64_t Nq, int H, int64_t seg_q, Mixture mx,
                const uint16_t* __restrict__ memory, float eps, uint16_t* __restrict__ O) {
    __shared__ __attribute__((aligned(16))) char smem[ReadLds<DR, KT, VT>::bytes];
    constexpr int Kp = KT * 32, DV = VT * 32, E = Kp * (DV + 1);
    const int64_t p = blockIdx.y;
    const int g = blockIdx.x;
    const int64_t lo_q = min<int64_t>(int64_t(g) * seg_q, Nq), hi_q = min<int64_t>(lo_q + seg_q, Nq);
    if (lo_q >= hi_q) return;  // uniform over the workgroup
    WaveParams<DR, Split<DR, KT, true>::CTW> P;
    read_body<DR, KT, VT, true>(smem, XQ, Nq, p, int(p % H), lo_q, hi_q, mx, P, memory + size_t(p) * E * 2, eps, O,
                                [] {});
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

hipError_t bf16_responsibilities(const Plan& p, const void* X, const float* mu, const float* s2, const float* pi,
                                 void* Gamma, gma_dtype_t gamma_dtype, char* ws, hipStream_t st) {
    (void)ws;
    const bf::Mixture mx{mu, s2, pi, int(p.K)};
    return bf::with_dr_kt(int(p.dr), kt_of(p), [&](auto D, auto T) {
        constexpr int DR = decltype(D)::value, KT = decltype(T)::value;
        using S = bf::Split<DR, KT>;
        // rounds per workgroup: about 512 workgroups in all, so each one's operand build serves
        // several rounds (measured: 2048 workgroups of two rounds took 13% longer at B8 H8 N4096)
        const int64_t rounds = (p.N + S::ROUND - 1) / S::ROUND;
        const int64_t rpw = std::max<int64_t>(1, (p.P * rounds + 511) / 512);
        dim3 grid(unsigned((rounds + rpw - 1) / rpw), unsigned(p.P));
        GMA_LAUNCH("bf16_resp", (bf::resp_kernel<DR, KT>), grid, dim3(S::NW * 64), 0, st,
                           static_cast<const uint16_t*>(X), p.N, int(p.H), int(rpw), mx, Gamma,
                           gamma_dtype == GMA_BF16 ? 1 : 0);
        return hipGetLastError();
    });
}

hipError_t bf16_write_partials(const Plan& p, const void* XK, const void* V, const float* mu, const float* s2,
                               const float* pi, char* ws, hipStream_t st, int64_t splits) {
    const bf::Mixture mx{mu, s2, pi, int(p.K)};
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

void bf16_bidir_geometry(int64_t dr, int64_t kt, int64_t vt, int* threads, int64_t* lds_bytes) {
    *threads = 0;
    *lds_bytes = 0;
    (void)bf::with_dr_kt(int(dr), int(kt), [&](auto D, auto T) {
        constexpr int DR = decltype(D)::value, KT = decltype(T)::value;
        return bf::with_vt(int(vt), [&](auto VV) {
            constexpr int VT = decltype(VV)::value;
            *threads = bf::Split<DR, KT>::NW * 64;
            *lds_bytes = int64_t(bf::bidir_lds_bytes<DR, KT, VT>());
            return hipSuccess;
        });
    });
}

int64_t bf16_bidir_per_cu(int64_t dr, int64_t kt, int64_t vt) {
    int threads = 0;
    int64_t lds = 0;
    bf16_bidir_geometry(dr, kt, vt, &threads, &lds);
    if (threads <= 0 || lds <= 0) return 1;
    // LDS: 160 KiB per CU; waves: the kernels declare the waves per SIMD their LDS allows
    // (bf::waves_for_lds), so the registers of that many waves of every SIMD are guaranteed
    const int64_t by_lds = (160 * 1024) / lds;
    const int64_t by_waves = (int64_t(bf::waves_for_lds(size_t(lds))) * 4 * 64) / threads;
    return std::max<int64_t>(1, std::min(by_lds, by_waves));
}

hipError_t bf16_bidir(const Plan& p, const void* XQ, const void* XK, const void* V, const float* mu, const float* s2,
                      const float* pi, float eps, void* O, char* ws, hipStream_t st) {
    const bf::Mixture mx{mu, s2, pi, int(p.K)};
    float* partials = reinterpret_cast<float*>(ws + p.off_partials);
    uint16_t* memory = reinterpret_cast<uint16_t*>(ws + p.off_memory);
    uint64_t* flags = reinterpret_cast<uint64_t*>(ws + p.off_flags);
    uint32_t* err = nullptr;
    hipError_t e = device_error_word(&err);
    if (e != hipSuccess) return e;
    return bf::with_dr_kt(int(p.dr), kt_of(p), [&](auto D, auto T) {
        constexpr int DR = decltype(D)::value, KT = decltype(T)::value;
        return bf::with_vt(int(p.dv / 32), [&](auto VV) -> hipError_t {
            constexpr int VT = decltype(VV)::value;
            using S = bf::Split<DR, KT>;
            constexpr int NT = S::NW * 64;
            const dim3 grid(unsigned(p.G), unsigned(p.P));
            // the single launch waits on every workgroup of a problem: only when the whole grid
            // is resident at once on this device (with one split per problem nothing waits on
            // another workgroup)
            bool single = single_launch_enabled() && p.G <= kBidirSingleMaxSplits;
            if (single && p.G > 1) {
                int64_t resident = 0;
                hipError_t r = resident_workgroups(reinterpret_cast<const void*>(&bf::bidir_kernel<DR, KT, VT>), NT,
                                                   &resident);
                if (r != hipSuccess) return r;
                single = p.P * p.G <= resident;
            }
            if (single) {
                GMA_LAUNCH(p.cross ? "bf16_cross" : "bf16_bidir", (bf::bidir_kernel<DR, KT, VT>), grid, dim3(NT), 0, st,
                           static_cast<const uint16_t*>(XQ), static_cast<const uint16_t*>(XK),
                           static_cast<const uint16_t*>(V), p.N, p.Nq, int(p.H), p.seg, p.seg_q, int(p.G), mx, partials,
                           memory, flags, launch_token(), wait_limit(), eps, static_cast<uint16_t*>(O), err);
                return hipGetLastError();
            }
            GMA_LAUNCH(p.cross ? "bf16_cross_write" : "bf16_write", (bf::write_kernel<DR, KT, VT>), grid, dim3(NT), 0, st,
                       static_cast<const uint16_t*>(XK), static_cast<const uint16_t*>(V), p.N, int(p.H), p.seg, int(p.G),
                       mx, partials);
            hipError_t r = hipGetLastError();
            if (r != hipSuccess) return r;
            GMA_LAUNCH(p.cross ? "bf16_cross_combine" : "bf16_combine", bf::combine_kernel, grid, dim3(256), 0, st,
                       partials, int(p.G), KT * 32, VT * 32, memory);
            if ((r = hipGetLastError()) != hipSuccess) return r;
            GMA_LAUNCH(p.cross ? "bf16_cross_read" : "bf16_read", (bf::read_kernel<DR, KT, VT>), grid, dim3(NT), 0, st,
                       static_cast<const uint16_t*>(XQ), p.Nq, int(p.H), p.seg_q, mx, memory, eps,
                       static_cast<uint16_t*>(O));
            return hipGetLastError();
        });
    });
}

}  // namespace gma
