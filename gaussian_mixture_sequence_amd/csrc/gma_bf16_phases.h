// Phase bodies of the bf16 forward shared by its kernels: the write of one split
// (Gamma_K^T [V | 1], Sec. 3.3 Eq. 5-6 of "Gaussian Mixture Attention") and the softmax
// statistics exchange.  Each body takes its LDS as a byte buffer, so a kernel that runs
// several phases reuses one allocation (the phases' layouts overlap).
#pragma once
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "gma_bf16_common.h"

namespace gma {
namespace bf {

constexpr int gcd_i(int a, int b) { return b == 0 ? a : gcd_i(b, a % b); }

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
//
// LDS of write_body: the arrays below, carved in this order out of one workgroup buffer.
template <int DR, int KT, int VT>
struct WriteLds {
    using S = Split<DR, KT>;
    static constexpr int NT = S::NW * 64, Kp = KT * 32, DV = VT * 32, LDG = Kp + 8, LDV = DV + 8;
    static constexpr int ZSPLIT = S::NW / gcd_i(KT, S::NW);
    static constexpr int BASE = S::TS * S::CS * 32 * 12 + S::ROUND * (LDG + LDV) * 2;
    // x is staged with its square split (XTile), except where one wave reads each token
    // subtile, the split tile would leave room for only one workgroup per CU and the wave's
    // registers have room to split its own fragments: then raw (RawTile, a third of the LDS)
    static constexpr bool RAW = S::CS == 1 && BASE + XTile<DR, S::ROUND, NT>::LDS_BYTES > 80 * 1024 &&
                                BASE + RawTile<DR, S::ROUND, NT>::LDS_BYTES <= 80 * 1024 && DR * VT <= 128;
    using XT = typename std::conditional<RAW, RawTile<DR, S::ROUND, NT>, XTile<DR, S::ROUND, NT>>::type;
    static constexpr int XB = (BASE + 2 * XT::LDS_BYTES <= 80 * 1024) ? 2 : 1;  // keep two workgroups per CU
    using st_t = Stats[S::CS > 1 ? S::TS * S::CS * 32 : 1];  // unused with one component group
    using xt_t = u32x4[XB][XT::LDS_BYTES / 16];
    using gs_t = uint16_t[S::ROUND * LDG];
    using vs_t = uint16_t[S::ROUND * LDV];
    using zr_t = float[KT * ZSPLIT * 32];
    // epilogue (after the last round, from offset 0): the part reduction, then the partial
    static constexpr int VSPLIT = S::NW / gcd_i(KT * VT, S::NW);
    static constexpr size_t RED = VSPLIT > 1 ? size_t(KT) * VT * 1024 : 0, EPI = (RED + size_t(Kp) * (DV + 1)) * 4;
    static constexpr size_t o_st = 0, o_xt = lds_align(o_st + sizeof(st_t)), o_gs = lds_align(o_xt + sizeof(xt_t)),
                            o_vs = lds_align(o_gs + sizeof(gs_t)),
                            o_zr = lds_align(o_vs + sizeof(vs_t)) > EPI ? lds_align(o_vs + sizeof(vs_t)) : lds_align(EPI),
                            bytes = lds_align(o_zr + sizeof(zr_t));
};

// Whether write_body builds its operand planes with the whole workgroup (PlaneBuilder, in its x
// tile buffer) rather than each wave for itself: the same planes a later PlaneBuilder build
// gives, bit for bit.
template <int DR, int KT, int VT>
constexpr bool write_planes_cooperative() {
    using LY = WriteLds<DR, KT, VT>;
    return sizeof(typename LY::xt_t) >= PlaneBuilder<DR, KT * 32, LY::NT>::LDS_BYTES;
}

// Rows [lo, hi) of problem p (head h) into the fp32 partial `mem` ([DV][Kp] Vt^T, then
// [Kp] Z), written with device-coherent stores for a consumer in the same launch.
// BUILD: the operand planes P are built here (overlapping the first loads); otherwise P
// holds them already.  smem: WriteLds<DR, KT, VT>::bytes of LDS.
template <int DR, int KT, int VT, bool BUILD>
__device__ __forceinline__ void write_body(char* __restrict__ smem, const uint16_t* __restrict__ XK,
                                           const uint16_t* __restrict__ V, int64_t N, int64_t p, int h, int64_t lo,
                                           int64_t hi, const Mixture& mx, WaveParams<DR, Split<DR, KT>::CTW>& P,
                                           float* __restrict__ mem) {
    using S = Split<DR, KT>;
    using LY = WriteLds<DR, KT, VT>;
    constexpr int NW = S::NW, NT = NW * 64;
    constexpr int Kp = KT * 32, DV = VT * 32;
    constexpr int LDG = Kp + 8, LDV = DV + 8;
    using XT = typename LY::XT;
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
    constexpr int XB = LY::XB;
    static_assert(ZSPLIT == LY::ZSPLIT, "layout mismatch");
    typename LY::st_t& st = *reinterpret_cast<typename LY::st_t*>(smem + LY::o_st);
    typename LY::xt_t& Xt = *reinterpret_cast<typename LY::xt_t*>(smem + LY::o_xt);
    typename LY::gs_t& Gs = *reinterpret_cast<typename LY::gs_t*>(smem + LY::o_gs);
    typename LY::vs_t& Vs = *reinterpret_cast<typename LY::vs_t*>(smem + LY::o_vs);
    typename LY::zr_t& Zred = *reinterpret_cast<typename LY::zr_t*>(smem + LY::o_zr);

    const int wave = wave_id(), l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const int cs = wave % S::CS, ts = wave / S::CS;
    const int64_t rows = hi - lo;
    const int64_t R = (rows + S::ROUND - 1) / S::ROUND;  // rounds of this split
    auto scores_tile = [&](const u32x4* xtile, f32x16 (&acc)[S::CTW]) __attribute__((always_inline)) {
        if constexpr (!LY::RAW) {
            scores_lds<DR, S::CTW>(P, xtile, ts, acc);
        } else {
            bf16x8 xs[S::KS];
            raw_frags<DR>(xtile, ts, xs);
            scores_x<DR, S::CTW>(P, xs, acc);
        }
    };
    // operand planes built by the whole workgroup in the x tile buffer when it is large
    // enough, else by every wave for itself
    using PB = PlaneBuilder<DR, Kp, NT>;
    constexpr bool COOP = write_planes_cooperative<DR, KT, VT>();
    typename WaveParams<DR, S::CTW>::Raw praw;
    PB pb;
    if constexpr (BUILD) {
        if constexpr (COOP) pb.load(mx, h);
        else P.fetch(mx, h, cs * S::CTW, praw);
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
            scores_tile(Xt[0], acc_a_init);
            __syncthreads();  // x tile 0 consumed by every wave
            xt1.commit(Xt[0]);
            __syncthreads();
        }
    }
    f32x16 acc_a[S::CTW], acc_b[S::CTW];
    if (XB == 2) scores_tile(Xt[0], acc_a);
    else
#pragma unroll
        for (int ct = 0; ct < S::CTW; ++ct) acc_a[ct] = acc_a_init[ct];

    // one pipelined iteration; `cur` holds round r's scores, `nxt` receives round r+1's
    auto iteration = [&](const int64_t r, f32x16 (&cur)[S::CTW], f32x16 (&nxt)[S::CTW]) __attribute__((always_inline)) {
        const int64_t r0 = r * S::ROUND;
        const int xb1 = int((r + 1) % XB);
        // ---- region A (the accumulation first: its transposing LDS reads bound the
        // scheduling region, so everything after them can be interleaved).  The wave runs
        // at raised priority while it feeds the matrix cores, so the other wave on its SIMD
        // fills the VALU around it rather than competing for issue.
        __builtin_amdgcn_s_setprio(1);
        accumulate();
        scores_tile(Xt[xb1], nxt);
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
        __builtin_amdgcn_s_setprio(0);
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
    // split unit are summed through LDS in increasing part order; the partial is assembled
    // in LDS (the round buffers are free) and stored with coalesced device-coherent stores.
    constexpr int E = Kp * (DV + 1), RED = int(LY::RED);
    static_assert(VSPLIT == LY::VSPLIT && LY::EPI <= LY::o_zr, "layout mismatch");
    float* red = reinterpret_cast<float*>(smem);
    float* stg = red + RED;
    __syncthreads();  // every wave is done with the tiles
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
                *reinterpret_cast<float4*>(stg + (vt * 32 + j) * Kp + comp) =
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
        stg[Kp * DV + k] = z;
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(mem, int64_t(E) * 4);
    for (int c = threadIdx.x; c < E / 4; c += NT)
        buf_store16_dev(rm, uint32_t(c * 16), *reinterpret_cast<const u32x4*>(stg + 4 * c));
}

}  // namespace bf
}  // namespace gma
