// Causal GMA of the bf16 path: chunked scan over one segment per workgroup.
//
// Sec. 3.5 of "Gaussian Mixture Attention" defines the prefix memory (Eq. 6b) and the
// output (Eq. 8b); the prefix sums run along the sequence.  A segment starts from the
// memory of all earlier positions (the sum of the earlier segments' aggregates, computed
// by the write kernel) and advances it chunk by chunk.  For a chunk of CH positions with
// responsibilities Gq, Gk (bf16, in LDS) and values Vc:
//   S    = Gq Gk^T, kept for key positions j <= query position i      (Eq. 9b support)
//   num  = S Vc + Gq Vt,   den = S 1 + Gq Z + eps                      (Eq. 8b split at the chunk)
//   Vt  += Gk^T Vc,  Z += Gk^T 1                                       (Eq. 6b advanced by the chunk)
// Only the memory (Vt, Z) chains one chunk to the next, so the chunks are software-
// pipelined.  Iteration c (two barriers):
//   region 1: V tile c+1 into LDS; lower-triangular 32x32 tiles of S^T(c) on MFMA, masked,
//             stored bf16 with fp32 row sums; partial sums of Gq(c) Z(c) on the VALU; MFMAs
//             of chunk c+2's scores; (several waves per token) local softmax statistics of
//             chunk c+1                                                     -> B_Q
//   region 2: local softmax of chunk c+1 (one wave per token), its Gq, Gk into the other
//             LDS buffer; O(c): each wave owns 16-wide value columns, intra part V^T S^T and
//             inter part Vt^T Gq^T (Vt split hi + lo), divided and stored; memory update
//             Vt += Gk^T Vc (fp32 registers held across chunks), Z += Gk^T 1 on MFMA with a
//             ones operand; x tiles of chunk c+3 into LDS                    -> B_P
// x tiles are fetched with coalesced loads and staged through LDS: split once and shared
// when several waves hold the components of a token, unsplit when one wave does.
// 16x16x32 MFMA layouts (lane l, g = l / 16): A row i = l % 16, k = 8 g + v; B col j =
// l % 16, k = 8 g + v; D row i = 4 g + r, col j = l % 16.
#include <cstdint>
#include <type_traits>

#include "gma_bf16_common.h"
#include "gma_bf16_phases.h"
#include "gma_internal.h"

namespace gma {
namespace bf {

template <int DR, int KT, int CH>
constexpr int scan_jpw() {  // 32-position score jobs per wave and chunk (query and key)
    return (2 * (CH / 32) + Split<DR, KT>::TS - 1) / Split<DR, KT>::TS;
}

// LDS bytes of scan_body for a chunk of CH positions (the ScanLds arrays, unaligned).
template <int DR, int KT, int VT, int CH>
constexpr int scan_lds_bytes() {
    using S = Split<DR, KT>;
    constexpr int Kp = KT * 32, DV = VT * 32, SUB = CH / 32;
    constexpr int xt = S::CS > 1 ? 2 * XTile<DR, CH, S::NW * 64>::LDS_BYTES : 2 * RawTile<DR, CH, S::NW * 64>::LDS_BYTES;
    return scan_jpw<DR, KT, CH>() * S::TS * S::CS * 32 * 12 + 4 * CH * (Kp + 8) * 2 + 2 * CH * (DV + 8) * 2 +
           CH * (CH + 8) * 2 + xt + (S::NW * 64 / CH) * CH * 4 + SUB * CH * 4 + Kp * 4;
}

// The chunk actually used: the requested one, halved while its tiles exceed the 160 KiB of
// LDS or the two chunks of scores the pipeline holds would exceed two 32x32 tiles per wave
// (the chunk length only changes the order of the sums).
template <int DR, int KT, int VT, int CH_REQ>
constexpr int scan_chunk() {
    return (CH_REQ > 32 && (scan_lds_bytes<DR, KT, VT, CH_REQ>() > 160 * 1024 ||
                            scan_jpw<DR, KT, CH_REQ>() * Split<DR, KT>::CTW > 2))
               ? CH_REQ / 2
               : CH_REQ;
}

// LDS of scan_body, carved in this order out of one workgroup buffer.
template <int DR, int KT, int VT, int CH>
struct ScanLds {
    using S = Split<DR, KT>;
    static constexpr int NT = S::NW * 64, Kp = KT * 32, DV = VT * 32, LDG = Kp + 8, LDV = DV + 8, LDSS = CH + 8;
    static constexpr int SUB = CH / 32, JPW = scan_jpw<DR, KT, CH>(), NPARTS = NT / CH;
    using XT = typename std::conditional<(S::CS > 1), XTile<DR, CH, NT>, RawTile<DR, CH, NT>>::type;
    using st_t = ScanStats[JPW][S::TS * S::CS * 32];
    using g_t = uint16_t[2][CH * LDG];
    using v_t = uint16_t[2][CH * LDV];
    using s_t = uint16_t[CH * LDSS];
    using x_t = u32x4[XT::LDS_BYTES / 16];
    using di_t = float[NPARTS][CH];
    using dp_t = float[SUB][CH];
    using z_t = float[Kp];
    static constexpr size_t o_st = 0, o_gq = lds_align(o_st + sizeof(st_t)), o_gk = lds_align(o_gq + sizeof(g_t)),
                            o_vs = lds_align(o_gk + sizeof(g_t)), o_ss = lds_align(o_vs + sizeof(v_t)),
                            o_xq = lds_align(o_ss + sizeof(s_t)), o_xk = lds_align(o_xq + sizeof(x_t)),
                            o_di = lds_align(o_xk + sizeof(x_t)), o_dp = lds_align(o_di + sizeof(di_t)),
                            o_zs = lds_align(o_dp + sizeof(dp_t)), bytes = lds_align(o_zs + sizeof(z_t));
};

// Positions [lo, hi) (segment seg_idx) of problem p (head h).  The segment starts from the
// sum of the aggregates 0 .. seg_idx-1 in `agg` (the problem's aggregates, E floats each,
// read device-coherent); wait() runs once the first tiles are in flight and before they
// are read.  BUILD as in write_body.  smem: ScanLds<DR, KT, VT, CH>::bytes of LDS.
template <int DR, int KT, int VT, int CH_REQ, bool BUILD, typename WaitF>
__device__ __forceinline__ void scan_body(char* __restrict__ smem, const uint16_t* __restrict__ XQ,
                                          const uint16_t* __restrict__ XK, const uint16_t* __restrict__ V, int64_t N,
                                          int64_t p, int h, int seg_idx, int64_t lo, int64_t hi, const Mixture& mx,
                                          WaveParams<DR, Split<DR, KT>::CTW>& P, const float* __restrict__ agg,
                                          float eps, uint16_t* __restrict__ O, WaitF&& wait,
                                          const float* __restrict__ state_in, float* __restrict__ state_out) {
    constexpr int CH = scan_chunk<DR, KT, VT, CH_REQ>();
    using LY = ScanLds<DR, KT, VT, CH>;
    using S = Split<DR, KT>;
    constexpr int NW = S::NW, NT = NW * 64;
    constexpr int Kp = KT * 32, DV = VT * 32;
    constexpr int CS = S::CS, TS = S::TS, CTW = S::CTW, KS = S::KS;
    constexpr int LDG = Kp + 8, LDV = DV + 8, LDSS = CH + 8;
    constexpr int SUB = CH / 32;                  // 32-position subtiles per chunk
    constexpr int JOBS = 2 * SUB;                 // query subtiles, then key subtiles
    constexpr int JPW = scan_jpw<DR, KT, CH>();   // jobs per wave
    constexpr int C16 = DV / 16;                  // 16-wide value column tiles
    constexpr int CPW = (C16 + NW - 1) / NW;      // column tiles per wave
    constexpr int KT16 = Kp / 16;                 // 16-row component tiles of the memory
    constexpr int ZPW = (KT16 + NW - 1) / NW;     // Z tiles per wave
    constexpr int STILES = SUB * (SUB + 1) / 2;   // lower-triangular tiles of S^T
    constexpr int VCHUNKS = CH * DV / 8, VCH = (VCHUNKS + NT - 1) / NT;
    constexpr bool VEVEN = VCHUNKS % NT == 0;
    constexpr int NPARTS = NW * 64 / CH, KPP = Kp / NPARTS;  // split of the Gq Z sums
    static_assert(KPP % 4 == 0, "Gq Z partial sums read 4 components at a time");
    // x tiles through LDS (coalesced loads): split once and shared when several waves use the
    // same token subtile (CS > 1); otherwise staged unsplit, each wave splitting its own
    constexpr bool SHARE_X = CS > 1;
    using XT = typename std::conditional<SHARE_X, XTile<DR, CH, NT>, RawTile<DR, CH, NT>>::type;

    static_assert(std::is_same<XT, typename LY::XT>::value && NPARTS == LY::NPARTS && JPW == LY::JPW, "layout mismatch");
    typename LY::st_t& st = *reinterpret_cast<typename LY::st_t*>(smem + LY::o_st);
    typename LY::g_t& Gq = *reinterpret_cast<typename LY::g_t*>(smem + LY::o_gq);
    typename LY::g_t& Gk = *reinterpret_cast<typename LY::g_t*>(smem + LY::o_gk);
    typename LY::v_t& Vs = *reinterpret_cast<typename LY::v_t*>(smem + LY::o_vs);
    typename LY::s_t& Ss = *reinterpret_cast<typename LY::s_t*>(smem + LY::o_ss);
    typename LY::x_t& XtQ = *reinterpret_cast<typename LY::x_t*>(smem + LY::o_xq);
    typename LY::x_t& XtK = *reinterpret_cast<typename LY::x_t*>(smem + LY::o_xk);
    typename LY::di_t& den_ip = *reinterpret_cast<typename LY::di_t*>(smem + LY::o_di);
    typename LY::dp_t& den_part = *reinterpret_cast<typename LY::dp_t*>(smem + LY::o_dp);
    typename LY::z_t& Zs = *reinterpret_cast<typename LY::z_t*>(smem + LY::o_zs);

    const int wave = wave_id(), l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const int g4 = l >> 4, i16 = l & 15;
    const int cs = wave % CS, ts = wave / CS;
    const int64_t rows = hi - lo;
    const int64_t C = (rows + CH - 1) / CH;  // chunks of this segment

    // operand planes built by the whole workgroup in the V tile buffers when they are large
    // enough, else by every wave for itself
    using PB = PlaneBuilder<DR, Kp, NT>;
    constexpr bool COOP = sizeof(Vs) >= PB::LDS_BYTES;
    typename WaveParams<DR, CTW>::Raw praw;
    PB pb;
    if constexpr (BUILD) {
        if constexpr (COOP) pb.load(mx, h);
        else P.fetch(mx, h, cs * CTW, praw);
    }
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(XQ + (size_t(p) * N + lo) * DR, rows * DR * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(XK + (size_t(p) * N + lo) * DR, rows * DR * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + (size_t(p) * N + lo) * DV, rows * DV * 2);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + (size_t(p) * N + lo) * DV, rows * DV * 2);

    // ---- inputs: V tile c+1 in registers while tile c is in LDS; x fragments of chunk
    // c+2 in registers (or, shared, x tile c+2 in LDS and c+3 in registers)
    u32x4 vr[VCH];
    auto load_v = [&](int64_t row0) {
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = threadIdx.x + u * NT;
            vr[u] = (VEVEN || c < VCHUNKS) ? buf_load16(rv, uint32_t((row0 * DV + int64_t(c) * 8) * 2))
                                           : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto commit_v = [&](uint16_t* dst) {
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = threadIdx.x + u * NT;
            if (VEVEN || c < VCHUNKS) {
                const int row = c / (DV / 8), col = (c - row * (DV / 8)) * 8;
                *reinterpret_cast<u32x4*>(dst + row * LDV + col) = vr[u];
            }
        }
    };
    auto job_of = [&](int jj, bool& is_q, int& sub) {  // this wave's jj-th job; false if none
        const int job = ts + jj * TS;
        is_q = job < SUB;
        sub = is_q ? job : job - SUB;
        if (job >= JOBS) sub = 0;
        return job < JOBS;
    };
    XT xq, xk;  // registers: the x tiles of the chunk after the one in LDS
    auto scores_chunk = [&](f32x16 (&acc)[JPW][CTW]) __attribute__((always_inline)) {  // from the LDS tiles
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
            bool is_q;
            int sub;
            job_of(jj, is_q, sub);
            if constexpr (SHARE_X) {
                scores_lds<DR, CTW>(P, is_q ? XtQ : XtK, sub, acc[jj]);
            } else {
                bf16x8 xs[KS];
                raw_frags<DR>(is_q ? XtQ : XtK, sub, xs);
                scores_x<DR, CTW>(P, xs, acc[jj]);
            }
        }
    };
    float zdummy[CTW][16];
    float sm_m[JPW], sm_L[JPW];
    auto softmax_local = [&](f32x16 (&acc)[JPW][CTW]) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
            float D;
            local_softmax<CTW, false>(acc[jj], zdummy, sm_m[jj], sm_L[jj], D);
            if (CS > 1) st[jj][(ts * CS + cs) * 32 + j] = ScanStats{sm_m[jj], sm_L[jj], 0.0f};  // both halves equal
        }
    };
    // Gamma of the chunk starting at row0 into Gq[b], Gk[b] (after softmax_local)
    auto store_gamma = [&](f32x16 (&acc)[JPW][CTW], int64_t row0, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
            bool is_q;
            int sub;
            if (!job_of(jj, is_q, sub)) continue;
            float scale;
            if (CS == 1) {
                scale = __builtin_amdgcn_rcpf(sm_L[jj]);
            } else {
                float mm = -INFINITY;
#pragma unroll
                for (int c = 0; c < CS; ++c) mm = fmaxf(mm, st[jj][(ts * CS + c) * 32 + j].m);
                float Lt = 0.0f;
#pragma unroll
                for (int c = 0; c < CS; ++c) {
                    const ScanStats sc = st[jj][(ts * CS + c) * 32 + j];
                    Lt = fmaf(sc.L, __builtin_amdgcn_exp2f(sc.m - mm), Lt);
                }
                scale = __builtin_amdgcn_exp2f(sm_m[jj] - mm) * __builtin_amdgcn_rcpf(Lt);
            }
            if (int64_t(sub) * 32 + j >= rows - row0) scale = 0.0f;  // positions past the segment
            store_gamma_lds<CTW>(acc[jj], scale, is_q ? Gq[b] : Gk[b], LDG, sub * 32 + j, cs * CTW);
        }
    };

    // ---- starting memory of the segment: the sum of the aggregates of segments
    // 0 .. seg_idx-1 (each stored as VtT [DV][Kp] then Z [Kp]), in increasing segment order
    const size_t E = size_t(Kp) * (DV + 1);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(agg, int64_t(seg_idx) * int64_t(E) * 4);
    f32x4 mem[CPW][KT16];
    init_memory<CPW, KT16, NW, DV, 4>(mem, Zs, Kp, NT, state_in, mx.K);

    // prologue loads first, so they overlap the operand build and the prefix sum
    load_v(0);
    xq.load(rq, 0);
    xk.load(rk, 0);
    if constexpr (BUILD && COOP) {
        pb.build(reinterpret_cast<char*>(&Vs[0][0]), mx.K);
        __syncthreads();
        P.template read_planes<Kp>(reinterpret_cast<const char*>(&Vs[0][0]), cs * CTW);
        __syncthreads();  // staging area free for the V tiles
    } else if constexpr (BUILD) {
        P.build(praw, mx.K, cs * CTW);
    }
    wait();
#pragma unroll 2
    for (int gs = 0; gs < seg_idx; ++gs) {
        const uint32_t a = uint32_t(size_t(gs) * E * 4);
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
            const int c16 = wave + cc * NW;
            if (c16 < C16) {
#pragma unroll
                for (int kt = 0; kt < KT16; ++kt) {
                    const u32x4 v = buf_load16_dev(ra, a + uint32_t(((c16 * 16 + i16) * Kp + kt * 16 + 4 * g4) * 4));
#pragma unroll
                    for (int r = 0; r < 4; ++r) mem[cc][kt][r] += __uint_as_float(v[r]);
                }
            }
        }
        for (int k = threadIdx.x * 4; k < Kp; k += NT * 4) {
            const u32x4 v = buf_load16_dev(ra, a + uint32_t((Kp * DV + k) * 4));
#pragma unroll
            for (int r = 0; r < 4; ++r) Zs[k + r] += __uint_as_float(v[r]);
        }
    }
    commit_v(Vs[0]);
    load_v(CH);

    // ---- prologue: Gamma of chunk 0 into Gq[0], Gk[0]; scores of chunk 1 held; x of
    // chunks 2 (and 3) staged
    f32x16 acc_a[JPW][CTW], acc_b[JPW][CTW];
    xq.commit(XtQ);
    xk.commit(XtK);
    xq.load(rq, CH);
    xk.load(rk, CH);
    __syncthreads();
    scores_chunk(acc_b);  // chunk 0
    softmax_local(acc_b);
    __syncthreads();      // statistics published; x tile 0 consumed
    store_gamma(acc_b, 0, 0);
    xq.commit(XtQ);
    xk.commit(XtK);
    xq.load(rq, 2 * CH);
    xk.load(rk, 2 * CH);
    __syncthreads();
    scores_chunk(acc_a);  // chunk 1
    __syncthreads();      // x tile 1 consumed
    xq.commit(XtQ);
    xk.commit(XtK);
    xq.load(rq, 3 * CH);
    xk.load(rk, 3 * CH);
    __syncthreads();

    // ---- one pipelined chunk: `cur` holds chunk c+1's scores, `nxt` receives chunk c+2's
    // (x tiles of chunk c+2 in LDS, c+3 in registers); b = c % 2 selects the LDS buffers
    auto chunk = [&](const int64_t c, const int b, f32x16 (&cur)[JPW][CTW], f32x16 (&nxt)[JPW][CTW])
                     __attribute__((always_inline)) {
        const int64_t nc = c * CH;
        // ---- region 1 (raised priority while the wave feeds the matrix cores: the other
        // wave on its SIMD fills the VALU around it)
        __builtin_amdgcn_s_setprio(1);
        commit_v(Vs[b ^ 1]);  // V tile c+1
        load_v(nc + 2 * CH);
        if (wave < STILES) {  // S^T tile (rows = key positions, cols = query positions)
            int qt = 0, kt = wave;
            while (kt > qt) { kt -= qt + 1; ++qt; }
            f32x16 sacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < Kp / 16; ++ks)
                sacc = mfma(read_rowfrag(Gk[b], LDG, kt * 32 + j, 16 * ks), read_rowfrag(Gq[b], LDG, qt * 32 + j, 16 * ks),
                            sacc);
            float rs = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = kt * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (kk > qt * 32 + j) sacc[r] = 0.0f;  // j > i is outside the causal support
                rs += sacc[r];
            }
            rs = xsum32(rs);
            if (lh == 0) den_part[kt][qt * 32 + j] = rs;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x2 v;
                v[0] = pack_bf16x2(sacc[4 * q + 0], sacc[4 * q + 1]);
                v[1] = pack_bf16x2(sacc[4 * q + 2], sacc[4 * q + 3]);
                *reinterpret_cast<u32x2*>(Ss + (qt * 32 + j) * LDSS + kt * 32 + 8 * q + 4 * lh) = v;
            }
        }
        {  // partial sums of Gq(c) Z(c): part `pt` covers components pt*KPP .. +KPP-1
            const int t = l % CH, pt = wave * (64 / CH) + l / CH;
            float d = 0.0f;
#pragma unroll
            for (int k4 = 0; k4 < KPP / 4; ++k4) {
                const int k = pt * KPP + 4 * k4;
                const u32x2 gv = *reinterpret_cast<const u32x2*>(Gq[b] + t * LDG + k);
                const float4 zv = *reinterpret_cast<const float4*>(Zs + k);
                d = fmaf(__uint_as_float(gv[0] << 16), zv.x, d);
                d = fmaf(__uint_as_float(gv[0] & 0xffff0000u), zv.y, d);
                d = fmaf(__uint_as_float(gv[1] << 16), zv.z, d);
                d = fmaf(__uint_as_float(gv[1] & 0xffff0000u), zv.w, d);
            }
            den_ip[pt][t] = d;
        }
        scores_chunk(nxt);  // chunk c+2
        if (CS > 1) softmax_local(cur);
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();  // B_Q: S(c), row sums, Gq Z partials, statistics of c+1 published
        // ---- region 2
        if (CS == 1) softmax_local(cur);
        store_gamma(cur, nc + CH, b ^ 1);  // chunk c+1
        __builtin_amdgcn_s_setprio(1);
        const uint16_t* Vc = Vs[b];
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
            const int c16 = wave + cc * NW;
            if (c16 >= C16) continue;
            f32x4 o[CH / 16];
#pragma unroll
            for (int t16 = 0; t16 < CH / 16; ++t16) {
                o[t16] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                // intra-chunk part: V^T S^T over key positions up to this query tile
#pragma unroll
                for (int ks = 0; ks < (t16 * 16 + 16 + 31) / 32; ++ks) {
                    bf16x8 a = read_colfrag16(Vc, LDV, 32 * ks, c16 * 16);
                    bf16x8 bb = *reinterpret_cast<const bf16x8*>(Ss + (t16 * 16 + i16) * LDSS + 32 * ks + 8 * g4);
                    o[t16] = mfma16(a, bb, o[t16]);
                }
            }
            // inter-chunk part: memory^T Gq^T, memory split into hi + lo bf16 once per k-step
#pragma unroll
            for (int m2 = 0; m2 < Kp / 32; ++m2) {
                u32x4 ah, al;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int v0 = 2 * q, v1 = 2 * q + 1;
                    const float x0 = mem[cc][2 * m2 + (v0 >> 2)][v0 & 3];
                    const float x1 = mem[cc][2 * m2 + (v1 >> 2)][v1 & 3];
                    const uint32_t hb = pack_bf16x2(x0, x1);
                    ah[q] = hb;
                    al[q] = pack_bf16x2(x0 - __uint_as_float(hb << 16), x1 - __uint_as_float(hb & 0xffff0000u));
                }
#pragma unroll
                for (int t16 = 0; t16 < CH / 16; ++t16) {
                    const int qrow = t16 * 16 + i16;
                    const u32x2 b0 = *reinterpret_cast<const u32x2*>(Gq[b] + qrow * LDG + 32 * m2 + 4 * g4);
                    const u32x2 b1 = *reinterpret_cast<const u32x2*>(Gq[b] + qrow * LDG + 32 * m2 + 16 + 4 * g4);
                    const bf16x8 bb = __builtin_bit_cast(bf16x8, u32x4{b0[0], b0[1], b1[0], b1[1]});
                    o[t16] = mfma16(__builtin_bit_cast(bf16x8, ah), bb, o[t16]);
                    o[t16] = mfma16(__builtin_bit_cast(bf16x8, al), bb, o[t16]);
                }
            }
#pragma unroll
            for (int t16 = 0; t16 < CH / 16; ++t16) {
                const int qrow = t16 * 16 + i16;
                float den = eps;
#pragma unroll
                for (int pt = 0; pt < NPARTS; ++pt) den += den_ip[pt][qrow];
#pragma unroll
                for (int kt = 0; kt < SUB; ++kt)
                    if (kt * 32 <= qrow) den += den_part[kt][qrow];
                const float rden = __builtin_amdgcn_rcpf(den);
                u32x2 v;
                v[0] = pack_bf16x2(o[t16][0] * rden, o[t16][1] * rden);
                v[1] = pack_bf16x2(o[t16][2] * rden, o[t16][3] * rden);
                // rows past the segment fall outside the resource and are dropped
                buf_store8(ro, uint32_t(((nc + qrow) * DV + c16 * 16 + 4 * g4) * 2), v);
            }
        }
        // memory update: Vt += Gk^T Vc (every wave its value columns), Z += Gk^T 1 (the
        // component tiles kt = wave (mod NW), ones operand)
        const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
        f32x4 zt[ZPW];
#pragma unroll
        for (int zi = 0; zi < ZPW; ++zi) zt[zi] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt)
#pragma unroll
            for (int ks = 0; ks < CH / 32; ++ks) {
                const bf16x8 a = read_colfrag16(Gk[b], LDG, 32 * ks, kt * 16);
#pragma unroll
                for (int cc = 0; cc < CPW; ++cc) {
                    const int c16 = wave + cc * NW;
                    if (c16 < C16) mem[cc][kt] = mfma16(a, read_colfrag16(Vc, LDV, 32 * ks, c16 * 16), mem[cc][kt]);
                }
                if (kt % NW == wave) zt[kt / NW] = mfma16(a, ones, zt[kt / NW]);
            }
        if (i16 == 0)
#pragma unroll
            for (int zi = 0; zi < ZPW; ++zi) {
                const int kt = wave + zi * NW;
                if (kt < KT16)
#pragma unroll
                    for (int r = 0; r < 4; ++r) Zs[kt * 16 + 4 * g4 + r] += zt[zi][r];
            }
        // x tiles of chunk c+3 (chunk c+2's were read in region 1); loads of c+4 issued
        xq.commit(XtQ);
        xk.commit(XtK);
        xq.load(rq, nc + 4 * CH);
        xk.load(rk, nc + 4 * CH);
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();  // B_P: Gamma(c+1), V(c+1), Z(c+1) visible; chunk c consumed
    };
    // chunks in pairs (static buffer roles), then the odd one
    int64_t c = 0;
    for (; c + 1 < C; c += 2) {
        chunk(c, 0, acc_a, acc_b);
        chunk(c + 1, 1, acc_b, acc_a);
    }
    if (c < C) chunk(c, 0, acc_a, acc_b);
    if (state_out) store_memory<CPW, KT16, NW, DV>(mem, Zs, state_out, mx.K);  // after B_P of the last chunk
}

// ---- the causal forward in one launch (shapes of the pipelined scan).  Grid (G, P);
// workgroup (s, p) owns segment s of problem p.  Segments 0 .. G-2 first write their
// aggregate (write_body over the segment) and publish it; every segment then waits for the
// aggregates of the segments before it (only lower-numbered workgroups, dispatched no later
// than itself, so the launch needs no co-residency), sums them in increasing order and
// scans.  The last segment's aggregate is never needed, so its workgroup builds its operand
// planes and goes straight to the wait.  flags: [P][G] words compared with `token`.  With
// `aggregated` set, the aggregates are already in place (written by an earlier launch,
// write_kernel): no segment writes one and nothing waits.  A workgroup whose wait times out
// writes NaN over its positions (and over state_out if it is the last segment) and raises
// kDevErrTimeout in `err`.
template <int DR, int KT, int VT, int CH_REQ>
constexpr size_t causal_lds_bytes() {
    constexpr size_t w = WriteLds<DR, KT, VT>::bytes;
    constexpr size_t sc = ScanLds<DR, KT, VT, scan_chunk<DR, KT, VT, CH_REQ>()>::bytes;
    return w > sc ? w : sc;
}

template <int DR, int KT, int VT, int CH_REQ>
__global__ void __launch_bounds__((Split<DR, KT>::NW * 64))
__attribute__((amdgpu_waves_per_eu(waves_for_lds(causal_lds_bytes<DR, KT, VT, CH_REQ>()))))
    causal_kernel(const uint16_t* __restrict__ XQ, const uint16_t* __restrict__ XK, const uint16_t* __restrict__ V,
                  int64_t N, int H, int64_t seg, int G, Mixture mx, float* __restrict__ aggregates,
                  uint64_t* __restrict__ flags, uint64_t token, uint32_t wait_limit, int aggregated, float eps,
                  uint16_t* __restrict__ O, const float* __restrict__ state_in, float* __restrict__ state_out,
                  uint32_t* __restrict__ err) {
    __shared__ __attribute__((aligned(16))) char smem[causal_lds_bytes<DR, KT, VT, CH_REQ>()];
    using S = Split<DR, KT>;
    constexpr int Kp = KT * 32, DV = VT * 32, E = Kp * (DV + 1), NT = S::NW * 64;
    const int64_t p = blockIdx.y;
    const int s = blockIdx.x, h = int(p % H);
    const int64_t lo = int64_t(s) * seg, hi = min<int64_t>(lo + seg, N);
    float* agg = aggregates + size_t(p) * G * E;
    uint64_t* fl = flags + size_t(p) * G;
    WaveParams<DR, S::CTW> P;
    const bool aggregate = s + 1 < G && !aggregated;
    if (aggregate) {
        write_body<DR, KT, VT, true>(smem, XK, V, N, p, h, lo, hi, mx, P, agg + size_t(s) * E);
        publish_token(fl + s, token);  // its barrier also frees the write phase's LDS
    }
    // the scan's planes are the same bits in every workgroup and either launch mode, so the
    // outputs do not depend on the launch mode: the write phase's when it built them with the
    // whole workgroup, else built here (uniform over the workgroup)
    if (!(aggregate && write_planes_cooperative<DR, KT, VT>())) {
        if constexpr (PlaneBuilder<DR, Kp, NT>::LDS_BYTES <= sizeof(smem)) {  // the whole buffer is free here
            PlaneBuilder<DR, Kp, NT> pb;
            pb.load(mx, h);
            pb.build(smem, mx.K);
            __syncthreads();
            P.template read_planes<Kp>(smem, (wave_id() % S::CS) * S::CTW);
            __syncthreads();
        } else {
            P.compute(mx, h, (wave_id() % S::CS) * S::CTW);
        }
    }
    bool ok = true;
    const size_t SE = size_t(mx.K) * (DV + 1);  // one problem's carried memory
    float* so = (state_out && s == G - 1) ? state_out + p * SE : nullptr;
    scan_body<DR, KT, VT, CH_REQ, false>(smem, XQ, XK, V, N, p, h, s, lo, hi, mx, P, agg, eps, O,
                                         [&] {
                                             if (!aggregated) ok = wait_tokens(fl, s, token, wait_limit);
                                         },
                                         state_in ? state_in + p * SE : nullptr, so);
    // waves poll on their own: agree on the outcome before acting on it
    ok = workgroup_all(ok, reinterpret_cast<int*>(smem));
    if (!ok) {  // the starting memory was never complete: make that visible in the outputs and to the host
        __builtin_amdgcn_s_waitcnt(0);  // the phase's own stores of these rows land first
        __syncthreads();
        uint16_t* op = O + (size_t(p) * N + lo) * DV;
        for (int64_t e = threadIdx.x; e < (hi - lo) * DV; e += NT) op[e] = 0x7fc0u;
        if (so)
            for (size_t e = threadIdx.x; e < SE; e += NT) so[e] = __builtin_nanf("");
        if (threadIdx.x == 0) atomicOr(err, kDevErrTimeout);
    }
}

// ---- serial variant: one chunk after another (four barriers per chunk), for the shapes
// whose fp32 memory plus two chunks of scores would not fit the registers of the
// pipelined kernel (many component tiles).
// LDS bytes of serial_scan_kernel for a chunk of CH positions (mirrors the declarations below).
template <int DR, int KT, int VT, int CH>
constexpr int serial_scan_lds_bytes() {
    using S = Split<DR, KT>;
    constexpr int Kp = KT * 32, DV = VT * 32, SUB = CH / 32;
    constexpr int JPW = (2 * SUB + S::TS - 1) / S::TS;
    constexpr int xt = S::CS > 1 ? 2 * XTile<DR, CH, S::NW * 64>::LDS_BYTES : 32;
    return JPW * S::TS * S::CS * 32 * 12 + 2 * CH * (Kp + 8) * 2 + 2 * CH * (DV + 8) * 2 + CH * (CH + 8) * 2 + xt +
           CH * 4 + SUB * CH * 4 + Kp * 4;
}

// The chunk actually used: the requested one, halved while its tiles exceed the 160 KiB of
// LDS (the chunk length only changes the order of the sums).
template <int DR, int KT, int VT, int CH_REQ>
constexpr int serial_scan_chunk() {
    return (CH_REQ > 32 && serial_scan_lds_bytes<DR, KT, VT, CH_REQ>() > 160 * 1024) ? CH_REQ / 2 : CH_REQ;
}

template <int DR, int KT, int VT, int CH_REQ>
__global__ void __launch_bounds__((Split<DR, KT>::NW * 64))
    serial_scan_kernel(const uint16_t* __restrict__ XQ, const uint16_t* __restrict__ XK, const uint16_t* __restrict__ V,
                int64_t N, int H, int64_t seg, int G, Mixture mx,
                const float* __restrict__ prefix, float eps, uint16_t* __restrict__ O,
                const float* __restrict__ state_in, float* __restrict__ state_out) {
    constexpr int CH = serial_scan_chunk<DR, KT, VT, CH_REQ>();
    using S = Split<DR, KT>;
    constexpr int NT = S::NW * 64;
    constexpr int Kp = KT * 32, DV = VT * 32;
    constexpr int NW = S::NW, CS = S::CS, TS = S::TS, CTW = S::CTW, KS = S::KS;
    constexpr int LDG = Kp + 8, LDV = DV + 8, LDSS = CH + 8;
    constexpr int SUB = CH / 32;                  // 32-token subtiles per chunk
    constexpr int JOBS = 2 * SUB;                 // query subtiles, then key subtiles
    constexpr int JPW = (JOBS + TS - 1) / TS;     // jobs per token slot
    constexpr int JG = (CS >= 8) ? 1 : JPW;       // jobs whose scores are held at once
    constexpr int C16 = DV / 16;                  // 16-wide value column tiles
    constexpr int CPW = (C16 + NW - 1) / NW;      // column tiles per wave
    constexpr int KT16 = Kp / 16;                 // 16-row component tiles of the memory
    constexpr int STILES = SUB * (SUB + 1) / 2;   // lower-triangular tiles of S^T
    constexpr int VCH = (CH * DV / 8 + NT - 1) / NT;
    // x tiles: split once and shared through LDS when several waves use the same token
    // subtile (CS > 1); otherwise every wave prefetches its own fragments into registers
    constexpr bool SHARE_X = CS > 1;
    using XT = XTile<DR, CH, NT>;

    __shared__ ScanStats st[JPW][TS * CS * 32];
    __shared__ __attribute__((aligned(16))) uint16_t Gq[CH * LDG];
    __shared__ __attribute__((aligned(16))) uint16_t Gk[CH * LDG];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][CH * LDV];
    __shared__ __attribute__((aligned(16))) uint16_t Ss[CH * LDSS];
    __shared__ __attribute__((aligned(16))) u32x4 XtQ[SHARE_X ? XT::LDS_BYTES / 16 : 1];
    __shared__ __attribute__((aligned(16))) u32x4 XtK[SHARE_X ? XT::LDS_BYTES / 16 : 1];
    __shared__ float den_inter[CH];
    __shared__ float den_part[SUB][CH];
    __shared__ float Zs[Kp];

    const int wave = wave_id(), l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const int g4 = l >> 4, i16 = l & 15;
    const int cs = wave % CS, ts = wave / CS;
    const int64_t p = blockIdx.y;
    const int seg_idx = blockIdx.x;
    const int h = int(p % H);
    const int64_t lo = int64_t(seg_idx) * seg, hi = min<int64_t>(lo + seg, N);
    const int64_t rows = hi - lo;

    WaveParams<DR, CTW> P;
    P.compute(mx, h, cs * CTW);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(XQ + (size_t(p) * N + lo) * DR, rows * DR * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(XK + (size_t(p) * N + lo) * DR, rows * DR * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + (size_t(p) * N + lo) * DV, rows * DV * 2);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + (size_t(p) * N + lo) * DV, rows * DV * 2);

    // ---- input pipeline: chunk c is consumed while chunk c+1 sits in LDS / registers and
    // chunk c+2 is in flight
    u32x4 vr[VCH];
    auto load_v = [&](int64_t row0) {
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = threadIdx.x + u * NT;
            vr[u] = (c < CH * DV / 8) ? buf_load16(rv, uint32_t((row0 * DV + int64_t(c) * 8) * 2))
                                      : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto commit_v = [&](uint16_t* dst) {
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = threadIdx.x + u * NT;
            if (c < CH * DV / 8) {
                const int row = c / (DV / 8), col = (c - row * (DV / 8)) * 8;
                *reinterpret_cast<u32x4*>(dst + row * LDV + col) = vr[u];
            }
        }
    };
    XT xq, xk;                      // SHARE_X: whole-tile chunks of the next chunk
    bf16x8 xf[JPW][KS], xn[JPW][KS];  // !SHARE_X: this wave's fragments, this and next chunk
    auto load_frags = [&](int64_t row0, bf16x8 (&dst)[JPW][KS]) {
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
            const int job = ts + jj * TS;
            const bool is_q = job < SUB;
            const int sub = is_q ? job : job - SUB;
            load_x_buf<DR>(is_q ? rq : rk, (job < JOBS) ? row0 + sub * 32 : int64_t(1) << 40, dst[jj]);
        }
    };

    // starting memory of the segment: the sum of the aggregates of segments 0 .. seg_idx-1
    // (each stored as VtT [DV][Kp] then Z [Kp]), added in increasing segment order
    const size_t E = size_t(Kp) * (DV + 1);
    const float* agg = prefix + size_t(p) * G * E;
    const size_t SE = size_t(mx.K) * (DV + 1);  // one problem's carried memory
    f32x4 mem[CPW][KT16];
    init_memory<CPW, KT16, NW, DV, 1>(mem, Zs, Kp, NT, state_in ? state_in + p * SE : nullptr, mx.K);

    // prologue loads are issued before the prefix sum so they overlap it
    load_v(0);
    if (SHARE_X) {
        xq.load(rq, 0);
        xk.load(rk, 0);
    } else {
        load_frags(0, xf);
    }
    for (int gs = 0; gs < seg_idx; ++gs) {
        const float* a = agg + size_t(gs) * E;
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
            const int c16 = wave + cc * NW;
            if (c16 < C16) {
#pragma unroll
                for (int kt = 0; kt < KT16; ++kt) {
                    const float4 v = *reinterpret_cast<const float4*>(a + size_t(c16 * 16 + i16) * Kp + kt * 16 + 4 * g4);
                    mem[cc][kt][0] += v.x;
                    mem[cc][kt][1] += v.y;
                    mem[cc][kt][2] += v.z;
                    mem[cc][kt][3] += v.w;
                }
            }
        }
        for (int k = threadIdx.x; k < Kp; k += NT) Zs[k] += a[size_t(Kp) * DV + k];
    }
    commit_v(Vs[0]);
    load_v(CH);
    if (SHARE_X) {
        xq.commit(XtQ);
        xk.commit(XtK);
        xq.load(rq, CH);
        xk.load(rk, CH);
    } else {
        load_frags(CH, xn);
    }

    // One chunk.  `xc` holds this chunk's x fragments (!SHARE_X) and is refilled with the
    // chunk after next once the scores are taken; the loop below alternates the two
    // fragment buffers and the two V buffers statically, so no register copy (and no
    // wait on loads still in flight) sits on the loop back-edge.
    auto chunk = [&](const int64_t nc, const int vb, bf16x8 (&xc)[JPW][KS]) __attribute__((always_inline)) {
        __syncthreads();  // B0: previous chunk consumed; this chunk's inputs and Zs visible
        // ---- phase L: scores and softmax of the chunk's query and key rows
        float zr[CTW][16];
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 z4 = *reinterpret_cast<const float4*>(Zs + (cs * CTW + ct) * 32 + 8 * q + 4 * lh);
                zr[ct][4 * q + 0] = z4.x;
                zr[ct][4 * q + 1] = z4.y;
                zr[ct][4 * q + 2] = z4.z;
                zr[ct][4 * q + 3] = z4.w;
            }
#pragma unroll
        for (int jg = 0; jg < JPW; jg += JG) {
            f32x16 acc[JG][CTW];
            float sm[JG], sL[JG], sD[JG];
            int valid_j[JG];
#pragma unroll
            for (int u = 0; u < JG; ++u) {
                const int jj = jg + u;
                const int job = ts + jj * TS;
                const bool is_q = job < SUB;
                const int sub = is_q ? job : job - SUB;
                valid_j[u] = (jj < JPW && job < JOBS) ? int(max<int64_t>(0, min<int64_t>(32, rows - nc - sub * 32))) : 0;
                if (SHARE_X)
                    scores_lds<DR, CTW>(P, is_q ? XtQ : XtK, sub, acc[u]);
                else
                    scores_x<DR, CTW>(P, xc[jj < JPW ? jj : 0], acc[u]);
                local_softmax<CTW, true>(acc[u], zr, sm[u], sL[u], sD[u]);
                if (CS > 1 && lh == 0 && jj < JPW) st[jj][(ts * CS + cs) * 32 + j] = ScanStats{sm[u], sL[u], sD[u]};
            }
            if (CS > 1) __syncthreads();  // B1: this group's softmax statistics published
#pragma unroll
            for (int u = 0; u < JG; ++u) {
                const int jj = jg + u;
                const int job = ts + jj * TS;
                if (jj >= JPW || job >= JOBS) continue;
                const bool is_q = job < SUB;
                const int sub = is_q ? job : job - SUB;
                float scale, dl;
                if (CS == 1) {
                    scale = 1.0f / sL[u];
                    dl = sD[u] / sL[u];
                } else {
                    float mm = -INFINITY;
#pragma unroll
                    for (int c = 0; c < CS; ++c) mm = fmaxf(mm, st[jj][(ts * CS + c) * 32 + j].m);
                    float Lt = 0.0f, Dt = 0.0f;
#pragma unroll
                    for (int c = 0; c < CS; ++c) {
                        const ScanStats sc = st[jj][(ts * CS + c) * 32 + j];
                        const float f = __builtin_amdgcn_exp2f(sc.m - mm);
                        Lt = fmaf(sc.L, f, Lt);
                        Dt = fmaf(sc.D, f, Dt);
                    }
                    scale = __builtin_amdgcn_exp2f(sm[u] - mm) / Lt;
                    dl = Dt / Lt;
                }
                if (j >= valid_j[u]) scale = 0.0f;
                store_gamma_lds<CTW>(acc[u], scale, is_q ? Gq : Gk, LDG, sub * 32 + j, cs * CTW);
                if (is_q && cs == 0 && lh == 0) den_inter[sub * 32 + j] = dl;
            }
        }
        if (!SHARE_X) load_frags(nc + 2 * CH, xc);
        __syncthreads();  // B2: Gq, Gk complete; this chunk's x tiles consumed
        // next chunk's inputs into the buffers that are now free; the loads of the one
        // after are issued
        commit_v(Vs[vb ^ 1]);
        load_v(nc + 2 * CH);
        if (SHARE_X) {
            xq.commit(XtQ);
            xk.commit(XtK);
            xq.load(rq, nc + 2 * CH);
            xk.load(rk, nc + 2 * CH);
        }
        // ---- phase S: S^T tiles (rows = key positions, cols = query positions)
        if (wave < STILES) {
            int qt = 0, kt = wave;
            while (kt > qt) { kt -= qt + 1; ++qt; }
            f32x16 sacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < Kp / 16; ++ks) {
                bf16x8 a = read_rowfrag(Gk, LDG, kt * 32 + j, 16 * ks);
                bf16x8 b = read_rowfrag(Gq, LDG, qt * 32 + j, 16 * ks);
                sacc = mfma(a, b, sacc);
            }
            float rs = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = kt * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (kk > qt * 32 + j) sacc[r] = 0.0f;  // j > i is outside the causal support
                rs += sacc[r];
            }
            rs = xsum32(rs);
            if (lh == 0) den_part[kt][qt * 32 + j] = rs;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x2 v;
                v[0] = pack_bf16x2(sacc[4 * q + 0], sacc[4 * q + 1]);
                v[1] = pack_bf16x2(sacc[4 * q + 2], sacc[4 * q + 3]);
                *reinterpret_cast<u32x2*>(Ss + (qt * 32 + j) * LDSS + kt * 32 + 8 * q + 4 * lh) = v;
            }
        }
        __syncthreads();  // B3: S tiles and row sums complete
        // ---- phase O: outputs of this wave's value columns, then the memory update
        const uint16_t* Vc = Vs[vb];
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
            const int c16 = wave + cc * NW;
            if (c16 >= C16) continue;
            f32x4 o[CH / 16];
#pragma unroll
            for (int t16 = 0; t16 < CH / 16; ++t16) {
                o[t16] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                // intra-chunk part: V^T S^T over key positions up to this query tile
#pragma unroll
                for (int ks = 0; ks < (t16 * 16 + 16 + 31) / 32; ++ks) {
                    bf16x8 a = read_colfrag16(Vc, LDV, 32 * ks, c16 * 16);
                    bf16x8 b = *reinterpret_cast<const bf16x8*>(Ss + (t16 * 16 + i16) * LDSS + 32 * ks + 8 * g4);
                    o[t16] = mfma16(a, b, o[t16]);
                }
            }
            // inter-chunk part: memory^T Gq^T, memory split into hi + lo bf16 once per k-step
#pragma unroll
            for (int m2 = 0; m2 < Kp / 32; ++m2) {
                u32x4 ah, al;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int v0 = 2 * q, v1 = 2 * q + 1;
                    const float x0 = mem[cc][2 * m2 + (v0 >> 2)][v0 & 3];
                    const float x1 = mem[cc][2 * m2 + (v1 >> 2)][v1 & 3];
                    const uint32_t hb = pack_bf16x2(x0, x1);
                    ah[q] = hb;
                    al[q] = pack_bf16x2(x0 - __uint_as_float(hb << 16), x1 - __uint_as_float(hb & 0xffff0000u));
                }
#pragma unroll
                for (int t16 = 0; t16 < CH / 16; ++t16) {
                    const int qrow = t16 * 16 + i16;
                    const u32x2 b0 = *reinterpret_cast<const u32x2*>(Gq + qrow * LDG + 32 * m2 + 4 * g4);
                    const u32x2 b1 = *reinterpret_cast<const u32x2*>(Gq + qrow * LDG + 32 * m2 + 16 + 4 * g4);
                    const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{b0[0], b0[1], b1[0], b1[1]});
                    o[t16] = mfma16(__builtin_bit_cast(bf16x8, ah), b, o[t16]);
                    o[t16] = mfma16(__builtin_bit_cast(bf16x8, al), b, o[t16]);
                }
            }
#pragma unroll
            for (int t16 = 0; t16 < CH / 16; ++t16) {
                const int qrow = t16 * 16 + i16;
                float den = den_inter[qrow] + eps;
#pragma unroll
                for (int kt = 0; kt < SUB; ++kt)
                    if (kt * 32 <= qrow) den += den_part[kt][qrow];
                const float rden = 1.0f / den;
                u32x2 v;
                v[0] = pack_bf16x2(o[t16][0] * rden, o[t16][1] * rden);
                v[1] = pack_bf16x2(o[t16][2] * rden, o[t16][3] * rden);
                // rows past the segment fall outside the resource and are dropped
                buf_store8(ro, uint32_t(((nc + qrow) * DV + c16 * 16 + 4 * g4) * 2), v);
            }
        }
        // memory update: Vt += Gk^T Vc (every wave its columns), Z += Gk^T 1 (wave 0)
        float zacc[KT16];
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt) zacc[kt] = 0.0f;
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt)
#pragma unroll
            for (int ks = 0; ks < CH / 32; ++ks) {
                const bf16x8 a = read_colfrag16(Gk, LDG, 32 * ks, kt * 16);
                if (wave == 0) {
#pragma unroll
                    for (int v = 0; v < 8; ++v) zacc[kt] += float(a[v]);
                }
#pragma unroll
                for (int cc = 0; cc < CPW; ++cc) {
                    const int c16 = wave + cc * NW;
                    if (c16 < C16) {
                        const bf16x8 b = read_colfrag16(Vc, LDV, 32 * ks, c16 * 16);
                        mem[cc][kt] = mfma16(a, b, mem[cc][kt]);
                    }
                }
            }
        if (wave == 0) {
#pragma unroll
            for (int kt = 0; kt < KT16; ++kt) {
                float z = zacc[kt];
                z += __shfl_xor(z, 16, 64);
                z += __shfl_xor(z, 32, 64);
                if (g4 == 0) Zs[kt * 16 + i16] += z;
            }
        }
    };
    // Chunks run in pairs.  A chunk past the segment end (odd chunk count) is harmless:
    // its loads read zeros, its rows get zero responsibilities (no memory update) and
    // its stores fall outside the output resource.
    for (int64_t nc = 0; nc < rows; nc += 2 * CH) {
        chunk(nc, 0, xf);
        chunk(nc + CH, 1, xn);
    }
    if (state_out && seg_idx == G - 1) {
        __syncthreads();  // the last chunk's Z update is visible
        store_memory<CPW, KT16, NW, DV>(mem, Zs, state_out + p * SE, mx.K);
    }
}

template <typename F>
hipError_t with_all(int dr, int kt, int vt, int ch, F&& f) {
#define GMA_SCAN_CH(D, T, W)                                                                                    \
    if (dr == D && kt == T && vt == W && ch == 32)                                                              \
        return f(std::integral_constant<int, D>(), std::integral_constant<int, T>(), std::integral_constant<int, W>(), \
                 std::integral_constant<int, 32>());                                                            \
    if (dr == D && kt == T && vt == W && ch == 64)                                                              \
        return f(std::integral_constant<int, D>(), std::integral_constant<int, T>(), std::integral_constant<int, W>(), \
                 std::integral_constant<int, 64>());
#define GMA_SCAN_VT(D, T) GMA_SCAN_CH(D, T, 1) GMA_SCAN_CH(D, T, 2) GMA_SCAN_CH(D, T, 4)
#define GMA_SCAN_KT(D) GMA_SCAN_VT(D, 1) GMA_SCAN_VT(D, 2) GMA_SCAN_VT(D, 4)
    // 8 component tiles with d_r <= 64 take the wide scan (gma_bf16_wide.hip)
    GMA_SCAN_KT(16) GMA_SCAN_KT(32) GMA_SCAN_KT(64) GMA_SCAN_KT(128) GMA_SCAN_VT(128, 8)
#undef GMA_SCAN_KT
#undef GMA_SCAN_VT
#undef GMA_SCAN_CH
    return hipErrorNotSupported;
}

}  // namespace bf

// The chunk the bf16 scans run: the requested one (32, 64 or 128 positions; the scans form their
// scores on 32-position subtiles, so 16 is refused when the call is validated), capped at 64,
// the largest compiled, and halved where the chunk's tiles do not fit (scan_chunk,
// serial_scan_chunk); the scan of 256 components takes 32.  The chunk length only changes the
// order of the sums.
int64_t bf16_causal_chunk(const Plan& p) {
    if (bf16_causal_wide_applies(p)) return 32;
    int64_t used = 0;
    (void)bf::with_all(int(p.dr), int(p.Kp / 32), int(p.dv / 32), p.chunk >= 64 ? 64 : 32,
                       [&](auto D, auto T, auto W, auto C) {
                           constexpr int DR = decltype(D)::value, KT = decltype(T)::value,
                                         VT = decltype(W)::value, CH = decltype(C)::value;
                           if constexpr (KT <= 4 && DR * KT <= 256)
                               used = bf::scan_chunk<DR, KT, VT, CH>();
                           else
                               used = bf::serial_scan_chunk<DR, KT, VT, CH>();
                           return hipSuccess;
                       });
    return used;
}

// Shapes whose registers fit the pipelined scan run the fused causal kernel; 256 components with
// d_r <= 64 the wide scan; the others the segment aggregates (write kernel) and then the serial scan.
hipError_t bf16_causal(const Plan& p, const void* XQ, const void* XK, const void* V, const float* mu, const float* s2,
                       const float* pi, float eps, void* O, char* ws, hipStream_t st, const float* state_in,
                       float* state_out) {
    if (bf16_causal_wide_applies(p))
        return bf16_causal_wide(p, XQ, XK, V, mu, s2, pi, eps, O, ws, st, state_in, state_out);
    const bf::Mixture mx{mu, s2, pi, int(p.K)};
    float* aggregates = reinterpret_cast<float*>(ws + p.off_partials);
    uint64_t* flags = reinterpret_cast<uint64_t*>(ws + p.off_flags);
    const int ch = p.chunk >= 64 ? 64 : 32;  // the compiled request; the kernels may halve it
    uint32_t* err = nullptr;
    hipError_t de = device_error_word(&err);
    if (de != hipSuccess) return de;
    return bf::with_all(int(p.dr), int(p.Kp / 32), int(p.dv / 32), ch, [&](auto D, auto T, auto W, auto C) {
        constexpr int DR = decltype(D)::value, KT = decltype(T)::value, VT = decltype(W)::value,
                      CH = decltype(C)::value;
        using S = bf::Split<DR, KT>;
        // pipelined scan where its registers suffice (up to 4 component tiles and d_r * K <= 8192)
        if constexpr (KT <= 4 && DR * KT <= 256) {
            // one launch; without the in-launch hand-off (single launch disabled) the aggregates
            // come from a launch of their own first
            const bool single = single_launch_enabled();
            if (!single && p.G > 1) {
                hipError_t e = bf16_write_partials(p, XK, V, mu, s2, pi, ws, st, p.G - 1);
                if (e != hipSuccess) return e;
            }
            GMA_LAUNCH("bf16_causal", (bf::causal_kernel<DR, KT, VT, CH>), dim3(unsigned(p.G), unsigned(p.P)),
                       dim3(S::NW * 64), 0, st, static_cast<const uint16_t*>(XQ), static_cast<const uint16_t*>(XK),
                       static_cast<const uint16_t*>(V), p.N, int(p.H), p.seg, int(p.G), mx, aggregates, flags,
                       launch_token(), wait_limit(), single ? 0 : 1, eps, static_cast<uint16_t*>(O), state_in,
                       state_out, err);
        } else {
            // aggregates of segments 0 .. G-2 (the last segment's aggregate is never read)
            if (p.G > 1) {
                hipError_t e = bf16_write_partials(p, XK, V, mu, s2, pi, ws, st, p.G - 1);
                if (e != hipSuccess) return e;
            }
            GMA_LAUNCH("bf16_scan", (bf::serial_scan_kernel<DR, KT, VT, CH>), dim3(unsigned(p.G), unsigned(p.P)),
                       dim3(S::NW * 64), 0, st, static_cast<const uint16_t*>(XQ), static_cast<const uint16_t*>(XK),
                       static_cast<const uint16_t*>(V), p.N, int(p.H), p.seg, int(p.G), mx, aggregates, eps,
                       static_cast<uint16_t*>(O), state_in, state_out);
        }
        return hipGetLastError();
    });
}

}  // namespace gma
