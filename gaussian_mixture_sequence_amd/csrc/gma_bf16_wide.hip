// Causal GMA of the bf16 path with 256 components (8 tiles of 32; K in (128, 256]), d_r <= 64:
// one launch, one sequence segment per workgroup of 8 waves.
//
// Sec. 3.5 of "Gaussian Mixture Attention" defines the prefix memory (Eq. 6b) and the output
// (Eq. 8b): Vt^(i) = sum_{j<=i} gamma^K_j V_j^T, Z^(i) = sum_{j<=i} gamma^K_j,
// O_i = gamma^Q_i Vt^(i) / (gamma^Q_i Z^(i) + eps), the sums running along the sequence.  The
// sequence of each (batch, head) problem is cut into G segments; workgroup (s, p) owns segment s:
//   1. key pass: the keys' responsibilities of the segment, chunk by chunk, into the workspace
//      ([N][256] bf16 per problem), and (segments 0 .. G-2) the segment's own memory, sum over its
//      positions of gamma^K_j [V_j | 1], published for the later segments;
//   2. once the aggregates of segments 0 .. s-1 are published (only lower-numbered workgroups,
//      dispatched no later than this one, so the launch needs no co-residency), the starting
//      memory is the carried memory plus those aggregates in increasing order;
//   3. scan: chunks of CH = 32 positions with responsibilities Gq (scored here), Gk (read back
//      from the key pass; bf16, in LDS) and values Vc:  S = Gq Gk^T kept for key j <= query i,
//      num = S Vc + Gq Vt,  den = S 1 + Gq Z + eps, then Vt += Gk^T Vc, Z += Gk^T 1.
// Each side's scores are formed once: the key pass writes 512 bytes per position and the scan
// reads them back, in place of a second set of key-side score products and softmax.
//
// Two kinds of waves.  Waves w and w + 4 of a workgroup run on the same SIMD, so every SIMD holds
// one of each and the matrix cores of one overlap the vector work of the other:
//   score waves 0..3:  wave s holds the score operands of component tiles 2s, 2s + 1 (the 5-term
//                      split-operand scores of gma_bf16_common.h) and turns the x tiles of the next
//                      chunk into its responsibilities (softmax statistics combined over the four
//                      waves through LDS); in the scan they also form the chunk's S tiles and the
//                      partial sums of Gq Z;
//   memory waves 4..7: wave 4 + m holds the fp32 memory of value-column tiles m (and m + 4 for
//                      d_v = 128) as sixteen 16x16 MFMA accumulators each (Vt^T's D layout) and
//                      computes the outputs and memory update; Z lives in LDS.
// Each kind runs its own loop; both pass the same barriers, two per chunk c (buffers b = c % 2
// hold chunk c):
//   part 1: score waves: S(c) tiles, partial sums of Gq(c) Z, scores of chunk c+1 (x tiles in
//           LDS) and their statistics; memory waves: inter part Vt^T Gq(c)^T (memory before
//           chunk c, split into hi + lo bf16)                                     -> B_Q
//   part 2: score waves: Gq of chunk c+1 into the other buffer, x tile of c+2 committed;
//           memory waves: Gk(c+1) and V(c+1) committed, memory update with chunk c, intra part
//           V(c)^T S(c)^T, outputs of chunk c divided and stored, Z advanced       -> B_P
// The key pass runs the same loops on the key side alone: the memory waves update the memory
// with chunk c and write Gk(c) to the workspace in part 1, the score waves turn the next chunk's
// keys into Gk.
#include <cstdint>
#include <type_traits>

#include "gma_bf16_common.h"
#include "gma_internal.h"

namespace gma {
namespace bf {

template <int DR, int VT, int NW>
struct WideLds {
    static constexpr int KT = 8, Kp = 256, DV = VT * 32, CH = 32, NS = NW / 2, NT = NW * 64, HT = NT / 2;
    static constexpr int LDG = Kp + 8, LDV = DV + 8, LDSS = CH + 8;
    using XT = XTile<DR, CH, HT>;  // staged by the score waves' threads
    using g_t = uint16_t[2][CH * LDG];
    using v_t = uint16_t[2][CH * LDV];
    using s_t = uint16_t[CH * LDSS];
    using x_t = u32x4[XT::LDS_BYTES / 16];
    using st_t = float[2][NS][CH][2];   // (m, L) per job (0: keys, 1: queries), score wave, position
    using di_t = float[CH];             // Gq Z per query
    using dp_t = float[2][CH];          // S row sums of key block 0 and 1
    using z_t = float[Kp];
    using c_t = float[Kp];              // score constants c_k (log2 units)
    using vote_t = int[NW];
    static constexpr size_t o_gq = 0, o_gk = lds_align(o_gq + sizeof(g_t)), o_vs = lds_align(o_gk + sizeof(g_t)),
                            o_ss = lds_align(o_vs + sizeof(v_t)), o_xq = lds_align(o_ss + sizeof(s_t)),
                            o_xk = lds_align(o_xq + sizeof(x_t)), o_st = lds_align(o_xk + sizeof(x_t)),
                            o_di = lds_align(o_st + sizeof(st_t)), o_dp = lds_align(o_di + sizeof(di_t)),
                            o_zs = lds_align(o_dp + sizeof(dp_t)), o_cs = lds_align(o_zs + sizeof(z_t)),
                            o_vote = lds_align(o_cs + sizeof(c_t)), bytes = lds_align(o_vote + sizeof(vote_t));
};

// Scores of one 32-token subtile for component tiles ct0 .. ct0 + CTW - 1 from an XTile in LDS,
// the accumulators starting at the score constants (in LDS, [Kp] fp32).
template <int DR, int CTW>
__device__ __forceinline__ void wide_scores(const WaveParams<DR, CTW>& P, const float* cst, int ct0, const u32x4* xt,
                                            f32x16 (&acc)[CTW]) {
    const int lh = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 cv = *reinterpret_cast<const float4*>(cst + (ct0 + ct) * 32 + 8 * q + 4 * lh);
            acc[ct][4 * q + 0] = cv.x;
            acc[ct][4 * q + 1] = cv.y;
            acc[ct][4 * q + 2] = cv.z;
            acc[ct][4 * q + 3] = cv.w;
        }
#pragma unroll
    for (int ks = 0; ks < DR / 16; ++ks) {
        bf16x8 x, x2h, x2l;
        xtile_frags<DR>(xt, 0, ks, x, x2h, x2l);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            acc[ct] = mfma(P.w[ct][ks][0], x, acc[ct]);
            acc[ct] = mfma(P.w[ct][ks][1], x, acc[ct]);
            acc[ct] = mfma(P.w[ct][ks][2], x2h, acc[ct]);
            acc[ct] = mfma(P.w[ct][ks][3], x2h, acc[ct]);
            acc[ct] = mfma(P.w[ct][ks][2], x2l, acc[ct]);
        }
    }
}

// mode 0: the whole forward (every segment runs its key pass, segments 0 .. G-2 publish their
// aggregates, every segment waits for the aggregates before it, then scans); mode 1: key passes
// only (grid G segments); mode 2: scans only, the key passes run by an earlier launch (no waits).
// gk_cache: [P][N][256] bf16 workspace for the keys' responsibilities.
template <int DR, int VT, int NW>
__global__ void __launch_bounds__(NW * 64)
    wide_causal_kernel(const uint16_t* __restrict__ XQ, const uint16_t* __restrict__ XK, const uint16_t* __restrict__ V,
                       int64_t N, int H, int64_t seg, int G, Mixture mx, float* __restrict__ aggregates,
                       uint64_t* __restrict__ flags, uint64_t token, uint32_t wait_limit, int mode, float eps,
                       uint16_t* __restrict__ O, const float* __restrict__ state_in, float* __restrict__ state_out,
                       uint16_t* __restrict__ gk_cache, uint32_t* __restrict__ err) {
    using LY = WideLds<DR, VT, NW>;
    constexpr int Kp = LY::Kp, DV = LY::DV, CH = LY::CH, NS = LY::NS, HT = LY::HT, NT = LY::NT;
    constexpr int CTS = LY::KT / NS;       // component tiles per score wave
    constexpr int NM = NW - NS;            // memory waves
    constexpr int LDG = LY::LDG, LDV = LY::LDV, LDSS = LY::LDSS;
    constexpr int KT16 = Kp / 16;          // 16-row component tiles of the memory
    constexpr int C16 = DV / 16;           // 16-wide value-column tiles
    constexpr int CPW = (C16 + NM - 1) / NM;  // column tiles per memory wave: tiles m, m + NM, ..
    constexpr int ZPW = KT16 / NM;         // Z tiles per memory wave: ZPW m ..
    constexpr int E = Kp * (DV + 1);
    constexpr int VCHUNKS = CH * DV / 8, VCH = (VCHUNKS + HT - 1) / HT;
    constexpr bool VEVEN = VCHUNKS % HT == 0;
    using XT = typename LY::XT;
    __shared__ __attribute__((aligned(16))) char smem[LY::bytes];
    typename LY::g_t& Gq = *reinterpret_cast<typename LY::g_t*>(smem + LY::o_gq);
    typename LY::g_t& Gk = *reinterpret_cast<typename LY::g_t*>(smem + LY::o_gk);
    typename LY::v_t& Vs = *reinterpret_cast<typename LY::v_t*>(smem + LY::o_vs);
    typename LY::s_t& Ss = *reinterpret_cast<typename LY::s_t*>(smem + LY::o_ss);
    typename LY::x_t& XtQ = *reinterpret_cast<typename LY::x_t*>(smem + LY::o_xq);
    typename LY::x_t& XtK = *reinterpret_cast<typename LY::x_t*>(smem + LY::o_xk);
    typename LY::st_t& st = *reinterpret_cast<typename LY::st_t*>(smem + LY::o_st);
    typename LY::di_t& den_ip = *reinterpret_cast<typename LY::di_t*>(smem + LY::o_di);
    typename LY::dp_t& den_part = *reinterpret_cast<typename LY::dp_t*>(smem + LY::o_dp);
    float* Zs = reinterpret_cast<float*>(smem + LY::o_zs);
    float* cst = reinterpret_cast<float*>(smem + LY::o_cs);
    int* vote = reinterpret_cast<int*>(smem + LY::o_vote);

    const int wave = wave_id(), l = threadIdx.x & 63, lh = l >> 5, j = l & 31, g4 = l >> 4, i16 = l & 15;
    const bool scorer = wave < NS;
    const int ht = int(threadIdx.x) & (HT - 1);  // thread index within its half (score or memory waves)
    const int64_t p = blockIdx.y;
    const int s = blockIdx.x, h = int(p % H);
    const int64_t lo = int64_t(s) * seg, hi = min<int64_t>(lo + seg, N), rows = hi - lo;
    const int64_t C = (rows + CH - 1) / CH;  // chunks of the segment
    float* agg = aggregates + size_t(p) * G * E;
    uint64_t* fl = flags + size_t(p) * G;
    const size_t SE = size_t(mx.K) * (DV + 1);  // one problem's carried memory
    const bool keypass = mode != 2, publish = s + 1 < G;  // the last segment's aggregate has no reader
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(XQ + (size_t(p) * N + lo) * DR, rows * DR * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(XK + (size_t(p) * N + lo) * DR, rows * DR * 2);
    bool ok = true;

    if (scorer) {
        // ================================================================ score waves
        const int ct0 = CTS * wave;
        WaveParams<DR, CTS> P;
        P.compute(mx, h, ct0);
        if (j == 0)  // the constants of the wave's tiles into LDS (lanes 0 and 32 hold both halves)
#pragma unroll
            for (int ct = 0; ct < CTS; ++ct)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int i = 0; i < 4; ++i) cst[(ct0 + ct) * 32 + 8 * q + 4 * lh + i] = P.c[ct][4 * q + i];
        // S tile (query block 0, key block 1) lies above the diagonal: zero for good
        for (int c = ht; c < CH * LDSS / 8; c += HT) reinterpret_cast<u32x4*>(Ss)[c] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();  // B_init: constants and the zero tile visible

        // one side per phase: the keys in the key pass, the queries in the scan.  The score
        // products run two chunks ahead of the Gamma stores, so a wave's softmax of chunk c+1
        // has the products of chunk c+2 to overlap; the x tiles of even and odd chunks use the
        // two x buffers in turn.
        auto run = [&](auto agg_tag) __attribute__((always_inline)) {
            constexpr bool AGG = decltype(agg_tag)::value;
            constexpr int JB = AGG ? 0 : 1;  // statistics slot: 0 keys, 1 queries
            const __amdgpu_buffer_rsrc_t rx = AGG ? rk : rq;
            u32x4* Xb[2] = {XtQ, XtK};
            XT xt;
            f32x16 acc0[CTS], acc1[CTS];
            float sm_m, sm_L;
            // the statistics of one chunk's raw scores (acc then holds the exponentials)
            auto softmax = [&](f32x16(&acc)[CTS]) __attribute__((always_inline)) {
                float D, zdummy[CTS][16];
                local_softmax<CTS, false>(acc, zdummy, sm_m, sm_L, D);
                if (lh == 0) {
                    st[JB][wave][j][0] = sm_m;
                    st[JB][wave][j][1] = sm_L;
                }
            };
            auto store_gamma = [&](const f32x16(&acc)[CTS], int64_t row0, int b) __attribute__((always_inline)) {
                const bool valid = row0 + j < rows;
                float mm = -INFINITY;
#pragma unroll
                for (int w = 0; w < NS; ++w) mm = fmaxf(mm, st[JB][w][j][0]);
                float Lt = 0.0f;
#pragma unroll
                for (int w = 0; w < NS; ++w)
                    Lt = fmaf(st[JB][w][j][1], __builtin_amdgcn_exp2f(st[JB][w][j][0] - mm), Lt);
                float scale = __builtin_amdgcn_exp2f(sm_m - mm) * __builtin_amdgcn_rcpf(Lt);
                if (!valid) scale = 0.0f;  // positions past the segment: no responsibility
                store_gamma_lds<CTS>(acc, scale, AGG ? Gk[b] : Gq[b], LDG, j, ct0);
            };
            // prologue (barriers P0, P1, P2): Gamma(0), the raw scores of chunk 1, x(2) in LDS
            xt.load(rx, 0);
            xt.commit(Xb[0]);
            xt.load(rx, CH);
            __syncthreads();  // P0: x(0) in LDS
            wide_scores<DR, CTS>(P, cst, ct0, Xb[0], acc0);
            softmax(acc0);
            xt.commit(Xb[1]);  // x(1)
            xt.load(rx, 2 * CH);
            __syncthreads();  // P1: statistics of chunk 0, x(1) in LDS, x(0) consumed
            store_gamma(acc0, 0, 0);
            wide_scores<DR, CTS>(P, cst, ct0, Xb[1], acc1);
            xt.commit(Xb[0]);  // x(2)
            xt.load(rx, 3 * CH);
            __syncthreads();  // P2: Gamma(0) and x(2) in LDS
            // chunk c: cur holds the raw scores of chunk c+1, nxt receives those of chunk c+2
            auto chunk = [&](int64_t c, f32x16(&cur)[CTS], f32x16(&nxt)[CTS]) __attribute__((always_inline)) {
                const int b = int(c & 1);
                if constexpr (!AGG) {
                    // S^T tiles of chunk c (rows keys, columns queries), blocks (q, k) = (0,0), (1,0),
                    // (1,1) on waves 0, 1, 2, with their masked row sums
                    if (wave < 3) {
                        const int qb = wave > 0 ? 1 : 0, kb = wave > 1 ? 1 : 0;
                        f32x4 sacc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int ks = 0; ks < Kp / 32; ++ks)
                            sacc = mfma16(
                                *reinterpret_cast<const bf16x8*>(Gk[b] + (kb * 16 + i16) * LDG + 32 * ks + 8 * g4),
                                *reinterpret_cast<const bf16x8*>(Gq[b] + (qb * 16 + i16) * LDG + 32 * ks + 8 * g4), sacc);
                        float rs = 0.0f;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (kb * 16 + 4 * g4 + r > qb * 16 + i16) sacc[r] = 0.0f;  // key after query
                            rs += sacc[r];
                        }
                        rs += __shfl_xor(rs, 16, kWave);
                        rs += __shfl_xor(rs, 32, kWave);
                        if (g4 == 0) den_part[kb][qb * 16 + i16] = rs;
                        *reinterpret_cast<u32x2*>(Ss + (qb * 16 + i16) * LDSS + kb * 16 + 4 * g4) =
                            u32x2{pack_bf16x2(sacc[0], sacc[1]), pack_bf16x2(sacc[2], sacc[3])};
                    }
                    {  // Gq(c) Z (memory before chunk c): thread (row, part) sums components
                       // CPP part .. + CPP - 1, then the PARTS parts of a row are summed across lanes
                        constexpr int PARTS = HT / CH, CPP = Kp / PARTS, NH = CPP / 8;
                        const int row = ht / PARTS, part = ht % PARTS;
                        const uint16_t* gr = Gq[b] + row * LDG + CPP * part;
                        float d = 0.0f;
#pragma unroll
                        for (int h4 = 0; h4 < NH; ++h4) {
                            const int hh = (h4 + part) % NH;  // staggered: fewer bank conflicts on Zs
                            const u32x4 gv = *reinterpret_cast<const u32x4*>(gr + 8 * hh);
                            const float4 z0 = *reinterpret_cast<const float4*>(Zs + CPP * part + 8 * hh);
                            const float4 z1 = *reinterpret_cast<const float4*>(Zs + CPP * part + 8 * hh + 4);
                            d = fmaf(__uint_as_float(gv[0] << 16), z0.x, d);
                            d = fmaf(__uint_as_float(gv[0] & 0xffff0000u), z0.y, d);
                            d = fmaf(__uint_as_float(gv[1] << 16), z0.z, d);
                            d = fmaf(__uint_as_float(gv[1] & 0xffff0000u), z0.w, d);
                            d = fmaf(__uint_as_float(gv[2] << 16), z1.x, d);
                            d = fmaf(__uint_as_float(gv[2] & 0xffff0000u), z1.y, d);
                            d = fmaf(__uint_as_float(gv[3] << 16), z1.z, d);
                            d = fmaf(__uint_as_float(gv[3] & 0xffff0000u), z1.w, d);
                        }
#pragma unroll
                        for (int o = 1; o < PARTS; o <<= 1) d += __shfl_xor(d, o, kWave);
                        if (part == 0) den_ip[row] = d;
                    }
                }
                __builtin_amdgcn_s_setprio(1);
                wide_scores<DR, CTS>(P, cst, ct0, Xb[b], nxt);  // chunk c+2: x(c+2) is in buffer b
                softmax(cur);                                   // chunk c+1
                __builtin_amdgcn_s_setprio(0);
                __syncthreads();  // B_Q
                store_gamma(cur, (c + 1) * CH, b ^ 1);
                xt.commit(Xb[b ^ 1]);  // x(c+3): x(c+1) was consumed in chunk c-1
                xt.load(rx, (c + 4) * CH);
                __syncthreads();  // B_P
            };
            for (int64_t c = 0; c < C; c += 2) {
                chunk(c, acc1, acc0);
                if (c + 1 < C) chunk(c + 1, acc0, acc1);
            }
        };
        if (keypass) {
            run(std::true_type());
            if (publish) publish_token(fl + s, token);  // after the memory waves' stores of the aggregate
            if (mode == 1) return;
        }
        run(std::false_type());
    } else {
        // ================================================================ memory waves
        const int m = wave - NS;
        const bool has_cols = m < C16;
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + (size_t(p) * N + lo) * DV, rows * DV * 2);
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + (size_t(p) * N + lo) * DV, rows * DV * 2);
        const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
        f32x4 mem[CPW][KT16];
        u32x4 vr[VCH];
        auto load_v = [&](int64_t row0) {
#pragma unroll
            for (int u = 0; u < VCH; ++u) {
                const int c = ht + u * HT;
                vr[u] = (VEVEN || c < VCHUNKS) ? buf_load16(rv, uint32_t((row0 * DV + int64_t(c) * 8) * 2))
                                               : u32x4{0u, 0u, 0u, 0u};
            }
        };
        auto commit_v = [&](uint16_t* dst) {
#pragma unroll
            for (int u = 0; u < VCH; ++u) {
                const int c = ht + u * HT;
                if (VEVEN || c < VCHUNKS) {
                    const int row = c / (DV / 8), col = (c - row * (DV / 8)) * 8;
                    *reinterpret_cast<u32x4*>(dst + row * LDV + col) = vr[u];
                }
            }
        };
        // the keys' responsibilities of the segment in the workspace, [rows][Kp] bf16: chunk c's
        // rows go out in the key pass (from Gk) and come back in the scan (into Gk); rows past
        // the segment fall outside the resource (stores dropped, loads zero)
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(gk_cache + (size_t(p) * N + lo) * Kp, rows * Kp * 2);
        constexpr int GCHUNKS = CH * Kp / 8, GCH = GCHUNKS / HT;  // 16-byte pieces of a chunk's Gk
        static_assert(GCHUNKS % HT == 0, "whole pieces per memory-wave thread");
        u32x4 gr[GCH];
        auto load_g = [&](int64_t row0) {
#pragma unroll
            for (int u = 0; u < GCH; ++u)
                gr[u] = buf_load16(rg, uint32_t((row0 * Kp + int64_t(ht + u * HT) * 8) * 2));
        };
        auto commit_g = [&](uint16_t* dst) {
#pragma unroll
            for (int u = 0; u < GCH; ++u) {
                const int c = ht + u * HT, row = c / (Kp / 8), col = (c - row * (Kp / 8)) * 8;
                *reinterpret_cast<u32x4*>(dst + row * LDG + col) = gr[u];
            }
        };
        auto store_g = [&](const uint16_t* src, int64_t row0) {
#pragma unroll
            for (int u = 0; u < GCH; ++u) {
                const int c = ht + u * HT, row = c / (Kp / 8), col = (c - row * (Kp / 8)) * 8;
                buf_store16(rg, uint32_t((row0 * Kp + int64_t(c) * 8) * 2),
                            *reinterpret_cast<const u32x4*>(src + row * LDG + col));
            }
        };
        auto owns = [&](int cc) { return has_cols && m + NM * cc < C16; };
        // in the chunk loop: with d_v a multiple of 64 a wave that owns its first column tile
        // owns all CPW of them (known at compile time; the loops then carry no branches)
        constexpr bool ALL = C16 % NM == 0;
        auto owns_next = [&](int cc) { return ALL || owns(cc); };
        // V(c) column fragments of the wave's own column tiles
        auto load_bv = [&](int bb, bf16x8(&bv)[CPW]) __attribute__((always_inline)) {
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc)
                bv[cc] = owns_next(cc) ? read_colfrag16(Vs[bb], LDV, 0, 16 * (m + NM * cc)) : bf16x8{};
        };
        // memory += Gk(c)^T V(c) (own columns), Z += Gk(c)^T 1 (tiles 4 m .. 4 m + 3)
        auto update_memory = [&](int bb, const bf16x8(&bv)[CPW]) __attribute__((always_inline)) {
            __builtin_amdgcn_s_setprio(1);  // matrix-core work: ahead of the score waves' vector work
            if (owns(0)) {
                // two steps of look-ahead on the Gk fragment reads
                bf16x8 a0 = read_colfrag16(Gk[bb], LDG, 0, 0), a1 = read_colfrag16(Gk[bb], LDG, 0, 16);
#pragma unroll
                for (int kt = 0; kt < KT16; ++kt) {
                    const bf16x8 a = a0;
                    a0 = a1;
                    if (kt + 2 < KT16) a1 = read_colfrag16(Gk[bb], LDG, 0, 16 * (kt + 2));
#pragma unroll
                    for (int cc = 0; cc < CPW; ++cc)
                        if (owns_next(cc)) mem[cc][kt] = mfma16(a, bv[cc], mem[cc][kt]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
            {  // Zs is read again only after B_P
                bf16x8 az[ZPW];
                f32x4 zt[ZPW];
#pragma unroll
                for (int zi = 0; zi < ZPW; ++zi) az[zi] = read_colfrag16(Gk[bb], LDG, 0, 16 * (ZPW * m + zi));
#pragma unroll
                for (int zi = 0; zi < ZPW; ++zi) zt[zi] = mfma16(az[zi], ones, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
                if (i16 == 0)
#pragma unroll
                    for (int zi = 0; zi < ZPW; ++zi)
#pragma unroll
                        for (int r = 0; r < 4; ++r) Zs[16 * (ZPW * m + zi) + 4 * g4 + r] += zt[zi][r];
            }
        };
        __syncthreads();  // B_init

        // pre(): after the first V load is in flight, before the memory is read
        auto run = [&](auto agg_tag, auto&& pre) __attribute__((always_inline)) {
            constexpr bool AGG = decltype(agg_tag)::value;
            // prologue (barriers P0, P1, P2)
            load_v(0);
            if (!AGG) load_g(0);
            pre();
            commit_v(Vs[0]);
            if (!AGG) commit_g(Gk[0]);
            load_v(CH);
            if (!AGG) load_g(CH);
            __syncthreads();  // P0
            __syncthreads();  // P1
            __syncthreads();  // P2
            for (int64_t c = 0; c < C; ++c) {
                const int b = int(c & 1);
                const int64_t nc = c * CH;
                f32x4 o[CPW][2];
                // ---- part 1 (key pass: the memory update and Gk(c) to the workspace, beside the
                // score waves' products)
                if constexpr (AGG) {
                    bf16x8 bv[CPW];
                    load_bv(b, bv);
                    update_memory(b, bv);
                    store_g(Gk[b], nc);
                } else {
                    // inter part: O^T = Vt^T Gq^T over the memory before this chunk (hi + lo bf16);
                    // each 32-component step reads its two Gq fragments once for both column
                    // tiles and issues the four hi products before the four lo ones
#pragma unroll
                    for (int cc = 0; cc < CPW; ++cc) o[cc][0] = o[cc][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    auto gq_frags = [&](int m2, bf16x8(&bq)[2]) {
#pragma unroll
                        for (int t16 = 0; t16 < 2; ++t16) {
                            const uint16_t* gq = Gq[b] + (t16 * 16 + i16) * LDG + 32 * m2 + 4 * g4;
                            const u32x2 b0 = *reinterpret_cast<const u32x2*>(gq);
                            const u32x2 b1 = *reinterpret_cast<const u32x2*>(gq + 16);
                            bq[t16] = __builtin_bit_cast(bf16x8, u32x4{b0[0], b0[1], b1[0], b1[1]});
                        }
                    };
                    if (owns(0)) {
#pragma unroll
                        for (int m2 = 0; m2 < Kp / 32; ++m2) {
                            // the split below covers the latency of these reads
                            bf16x8 bq[2];
                            gq_frags(m2, bq);
#pragma unroll
                            for (int cc = 0; cc < CPW; ++cc) {
                                if (!owns_next(cc)) continue;
                                u32x4 ah, al;
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    const int v0 = 2 * q, v1 = 2 * q + 1;
                                    const float x0 = mem[cc][2 * m2 + (v0 >> 2)][v0 & 3];
                                    const float x1 = mem[cc][2 * m2 + (v1 >> 2)][v1 & 3];
                                    const uint32_t hb = pack_bf16x2(x0, x1);
                                    ah[q] = hb;
                                    al[q] = pack_bf16x2(x0 - __uint_as_float(hb << 16),
                                                        x1 - __uint_as_float(hb & 0xffff0000u));
                                }
#pragma unroll
                                for (int t16 = 0; t16 < 2; ++t16)
                                    o[cc][t16] = mfma16(__builtin_bit_cast(bf16x8, ah), bq[t16], o[cc][t16]);
#pragma unroll
                                for (int t16 = 0; t16 < 2; ++t16)
                                    o[cc][t16] = mfma16(__builtin_bit_cast(bf16x8, al), bq[t16], o[cc][t16]);
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
                __syncthreads();  // B_Q
                // ---- part 2: V(c+1) (and, in the scan, Gk(c+1)) into the free buffers first
                // (their waits then cover no output stores); scans: memory update with chunk c,
                // outputs of chunk c
                commit_v(Vs[b ^ 1]);
                load_v(nc + 2 * CH);
                if constexpr (!AGG) {
                    commit_g(Gk[b ^ 1]);
                    load_g(nc + 2 * CH);
                }
                if constexpr (!AGG) {
                    bf16x8 bv[CPW];  // V(c) column fragments: memory update and intra part
                    load_bv(b, bv);
                    update_memory(b, bv);
                    float rden[2];
#pragma unroll
                    for (int t16 = 0; t16 < 2; ++t16) {
                        const int q = t16 * 16 + i16;
                        float den = eps + den_ip[q] + den_part[0][q];
                        if (t16 == 1) den += den_part[1][q];
                        rden[t16] = __builtin_amdgcn_rcpf(den);
                    }
#pragma unroll
                    for (int cc = 0; cc < CPW; ++cc) {
                        if (!owns_next(cc)) continue;
                        const int c16 = m + NM * cc;
#pragma unroll
                        for (int t16 = 0; t16 < 2; ++t16) {
                            const bf16x8 bb = *reinterpret_cast<const bf16x8*>(Ss + (t16 * 16 + i16) * LDSS + 8 * g4);
                            o[cc][t16] = mfma16(bv[cc], bb, o[cc][t16]);
                        }
#pragma unroll
                        for (int t16 = 0; t16 < 2; ++t16) {
                            const int q = t16 * 16 + i16;
                            const float rd = rden[t16];
                            // positions past the segment fall outside the resource and are dropped
                            buf_store8(ro, uint32_t(((nc + q) * DV + 16 * c16 + 4 * g4) * 2),
                                       u32x2{pack_bf16x2(o[cc][t16][0] * rd, o[cc][t16][1] * rd),
                                             pack_bf16x2(o[cc][t16][2] * rd, o[cc][t16][3] * rd)});
                        }
                    }
                }
                __syncthreads();  // B_P
            }
        };

        if (keypass) {
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
                for (int kt = 0; kt < KT16; ++kt) mem[cc][kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            for (int k = ht; k < Kp; k += HT) Zs[k] = 0.0f;
            run(std::true_type(), [] {});
        }
        if (keypass && publish) {
            // VtT [DV][Kp] then Z [Kp], device-coherent for the consumers in this launch
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(agg + size_t(s) * E, int64_t(E) * 4);
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc)
                if (owns(cc))
#pragma unroll
                    for (int kt = 0; kt < KT16; ++kt)
                        buf_store16_dev(ra, uint32_t(((16 * (m + NM * cc) + i16) * Kp + 16 * kt + 4 * g4) * 4),
                                        u32x4{__float_as_uint(mem[cc][kt][0]), __float_as_uint(mem[cc][kt][1]),
                                              __float_as_uint(mem[cc][kt][2]), __float_as_uint(mem[cc][kt][3])});
            if (ht < Kp / 4) {
                const float4 z = *reinterpret_cast<const float4*>(Zs + 4 * ht);
                buf_store16_dev(ra, uint32_t((Kp * DV + 4 * ht) * 4),
                                u32x4{__float_as_uint(z.x), __float_as_uint(z.y), __float_as_uint(z.z), __float_as_uint(z.w)});
            }
            publish_token(fl + s, token);  // its barrier pairs with the score waves' publish
        }
        if (mode == 1) return;

        // the starting memory: the carried memory [K][DV + 1] (row k: Vt_k then Z_k) or zeros
        // (rows k >= K lie past the resource's end and read as zero), then the earlier aggregates
        {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(state_in ? state_in + p * SE : nullptr,
                                                        state_in ? int64_t(SE) * 4 : 0);
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
                for (int kt = 0; kt < KT16; ++kt) mem[cc][kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (state_in)
#pragma unroll
                for (int cc = 0; cc < CPW; ++cc)
                    if (owns(cc))
#pragma unroll
                        for (int kt = 0; kt < KT16; ++kt)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                mem[cc][kt][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                    rs, uint32_t(((16 * kt + 4 * g4 + r) * (DV + 1) + 16 * (m + NM * cc) + i16) * 4), 0, 0));
            if (ht < Kp / 4)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Zs[4 * ht + r] = state_in ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                                    rs, uint32_t(((4 * ht + r) * (DV + 1) + DV) * 4), 0, 0))
                                              : 0.0f;
        }
        run(std::false_type(), [&] {
            if (mode == 0) ok = wait_tokens(fl, s, token, wait_limit);
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(agg, int64_t(s) * int64_t(E) * 4);
            for (int gs = 0; gs < s; ++gs) {  // increasing segment order
                const uint32_t a = uint32_t(size_t(gs) * E * 4);
#pragma unroll
                for (int cc = 0; cc < CPW; ++cc)
                    if (owns(cc))
#pragma unroll
                        for (int kt = 0; kt < KT16; ++kt) {
                            const u32x4 v =
                                buf_load16_dev(ra, a + uint32_t(((16 * (m + NM * cc) + i16) * Kp + 16 * kt + 4 * g4) * 4));
#pragma unroll
                            for (int r = 0; r < 4; ++r) mem[cc][kt][r] += __uint_as_float(v[r]);
                            if (kt % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // bounds the loads in flight
                        }
                if (ht < Kp / 4) {
                    const u32x4 v = buf_load16_dev(ra, a + uint32_t((Kp * DV + 4 * ht) * 4));
#pragma unroll
                    for (int r = 0; r < 4; ++r) Zs[4 * ht + r] += __uint_as_float(v[r]);
                }
            }
        });
        float* so = (state_out && s == G - 1) ? state_out + p * SE : nullptr;
        if (so) {  // the memory after the last position, same layout; rows k >= K are dropped
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(so, int64_t(SE) * 4);
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc)
                if (owns(cc))
#pragma unroll
                    for (int kt = 0; kt < KT16; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            __builtin_amdgcn_raw_buffer_store_b32(
                                __float_as_uint(mem[cc][kt][r]), rs,
                                uint32_t(((16 * kt + 4 * g4 + r) * (DV + 1) + 16 * (m + NM * cc) + i16) * 4), 0, 0);
            if (ht < Kp / 4)  // Zs is complete after B_P of the last chunk
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Zs[4 * ht + r]), rs,
                                                          uint32_t(((4 * ht + r) * (DV + 1) + DV) * 4), 0, 0);
        }
    }

    // waves poll on their own: agree on the outcome before acting on it
    ok = workgroup_all(ok, vote);
    if (!ok) {  // the starting memory was never complete: make that visible in the outputs and to the host
        __builtin_amdgcn_s_waitcnt(0);  // the scan's own stores of these rows land first
        __syncthreads();
        uint16_t* op = O + (size_t(p) * N + lo) * DV;
        for (int64_t e = threadIdx.x; e < rows * DV; e += NT) op[e] = 0x7fc0u;
        if (state_out && s == G - 1)
            for (size_t e = threadIdx.x; e < SE; e += NT) state_out[p * SE + e] = __builtin_nanf("");
        if (threadIdx.x == 0) atomicOr(err, kDevErrTimeout);
    }
}

// Waves per workgroup.  Sixteen (one component tile per score wave, one column tile per memory
// wave) leave 128 registers per wave, which d_r = 64 exceeds: 79 spilled VGPRs and twice the time.
constexpr int kWideWaves = 8;

template <typename F>
hipError_t with_wide(int dr, int vt, F&& f) {
#define GMA_WIDE(D, W) \
    if (dr == D && vt == W) return f(std::integral_constant<int, D>(), std::integral_constant<int, W>());
    GMA_WIDE(16, 1) GMA_WIDE(16, 2) GMA_WIDE(16, 4)
    GMA_WIDE(32, 1) GMA_WIDE(32, 2) GMA_WIDE(32, 4)
    GMA_WIDE(64, 1) GMA_WIDE(64, 2) GMA_WIDE(64, 4)
#undef GMA_WIDE
    return hipErrorNotSupported;
}

}  // namespace bf

bool bf16_causal_wide_applies(const Plan& p) { return p.Kp == 256 && p.dr <= 64; }

hipError_t bf16_causal_wide(const Plan& p, const void* XQ, const void* XK, const void* V, const float* mu,
                            const float* s2, const float* pi, float eps, void* O, char* ws, hipStream_t st,
                            const float* state_in, float* state_out) {
    const bf::Mixture mx{mu, s2, pi, int(p.K)};
    float* aggregates = reinterpret_cast<float*>(ws + p.off_partials);
    uint64_t* flags = reinterpret_cast<uint64_t*>(ws + p.off_flags);
    uint16_t* gk_cache = reinterpret_cast<uint16_t*>(ws + p.off_gk);
    uint32_t* err = nullptr;
    hipError_t e = device_error_word(&err);
    if (e != hipSuccess) return e;
    return bf::with_wide(int(p.dr), int(p.dv / 32), [&](auto D, auto W) {
        constexpr int DR = decltype(D)::value, VT = decltype(W)::value;
        const bool single = single_launch_enabled();
        const uint64_t token = launch_token();
        auto launch = [&](unsigned grid_x, int mode) {
            GMA_LAUNCH(mode == 1 ? "bf16_causal_aggregate" : "bf16_causal", (bf::wide_causal_kernel<DR, VT, bf::kWideWaves>),
                       dim3(grid_x, unsigned(p.P)), dim3(bf::kWideWaves * 64), 0, st, static_cast<const uint16_t*>(XQ),
                       static_cast<const uint16_t*>(XK), static_cast<const uint16_t*>(V), p.N, int(p.H), p.seg,
                       int(p.G), mx, aggregates, flags, token, wait_limit(), mode, eps, static_cast<uint16_t*>(O),
                       state_in, state_out, gk_cache, err);
            return hipGetLastError();
        };
        if (single) return launch(unsigned(p.G), 0);
        // the key passes in a launch of their own, then the scans without waits
        hipError_t r = launch(unsigned(p.G), 1);
        if (r != hipSuccess) return r;
        return launch(unsigned(p.G), 2);
    });
}

}  // namespace gma
