// Causal GMA of the bf16 path with 256 components (8 tiles of 32; K in (128, 256]), d_r <= 64:
// one launch, one sequence segment per workgroup of 8 waves.
//
// Sec. 3.5 of "Gaussian Mixture Attention" defines the prefix memory (Eq. 6b) and the output
// (Eq. 8b): Vt^(i) = sum_{j<=i} gamma^K_j V_j^T, Z^(i) = sum_{j<=i} gamma^K_j,
// O_i = gamma^Q_i Vt^(i) / (gamma^Q_i Z^(i) + eps), the sums running along the sequence.  The
// sequence of each (batch, head) problem is cut into G segments; workgroup (s, p) owns segment s:
//   1. aggregate (segments 0 .. G-2): the segment's own memory, sum over its positions of
//      gamma^K_j [V_j | 1], chunk by chunk; published for the later segments;
//   2. once the aggregates of segments 0 .. s-1 are published (only lower-numbered workgroups,
//      dispatched no later than this one, so the launch needs no co-residency), the starting
//      memory is the carried memory plus those aggregates in increasing order;
//   3. scan: chunks of CH = 32 positions with responsibilities Gq, Gk (bf16, in LDS) and values
//      Vc:  S = Gq Gk^T kept for key j <= query i,  num = S Vc + Gq Vt,  den = S 1 + Gq Z + eps,
//      then Vt += Gk^T Vc, Z += Gk^T 1.
//
// Work split over the 8 waves: wave w holds the score operands of component tile w (the 5-term
// split-operand scores of gma_bf16_common.h), so the softmax over the 256 components combines
// the waves' statistics through LDS; wave w owns value columns 16 w .. 16 w + 15 of the fp32
// memory, kept in registers as sixteen 16x16 MFMA accumulators (Vt^T's D layout,
// init_memory), and computes those columns of the outputs; Z lives in LDS.
//
// Software pipeline, two barriers per chunk c (buffers b = c % 2 hold chunk c):
//   region 1: S(c) tiles (3 waves), partial sums of Gq(c) Z, scores of chunk c+1 (x tiles of
//             c+1 in LDS) and their per-wave softmax statistics                   -> B_Q
//   region 2: Gq, Gk of chunk c+1 into the other buffers (statistics combined); inter part
//             Vt^T Gq(c)^T over the memory before chunk c (split into hi + lo bf16), memory
//             update with chunk c, intra part V(c)^T S(c)^T, outputs of chunk c divided and
//             stored, Z advanced; V(c+1) and the x tiles of c+2 committed, loads of V(c+2)
//             and x(c+3) issued                                                  -> B_P
// (the scores live across B_Q only until they are stored, so the memory's products in region 2
// have the registers the scores had)
// The aggregate phase runs the same loop on the key side alone.
#include <cstdint>
#include <type_traits>

#include "gma_bf16_common.h"
#include "gma_internal.h"

namespace gma {
namespace bf {

template <int DR, int VT>
struct WideLds {
    static constexpr int KT = 8, Kp = 256, DV = VT * 32, CH = 32, NW = 8, NT = NW * 64;
    static constexpr int LDG = Kp + 8, LDV = DV + 8, LDSS = CH + 8, DPARTS = 16;
    using XT = XTile<DR, CH, NT>;
    using g_t = uint16_t[2][CH * LDG];
    using v_t = uint16_t[2][CH * LDV];
    using s_t = uint16_t[CH * LDSS];
    using x_t = u32x4[XT::LDS_BYTES / 16];
    using st_t = float[2][NW][CH][2];   // (m, L) per job (0: keys, 1: queries), wave, position
    using di_t = float[DPARTS][CH];     // partial sums of Gq Z over 16 components each
    using dp_t = float[2][CH];          // S row sums of key block 0 and 1
    using z_t = float[Kp];
    using vote_t = int[NW];
    static constexpr size_t o_gq = 0, o_gk = lds_align(o_gq + sizeof(g_t)), o_vs = lds_align(o_gk + sizeof(g_t)),
                            o_ss = lds_align(o_vs + sizeof(v_t)), o_xq = lds_align(o_ss + sizeof(s_t)),
                            o_xk = lds_align(o_xq + sizeof(x_t)), o_st = lds_align(o_xk + sizeof(x_t)),
                            o_di = lds_align(o_st + sizeof(st_t)), o_dp = lds_align(o_di + sizeof(di_t)),
                            o_zs = lds_align(o_dp + sizeof(dp_t)), o_vote = lds_align(o_zs + sizeof(z_t)),
                            bytes = lds_align(o_vote + sizeof(vote_t));
};

// mode 0: the whole forward (segments 0 .. G-2 aggregate and publish first, every segment
// waits for the aggregates before it, then scans); mode 1: aggregates only (grid G-1 segments);
// mode 2: scans only, the aggregates written by an earlier launch (no waits).
template <int DR, int VT>
__global__ void __launch_bounds__(512)
    wide_causal_kernel(const uint16_t* __restrict__ XQ, const uint16_t* __restrict__ XK, const uint16_t* __restrict__ V,
                       int64_t N, int H, int64_t seg, int G, Mixture mx, float* __restrict__ aggregates,
                       uint64_t* __restrict__ flags, uint64_t token, uint32_t wait_limit, int mode, float eps,
                       uint16_t* __restrict__ O, const float* __restrict__ state_in, float* __restrict__ state_out,
                       uint32_t* __restrict__ err) {
    using LY = WideLds<DR, VT>;
    constexpr int Kp = LY::Kp, DV = LY::DV, CH = LY::CH, NW = LY::NW, NT = LY::NT;
    constexpr int LDG = LY::LDG, LDV = LY::LDV, LDSS = LY::LDSS;
    constexpr int KT16 = Kp / 16;   // 16-row component tiles of the memory
    constexpr int C16 = DV / 16;    // 16-wide value column tiles: wave w < C16 owns tile w
    constexpr int E = Kp * (DV + 1);
    constexpr int VCHUNKS = CH * DV / 8, VCH = (VCHUNKS + NT - 1) / NT;
    constexpr bool VEVEN = VCHUNKS % NT == 0;
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
    int* vote = reinterpret_cast<int*>(smem + LY::o_vote);

    const int wave = wave_id(), l = threadIdx.x & 63, lh = l >> 5, j = l & 31, g4 = l >> 4, i16 = l & 15;
    const int64_t p = blockIdx.y;
    const int s = blockIdx.x, h = int(p % H);
    const int64_t lo = int64_t(s) * seg, hi = min<int64_t>(lo + seg, N), rows = hi - lo;
    float* agg = aggregates + size_t(p) * G * E;
    uint64_t* fl = flags + size_t(p) * G;
    const size_t SE = size_t(mx.K) * (DV + 1);  // one problem's carried memory
    const bool owns_cols = wave < C16;

    WaveParams<DR, 1> P;  // component tile `wave`
    P.compute(mx, h, wave);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(XQ + (size_t(p) * N + lo) * DR, rows * DR * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(XK + (size_t(p) * N + lo) * DR, rows * DR * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + (size_t(p) * N + lo) * DV, rows * DV * 2);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + (size_t(p) * N + lo) * DV, rows * DV * 2);
    // S tile (query block 0, key block 1) lies above the diagonal: zero for good
    for (int c = threadIdx.x; c < CH * LDSS / 8; c += NT) reinterpret_cast<u32x4*>(Ss)[c] = u32x4{0u, 0u, 0u, 0u};

    f32x4 mem[KT16];
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
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

    // The chunk loop over the segment.  AGG: the key side alone (aggregate); otherwise the scan.
    // pre() runs once the first loads are in flight, before anything reads the memory.
    auto run = [&](auto agg_tag, auto&& pre) __attribute__((always_inline)) {
        constexpr bool AGG = decltype(agg_tag)::value;
        constexpr int JOBS = AGG ? 1 : 2;  // score jobs: 0 keys, 1 queries
        const int64_t C = (rows + CH - 1) / CH;
        XT xq, xk;
        f32x16 acc[2][1];
        float zdummy[1][16];
        float sm_m[2], sm_L[2];
        auto scores_next = [&]() __attribute__((always_inline)) {  // from the x tiles in LDS
            scores_lds<DR, 1>(P, XtK, 0, acc[0]);
            if (!AGG) scores_lds<DR, 1>(P, XtQ, 0, acc[1]);
        };
        auto softmax_local = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int jb = 0; jb < JOBS; ++jb) {
                float D;
                local_softmax<1, false>(acc[jb], zdummy, sm_m[jb], sm_L[jb], D);
                if (lh == 0) {
                    st[jb][wave][j][0] = sm_m[jb];
                    st[jb][wave][j][1] = sm_L[jb];
                }
            }
        };
        // responsibilities of the chunk starting at row0 into buffer b (after the statistics)
        auto store_gamma = [&](int64_t row0, int b) __attribute__((always_inline)) {
            const bool valid = row0 + j < rows;
#pragma unroll
            for (int jb = 0; jb < JOBS; ++jb) {
                float mm = -INFINITY;
#pragma unroll
                for (int w = 0; w < NW; ++w) mm = fmaxf(mm, st[jb][w][j][0]);
                float Lt = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w) Lt = fmaf(st[jb][w][j][1], __builtin_amdgcn_exp2f(st[jb][w][j][0] - mm), Lt);
                float scale = __builtin_amdgcn_exp2f(sm_m[jb] - mm) * __builtin_amdgcn_rcpf(Lt);
                if (!valid) scale = 0.0f;  // positions past the segment: no responsibility
                store_gamma_lds<1>(acc[jb], scale, jb == 0 ? Gk[b] : Gq[b], LDG, j, wave);
            }
        };

        // ---- prologue: V(0) and x(0) loaded, pre(), V(0) and x(0) into LDS, responsibilities
        // of chunk 0 into buffer 0, x(1) into LDS; V(1) and x(2) in flight
        load_v(0);
        if (!AGG) xq.load(rq, 0);
        xk.load(rk, 0);
        pre();
        commit_v(Vs[0]);
        load_v(CH);
        if (!AGG) xq.commit(XtQ);
        xk.commit(XtK);
        if (!AGG) xq.load(rq, CH);
        xk.load(rk, CH);
        __syncthreads();
        scores_next();
        softmax_local();
        __syncthreads();  // statistics published; x(0) consumed
        store_gamma(0, 0);
        if (!AGG) xq.commit(XtQ);
        xk.commit(XtK);
        if (!AGG) xq.load(rq, 2 * CH);
        xk.load(rk, 2 * CH);
        __syncthreads();

        auto chunk = [&](const int64_t c, const int b) __attribute__((always_inline)) {
            const int64_t nc = c * CH;
            // ================= region 1
            __builtin_amdgcn_s_setprio(1);
            f32x4 o[2];
            if constexpr (!AGG) {
                // S^T tiles (rows keys, columns queries) of blocks (q, k) = (0,0), (1,0), (1,1)
                if (wave >= NW - 3) {
                    const int t = wave - (NW - 3), qb = t > 0 ? 1 : 0, kb = t > 1 ? 1 : 0;
                    f32x4 sacc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int ks = 0; ks < Kp / 32; ++ks)
                        sacc = mfma16(*reinterpret_cast<const bf16x8*>(Gk[b] + (kb * 16 + i16) * LDG + 32 * ks + 8 * g4),
                                      *reinterpret_cast<const bf16x8*>(Gq[b] + (qb * 16 + i16) * LDG + 32 * ks + 8 * g4),
                                      sacc);
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
                {  // partial sums of Gq(c) Z over components 16 part .. + 15
                    const int row = threadIdx.x & 31, part = threadIdx.x >> 5;
                    const u32x4* gr = reinterpret_cast<const u32x4*>(Gq[b] + row * LDG + 16 * part);
                    float d = 0.0f;
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const u32x4 gv = gr[h2];
                        const float4 z0 = *reinterpret_cast<const float4*>(Zs + 16 * part + 8 * h2);
                        const float4 z1 = *reinterpret_cast<const float4*>(Zs + 16 * part + 8 * h2 + 4);
                        d = fmaf(__uint_as_float(gv[0] << 16), z0.x, d);
                        d = fmaf(__uint_as_float(gv[0] & 0xffff0000u), z0.y, d);
                        d = fmaf(__uint_as_float(gv[1] << 16), z0.z, d);
                        d = fmaf(__uint_as_float(gv[1] & 0xffff0000u), z0.w, d);
                        d = fmaf(__uint_as_float(gv[2] << 16), z1.x, d);
                        d = fmaf(__uint_as_float(gv[2] & 0xffff0000u), z1.y, d);
                        d = fmaf(__uint_as_float(gv[3] << 16), z1.z, d);
                        d = fmaf(__uint_as_float(gv[3] & 0xffff0000u), z1.w, d);
                    }
                    den_ip[part][row] = d;
                }
            }
            scores_next();  // chunk c+1 (x tiles in LDS)
            softmax_local();
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();  // B_Q
            // ================= region 2
            store_gamma(nc + CH, b ^ 1);
            if constexpr (!AGG) {
                // inter part: O^T = Vt^T Gq^T over the memory before this chunk (hi + lo bf16)
                if (owns_cols) {
                    o[0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    o[1] = o[0];
#pragma unroll
                    for (int m2 = 0; m2 < Kp / 32; ++m2) {
                        u32x4 ah, al;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int v0 = 2 * q, v1 = 2 * q + 1;
                            const float x0 = mem[2 * m2 + (v0 >> 2)][v0 & 3];
                            const float x1 = mem[2 * m2 + (v1 >> 2)][v1 & 3];
                            const uint32_t hb = pack_bf16x2(x0, x1);
                            ah[q] = hb;
                            al[q] = pack_bf16x2(x0 - __uint_as_float(hb << 16), x1 - __uint_as_float(hb & 0xffff0000u));
                        }
#pragma unroll
                        for (int t16 = 0; t16 < 2; ++t16) {
                            const uint16_t* gq = Gq[b] + (t16 * 16 + i16) * LDG + 32 * m2 + 4 * g4;
                            const u32x2 b0 = *reinterpret_cast<const u32x2*>(gq);
                            const u32x2 b1 = *reinterpret_cast<const u32x2*>(gq + 16);
                            const bf16x8 bb = __builtin_bit_cast(bf16x8, u32x4{b0[0], b0[1], b1[0], b1[1]});
                            o[t16] = mfma16(__builtin_bit_cast(bf16x8, ah), bb, o[t16]);
                            o[t16] = mfma16(__builtin_bit_cast(bf16x8, al), bb, o[t16]);
                        }
                    }
                }
            }
            // memory update with chunk c: Vt += Gk^T Vc (own columns), Z += Gk^T 1 (tiles wave, wave + 8)
            f32x4 zt[2];
            {
                if (owns_cols) {
                    const bf16x8 bv = read_colfrag16(Vs[b], LDV, 0, 16 * wave);
#pragma unroll
                    for (int kt = 0; kt < KT16; ++kt) mem[kt] = mfma16(read_colfrag16(Gk[b], LDG, 0, 16 * kt), bv, mem[kt]);
                }
#pragma unroll
                for (int zi = 0; zi < 2; ++zi)
                    zt[zi] = mfma16(read_colfrag16(Gk[b], LDG, 0, 16 * (wave + NW * zi)), ones,
                                    f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            }
            if constexpr (!AGG) {
                if (owns_cols) {
                    const bf16x8 av = read_colfrag16(Vs[b], LDV, 0, 16 * wave);
#pragma unroll
                    for (int t16 = 0; t16 < 2; ++t16) {
                        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(Ss + (t16 * 16 + i16) * LDSS + 8 * g4);
                        o[t16] = mfma16(av, bb, o[t16]);
                    }
#pragma unroll
                    for (int t16 = 0; t16 < 2; ++t16) {
                        const int q = t16 * 16 + i16;
                        float den = eps + den_part[0][q];
                        if (t16 == 1) den += den_part[1][q];
#pragma unroll
                        for (int pt = 0; pt < LY::DPARTS; ++pt) den += den_ip[pt][q];
                        const float rden = __builtin_amdgcn_rcpf(den);
                        // positions past the segment fall outside the resource and are dropped
                        buf_store8(ro, uint32_t(((nc + q) * DV + 16 * wave + 4 * g4) * 2),
                                   u32x2{pack_bf16x2(o[t16][0] * rden, o[t16][1] * rden),
                                         pack_bf16x2(o[t16][2] * rden, o[t16][3] * rden)});
                    }
                }
            }
            if (i16 == 0)
#pragma unroll
                for (int zi = 0; zi < 2; ++zi)
#pragma unroll
                    for (int r = 0; r < 4; ++r) Zs[16 * (wave + NW * zi) + 4 * g4 + r] += zt[zi][r];
            commit_v(Vs[b ^ 1]);  // V(c+1)
            load_v(nc + 2 * CH);
            if (!AGG) xq.commit(XtQ);  // x(c+2)
            xk.commit(XtK);
            if (!AGG) xq.load(rq, nc + 3 * CH);
            xk.load(rk, nc + 3 * CH);
            __syncthreads();  // B_P
        };
        for (int64_t c = 0; c < C; ++c) chunk(c, int(c & 1));
    };

    // ---- 1. the segment's aggregate (not needed for the last segment)
    const bool aggregate = mode == 1 || (mode == 0 && s + 1 < G);
    if (aggregate) {
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt) mem[kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int k = threadIdx.x; k < Kp; k += NT) Zs[k] = 0.0f;
        run(std::true_type(), [] {});
        // VtT [DV][Kp] then Z [Kp], device-coherent for the consumers in this launch
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(agg + size_t(s) * E, int64_t(E) * 4);
        if (owns_cols)
#pragma unroll
            for (int kt = 0; kt < KT16; ++kt)
                buf_store16_dev(ra, uint32_t(((16 * wave + i16) * Kp + 16 * kt + 4 * g4) * 4),
                                u32x4{__float_as_uint(mem[kt][0]), __float_as_uint(mem[kt][1]),
                                      __float_as_uint(mem[kt][2]), __float_as_uint(mem[kt][3])});
        if (threadIdx.x < Kp / 4) {
            const float4 z = *reinterpret_cast<const float4*>(Zs + 4 * threadIdx.x);
            buf_store16_dev(ra, uint32_t((Kp * DV + 4 * threadIdx.x) * 4),
                            u32x4{__float_as_uint(z.x), __float_as_uint(z.y), __float_as_uint(z.z), __float_as_uint(z.w)});
        }
        publish_token(fl + s, token);  // its barrier also ends every use of the aggregate's LDS
        if (mode == 1) return;
    }

    // ---- 2. + 3. the starting memory, then the scan
    bool ok = true;
    {  // the carried memory [K][DV + 1] (row k: Vt_k then Z_k) or zeros; rows k >= K lie past the
       // resource's end and read as zero
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(state_in ? state_in + p * SE : nullptr,
                                                    state_in ? int64_t(SE) * 4 : 0);
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt) mem[kt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (state_in && owns_cols)
#pragma unroll
            for (int kt = 0; kt < KT16; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    mem[kt][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        rs, uint32_t(((16 * kt + 4 * g4 + r) * (DV + 1) + 16 * wave + i16) * 4), 0, 0));
        if (threadIdx.x < Kp / 4)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Zs[4 * threadIdx.x + r] =
                    state_in ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                   rs, uint32_t(((4 * threadIdx.x + r) * (DV + 1) + DV) * 4), 0, 0))
                             : 0.0f;
    }
    run(std::false_type(), [&] {
        if (mode == 0) ok = wait_tokens(fl, s, token, wait_limit);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(agg, int64_t(s) * int64_t(E) * 4);
        for (int gs = 0; gs < s; ++gs) {  // increasing segment order
            const uint32_t a = uint32_t(size_t(gs) * E * 4);
            if (owns_cols)
#pragma unroll
                for (int kt = 0; kt < KT16; ++kt) {
                    const u32x4 v = buf_load16_dev(ra, a + uint32_t(((16 * wave + i16) * Kp + 16 * kt + 4 * g4) * 4));
#pragma unroll
                    for (int r = 0; r < 4; ++r) mem[kt][r] += __uint_as_float(v[r]);
                }
            if (threadIdx.x < Kp / 4) {
                const u32x4 v = buf_load16_dev(ra, a + uint32_t((Kp * DV + 4 * threadIdx.x) * 4));
#pragma unroll
                for (int r = 0; r < 4; ++r) Zs[4 * threadIdx.x + r] += __uint_as_float(v[r]);
            }
        }
    });
    float* so = (state_out && s == G - 1) ? state_out + p * SE : nullptr;
    if (so) {  // the memory after the last position, same layout; rows k >= K are dropped
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(so, int64_t(SE) * 4);
        if (owns_cols)
#pragma unroll
            for (int kt = 0; kt < KT16; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mem[kt][r]), rs,
                                                          uint32_t(((16 * kt + 4 * g4 + r) * (DV + 1) + 16 * wave + i16) * 4),
                                                          0, 0);
        if (threadIdx.x < Kp / 4)  // Zs is complete after B_P of the last chunk
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Zs[4 * threadIdx.x + r]), rs,
                                                      uint32_t(((4 * threadIdx.x + r) * (DV + 1) + DV) * 4), 0, 0);
    }
    // waves poll on their own: agree on the outcome before acting on it
    ok = workgroup_all(ok, vote);
    if (!ok) {  // the starting memory was never complete: make that visible in the outputs and to the host
        __builtin_amdgcn_s_waitcnt(0);  // the scan's own stores of these rows land first
        __syncthreads();
        uint16_t* op = O + (size_t(p) * N + lo) * DV;
        for (int64_t e = threadIdx.x; e < rows * DV; e += NT) op[e] = 0x7fc0u;
        if (so)
            for (size_t e = threadIdx.x; e < SE; e += NT) so[e] = __builtin_nanf("");
        if (threadIdx.x == 0) atomicOr(err, kDevErrTimeout);
    }
}

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
    uint32_t* err = nullptr;
    hipError_t e = device_error_word(&err);
    if (e != hipSuccess) return e;
    return bf::with_wide(int(p.dr), int(p.dv / 32), [&](auto D, auto W) {
        constexpr int DR = decltype(D)::value, VT = decltype(W)::value;
        const bool single = single_launch_enabled();
        const uint64_t token = launch_token();
        auto launch = [&](unsigned grid_x, int mode) {
            GMA_LAUNCH(mode == 1 ? "bf16_causal_aggregate" : "bf16_causal", (bf::wide_causal_kernel<DR, VT>),
                       dim3(grid_x, unsigned(p.P)), dim3(512), 0, st, static_cast<const uint16_t*>(XQ),
                       static_cast<const uint16_t*>(XK), static_cast<const uint16_t*>(V), p.N, int(p.H), p.seg,
                       int(p.G), mx, aggregates, flags, token, wait_limit(), mode, eps, static_cast<uint16_t*>(O),
                       state_in, state_out, err);
            return hipGetLastError();
        };
        if (single) return launch(unsigned(p.G), 0);
        if (p.G > 1) {  // the aggregates in a launch of their own, then the scans without waits
            hipError_t r = launch(unsigned(p.G - 1), 1);
            if (r != hipSuccess) return r;
        }
        return launch(unsigned(p.G), 2);
    });
}

}  // namespace gma
