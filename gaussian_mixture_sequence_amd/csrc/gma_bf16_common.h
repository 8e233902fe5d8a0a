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

// Index of this wave in its workgroup, as a wave-uniform (scalar) value: without the
// readfirstlane the compiler cannot prove uniformity, keeps everything derived from it in
// VGPRs and turns buffer loads whose resource depends on it into per-lane waterfall loops.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)); }

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

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// x^2 split into hi + lo bf16 for a packed pair of bf16 values (exact: the square of an
// 8-bit significand has 16 bits, so x^2 - hi has at most 8 and is a bf16 value).
__device__ __forceinline__ u32x2 square_split_pair(uint32_t x) {
    const float x0 = __uint_as_float(x << 16), x1 = __uint_as_float(x & 0xffff0000u);
    const float s0 = x0 * x0, s1 = x1 * x1;
    const uint32_t hi = pack_bf16x2(s0, s1);
    return u32x2{hi, pack_bf16x2(s0 - __uint_as_float(hi << 16), s1 - __uint_as_float(hi & 0xffff0000u))};
}

__device__ __forceinline__ void square_split(bf16x8 x, bf16x8& hi, bf16x8& lo) {
    const u32x4 xv = __builtin_bit_cast(u32x4, x);
    u32x4 h, l;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u32x2 hl = square_split_pair(xv[q]);
        h[q] = hl[0];
        l[q] = hl[1];
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// ---- buffer access: a resource covering [base, base + bytes); loads past the end
// return zeros and stores past the end are dropped, so tiles need no guard branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int32_t n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : int32_t(bytes));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), r, off, 0, 0);
}

// Device-coherent accesses (cache policy SC1) for data that another workgroup of the same
// launch wrote or reads: they are performed at the coherence point every XCD shares, so no
// cache-wide write-back or invalidate is needed around the hand-off.  Full 16-byte lanes
// of a coalesced wave keep these at whole-line granularity.
constexpr int kCoherent = 16;
__device__ __forceinline__ u32x4 buf_load16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}
__device__ __forceinline__ void buf_store16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), r, off, 0,
                                           kCoherent);
}
__device__ __forceinline__ void buf_store8_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v), r, off, 0,
                                          kCoherent);
}

// ---- a tile of ROUND routing vectors, split once into the score MFMA's B fragments
// (x, x^2 hi, x^2 lo) and shared through LDS by every wave that needs it.
// Global loads are fully coalesced: thread t fetches 16-byte chunk t (+ NTHREADS, ...) of
// the row-major [ROUND][DR] tile, so every wave instruction reads whole 128-byte lines
// (partial-line reads of the same line from several waves make L2 fetch it again).
// LDS layout: fragment fi = (token subtile ts, k-step ks) holds, for each piece
// (x, x^2 hi, x^2 lo), 64 lane slots of 16 bytes; lane (lh, j) of the MFMA B operand
// needs x[ts * 32 + j][16 ks + 8 lh .. + 7].  Pieces are FS = 68 slots apart (4 of
// padding) and lane slots are swizzled (slot = lane ^ 2 lh): with those, both the
// scattered commit of a wave's chunks and the fragment reads are bank-conflict free
// for d_r = 64 (at most 2-way otherwise).
template <int DR, int ROUND, int NTHREADS>
struct XTile {
    static constexpr int KS = DR / 16;
    static constexpr int CPR = DR / 8;  // 16-byte chunks per row
    static constexpr int CHUNKS = ROUND * CPR;
    static constexpr int PER = (CHUNKS + NTHREADS - 1) / NTHREADS;
    static constexpr bool EVEN = CHUNKS % NTHREADS == 0;
    static constexpr int FRAGS = (ROUND / 32) * KS;
    static constexpr int FS = 68;
    static constexpr int LDS_BYTES = FRAGS * 3 * FS * 16;
    u32x4 r[PER];

    // the tile that starts `row0` rows into the resource
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int64_t row0) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = threadIdx.x + u * NTHREADS;
            r[u] = (EVEN || c < CHUNKS) ? buf_load16(rs, uint32_t((row0 * DR + int64_t(c) * 8) * 2))
                                        : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void commit(u32x4* lds) const {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = threadIdx.x + u * NTHREADS;
            if (EVEN || c < CHUNKS) {
                const int row = c / CPR, cc = c - row * CPR;
                const int lh = cc & 1;
                const int slot = (32 * lh + (row & 31)) ^ (2 * lh);
                u32x4 h, lo;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x2 hl = square_split_pair(r[u][q]);
                    h[q] = hl[0];
                    lo[q] = hl[1];
                }
                u32x4* f = lds + ((row >> 5) * KS + (cc >> 1)) * 3 * FS + slot;
                f[0] = r[u];
                f[FS] = h;
                f[2 * FS] = lo;
            }
        }
    }
};

// ---- a row-major [ROWS][DR] bf16 tile staged through LDS unsplit, with the same coalesced
// loads; rows are padded to DR + 8 elements, which makes the 16-byte row-fragment reads
// bank-conflict free.  Used where one wave alone consumes each token subtile (it splits
// its own fragments in registers).
template <int DR, int ROWS, int NTHREADS>
struct RawTile {
    static constexpr int CPR = DR / 8;
    static constexpr int CHUNKS = ROWS * CPR;
    static constexpr int PER = (CHUNKS + NTHREADS - 1) / NTHREADS;
    static constexpr bool EVEN = CHUNKS % NTHREADS == 0;
    static constexpr int LD = DR + 8;
    static constexpr int LDS_BYTES = ROWS * LD * 2;
    u32x4 r[PER];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int64_t row0) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = threadIdx.x + u * NTHREADS;
            r[u] = (EVEN || c < CHUNKS) ? buf_load16(rs, uint32_t((row0 * DR + int64_t(c) * 8) * 2))
                                        : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void commit(u32x4* lds) const {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = threadIdx.x + u * NTHREADS;
            if (EVEN || c < CHUNKS) {
                const int row = c / CPR, cc = c - row * CPR;
                *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(lds) + row * LD + cc * 8) = r[u];
            }
        }
    }
};

// B fragments (one per k-step) of 32-row subtile `sub` of a RawTile in LDS, unsplit.
template <int DR>
__device__ __forceinline__ void raw_frags(const u32x4* lds, int sub, bf16x8 (&xs)[DR / 16]) {
    const int l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const uint16_t* row = reinterpret_cast<const uint16_t*>(lds) + (sub * 32 + j) * (DR + 8) + 8 * lh;
#pragma unroll
    for (int ks = 0; ks < DR / 16; ++ks) xs[ks] = *reinterpret_cast<const bf16x8*>(row + 16 * ks);
}

// B fragments of token subtile `ts` from an XTile in LDS.
template <int DR>
__device__ __forceinline__ void xtile_frags(const u32x4* lds, int ts, int ks, bf16x8& x, bf16x8& x2h, bf16x8& x2l) {
    constexpr int FS = 68;
    const int l = threadIdx.x & 63;
    const u32x4* f = lds + ((ts * (DR / 16) + ks) * 3) * FS + (l ^ (2 * (l >> 5)));
    x = __builtin_bit_cast(bf16x8, f[0]);
    x2h = __builtin_bit_cast(bf16x8, f[FS]);
    x2l = __builtin_bit_cast(bf16x8, f[2 * FS]);
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
// token subtile (each holds KT / CS component tiles of the parameter planes in registers),
// TS = NW / CS token subtiles of 32 tokens are processed side by side.  NW = max(KT, 4) waves
// per workgroup in either phase.  The write phase (and the scan, the responsibilities) take
// one component tile per wave: its accumulators for the memory leave no registers for a
// second.  The read phase (READ) takes two per wave where d_r <= 32 (the planes of two tiles
// then fit in 64 VGPRs), which halves its rounds' fixed costs.
template <int DR, int KT, bool READ = false>
struct Split {
    static constexpr int NW = KT > 4 ? KT : 4;  // waves per workgroup
    static constexpr int CSR0 = (KT * DR) / 64 > KT / 2 ? (KT * DR) / 64 : KT / 2;
    static constexpr int CS = READ ? (CSR0 < 1 ? 1 : (CSR0 > KT ? KT : CSR0)) : KT;
    static constexpr int CTW = KT / CS;         // component tiles per wave
    static constexpr int TS = NW / CS;          // token subtiles per round
    static constexpr int ROUND = 32 * TS;       // tokens per round
    static constexpr int KS = DR / 16;          // k-steps of the d contraction
};

constexpr size_t lds_align(size_t x) { return (x + 15) & ~size_t(15); }

// Waves per SIMD a 4-wave workgroup of `lds` bytes can keep resident (160 KiB of LDS per
// CU): kernels declare it so the register allocator keeps within that occupancy.
constexpr int waves_for_lds(size_t lds) { return lds <= 80 * 1024 ? 2 : 1; }

// ---- hand-off between workgroups of one launch
// Data handed to another workgroup is written and read with the device-coherent accesses
// above.  A workgroup publishes a 64-bit word once every such store of all its waves has
// completed; waiters poll until each word they need holds the launch's token, a per-call
// random value, so stale words from earlier calls never match.  Waiters only depend on
// workgroups dispatched no later than themselves or alongside them, and the poll is
// bounded (`limit` polls, a launch argument): on time-out the waiter reports failure
// instead of hanging.

__device__ __forceinline__ void publish_token(uint64_t* flag, uint64_t token) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
    __syncthreads();                // ... and those of every wave of the workgroup
    if (threadIdx.x == 0) __hip_atomic_store(flag, token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// AND of a per-wave flag over the workgroup, through NW ints of LDS that no wave uses any
// more (`scratch`); every wave gets the same result.
__device__ __forceinline__ bool workgroup_all(bool v, int* scratch) {
    __syncthreads();  // scratch free
    if ((threadIdx.x & 63) == 0) scratch[wave_id()] = v ? 1 : 0;
    __syncthreads();
    bool r = true;
    for (int w = 0; w < int(blockDim.x >> 6); ++w) r = r && scratch[w] != 0;
    return r;
}

// Every wave polls flags[0 .. n) itself (no LDS, no barrier); true when all hold `token`
// within `limit` polls.
__device__ __forceinline__ bool wait_tokens(const uint64_t* flags, int n, uint64_t token, uint32_t limit) {
    const int l = threadIdx.x & 63;
    bool done = false;
    for (uint32_t it = 0; it < limit; ++it) {
        bool mine = true;
        for (int i = l; i < n; i += 64)
            mine = mine && (__hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == token);
        done = __all(mine);
        if (done) break;
        __builtin_amdgcn_s_sleep(2);
    }
    // The polls are relaxed atomics: keep the compiler from moving the caller's reads of the
    // handed-off data above them (the hardware issues those reads only after the polls'
    // values have returned, and the data reached the coherence point before the word did).
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return done;
}

// Mixture parameters of every head: mu, s2 [H][K][d_r] fp32 row-major, pi [H][K] fp32.
struct Mixture {
    const float* mu;
    const float* s2;
    const float* pi;
    int K;
};

// One head's score operands built once per workgroup (Gaussian Mixture Attention, Eq. 16
// with the square expanded, in log2 units):
//   a = log2(e) mu / sigma2,  b = -log2(e) / (2 sigma2),  each as a bf16 hi + lo pair,
//   c = log2 pi - (sum_d log2 sigma2 + log2(e) mu^2 / sigma2) / 2   (fp32).
// Every thread fetches whole 16-byte chunks of mu and sigma2 rows (coalesced), computes the
// planes of its chunks' 4 dims, and stores them in LDS in MFMA A-fragment order:
//   planes [KP/32][DR/16][4: a_hi, a_lo, b_hi, b_lo][64 lanes] of 16 bytes
// followed by c [KP] fp32.  Lane (lh, j) of component tile ct, k-step ks holds component
// 32 ct + j, dims 16 ks + 8 lh .. + 7, so each wave then loads its fragments with one
// conflict-free 16-byte read per plane (WaveParams::read_planes).  Each (component, dim)
// pair is computed once per workgroup, not once per wave that needs it.  Components k >= K
// (padding up to KP) get zero planes and c = -inf, so their responsibility is exactly 0.
// sigma2 must be a positive normal float.
template <int DR, int KP, int NT>
struct PlaneBuilder {
    static constexpr int KT = KP / 32, KS = DR / 16;
    static constexpr int CPR = DR / 4;  // 16-byte chunks per parameter row
    static constexpr int CHUNKS = KP * CPR, PER = (CHUNKS + NT - 1) / NT;
    static constexpr bool EVEN = CHUNKS % NT == 0;
    static constexpr int PLANE_BYTES = KT * KS * 4 * 64 * 16;
    static constexpr int LDS_BYTES = PLANE_BYTES + KP * 4;
    static_assert(NT % CPR == 0 && CPR <= 64, "a row's chunks must sit in consecutive lanes of one wave");
    float4 m[PER], v[PER];
    float pk[PER];

    // Raw parameters of this thread's chunks (rows past K repeat row K - 1), fetched apart
    // from the arithmetic so a kernel can put its first tile loads in flight before it
    // waits for them.
    __device__ __forceinline__ void load(const Mixture& mx, int h) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = threadIdx.x + u * NT;
            if (EVEN || c < CHUNKS) {
                const int row = c / CPR, col = c - row * CPR;
                const size_t kr = size_t(h) * mx.K + (row < mx.K ? row : mx.K - 1);
                m[u] = *reinterpret_cast<const float4*>(mx.mu + kr * DR + 4 * col);
                v[u] = *reinterpret_cast<const float4*>(mx.s2 + kr * DR + 4 * col);
                pk[u] = mx.pi[kr];
            }
        }
    }

    // Planes and constants into `lds` (LDS_BYTES); the caller synchronises before reading.
    __device__ __forceinline__ void build(char* lds, int K) const {
        const float L2E = 1.4426950408889634f;
        float* cst = reinterpret_cast<float*>(lds + PLANE_BYTES);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = threadIdx.x + u * NT;
            if (EVEN || c < CHUNKS) {  // uniform over the CPR lanes of a row
                const int row = c / CPR, col = c - row * CPR;
                const bool valid = row < K;
                const float mm[4] = {m[u].x, m[u].y, m[u].z, m[u].w};
                const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                float a[4], b[4], csum = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float inv2 = __builtin_amdgcn_rcpf(valid ? vv[e] : INFINITY) * L2E;
                    a[e] = mm[e] * inv2;
                    b[e] = -0.5f * inv2;
                    csum += __builtin_amdgcn_logf(vv[e]) + mm[e] * a[e];
                }
                uint32_t w[4][2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint32_t ah = pack_bf16x2(a[2 * q], a[2 * q + 1]);
                    const uint32_t bh = pack_bf16x2(b[2 * q], b[2 * q + 1]);
                    w[0][q] = ah;
                    w[1][q] = pack_bf16x2(a[2 * q] - __uint_as_float(ah << 16), a[2 * q + 1] - __uint_as_float(ah & 0xffff0000u));
                    w[2][q] = bh;
                    w[3][q] = pack_bf16x2(b[2 * q] - __uint_as_float(bh << 16), b[2 * q + 1] - __uint_as_float(bh & 0xffff0000u));
                }
                const int d0 = 4 * col, ct = row >> 5, j = row & 31;
                const int ks = d0 >> 4, lh = (d0 >> 3) & 1, half = (d0 >> 2) & 1;
                char* dst = lds + (size_t((ct * KS + ks) * 4) * 64 + 32 * lh + j) * 16 + half * 8;
#pragma unroll
                for (int pl = 0; pl < 4; ++pl) *reinterpret_cast<u32x2*>(dst + pl * 64 * 16) = u32x2{w[pl][0], w[pl][1]};
#pragma unroll
                for (int o = CPR / 2; o >= 1; o >>= 1) csum += __shfl_xor(csum, o, kWave);
                if (col == 0) cst[row] = valid ? __builtin_amdgcn_logf(pk[u]) - 0.5f * csum : -INFINITY;
            }
        }
    }
};

// Parameter planes of one wave: 4 bf16 planes (a_hi, a_lo, b_hi, b_lo) for its CTW
// component tiles, as MFMA A fragments, and the score constants in D-row order.
template <int DR, int CTW>
struct WaveParams {
    bf16x8 w[CTW][DR / 16][4];
    float c[CTW][16];

    // Raw parameters behind this lane's fragments, fetched apart from the arithmetic so a
    // kernel can put its first tile loads in flight before it waits for them.
    struct Raw {
        float4 m[CTW][DR / 16][2], v[CTW][DR / 16][2];
        float pk[CTW];
    };

    // Lane (lh, j) owns component 32 tile + j and dims 16 ks + 8 lh .. + 7 of every k-step,
    // which is exactly its A fragment.  mu, s2: [H][K][DR], pi: [H][K]; h: head; ct0: first
    // component tile of this wave.  Lanes of padded components (k >= K) read row K - 1.
    __device__ __forceinline__ static void fetch(const Mixture& mx, int h, int ct0, Raw& r) {
        const int l = threadIdx.x & 63, lh = l >> 5, K = mx.K;
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int k = (ct0 + ct) * 32 + (l & 31);
            const int kr = k < K ? k : K - 1;
            const size_t row = (size_t(h) * K + kr) * DR + 8 * lh;
#pragma unroll
            for (int ks = 0; ks < DR / 16; ++ks)
#pragma unroll
                for (int h4 = 0; h4 < 2; ++h4) {
                    r.m[ct][ks][h4] = *reinterpret_cast<const float4*>(mx.mu + row + 16 * ks + 4 * h4);
                    r.v[ct][ks][h4] = *reinterpret_cast<const float4*>(mx.s2 + row + 16 * ks + 4 * h4);
                }
            r.pk[ct] = mx.pi[size_t(h) * K + kr];
        }
    }

    // This wave's fragments and constants from a PlaneBuilder buffer of KP components.
    template <int KP>
    __device__ __forceinline__ void read_planes(const char* lds, int ct0) {
        const int l = threadIdx.x & 63, lh = l >> 5;
        const u32x4* pl = reinterpret_cast<const u32x4*>(lds);
        const float* cst = reinterpret_cast<const float*>(lds + PlaneBuilder<DR, KP, 64>::PLANE_BYTES);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
#pragma unroll
            for (int ks = 0; ks < DR / 16; ++ks)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w[ct][ks][q] = __builtin_bit_cast(bf16x8, pl[(((ct0 + ct) * (DR / 16) + ks) * 4 + q) * 64 + l]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 cv = *reinterpret_cast<const float4*>(cst + (ct0 + ct) * 32 + 8 * q + 4 * lh);
                c[ct][4 * q + 0] = cv.x;
                c[ct][4 * q + 1] = cv.y;
                c[ct][4 * q + 2] = cv.z;
                c[ct][4 * q + 3] = cv.w;
            }
        }
    }

    // Builds the planes from the mixture parameters (Gaussian Mixture Attention, Eq. 16 with
    // the square expanded, in log2 units):
    //   a = log2(e) mu / sigma2,  b = -log2(e) / (2 sigma2),  each as a bf16 hi + lo pair,
    //   c = log2 pi - (sum_d log2 sigma2 + log2(e) mu^2 / sigma2) / 2   (fp32).
    // Padded components get zero planes (sigma2 taken as +inf) and c = -inf, so their
    // responsibility is exactly 0.  sigma2 must be a positive normal float.
    // Bitwise the same planes and constants as PlaneBuilder::build, so that kernels (and the
    // workgroups of one kernel) that build them either way agree exactly: the same operations per
    // (component, dim), and the constant's sum taken over 4-dim chunks combined in the same tree.
    __device__ __forceinline__ void build(const Raw& r, int K, int ct0) {
        const float L2E = 1.4426950408889634f;
        constexpr int KS = DR / 16, CPR = DR / 4;  // 4-dim chunks per component row
        const int l = threadIdx.x & 63, lh = l >> 5;
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const bool valid = (ct0 + ct) * 32 + (l & 31) < K;
            float part[2 * KS];  // this lane's chunks: chunk 4 ks + 2 lh + h4 at index 2 ks + h4
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 ah, al, bh, bl;
#pragma unroll
                for (int h4 = 0; h4 < 2; ++h4) {
                    const float4 mv = r.m[ct][ks][h4], vv4 = r.v[ct][ks][h4];
                    const float mm[4] = {mv.x, mv.y, mv.z, mv.w};
                    const float vv[4] = {vv4.x, vv4.y, vv4.z, vv4.w};
                    float a[4], b[4], csum = 0.0f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float inv2 = __builtin_amdgcn_rcpf(valid ? vv[e] : INFINITY) * L2E;
                        a[e] = mm[e] * inv2;
                        b[e] = -0.5f * inv2;
                        csum += __builtin_amdgcn_logf(vv[e]) + mm[e] * a[e];
                    }
                    part[2 * ks + h4] = csum;
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const uint32_t hi_a = pack_bf16x2(a[2 * q], a[2 * q + 1]);
                        const uint32_t hi_b = pack_bf16x2(b[2 * q], b[2 * q + 1]);
                        ah[2 * h4 + q] = hi_a;
                        al[2 * h4 + q] = pack_bf16x2(a[2 * q] - __uint_as_float(hi_a << 16),
                                                     a[2 * q + 1] - __uint_as_float(hi_a & 0xffff0000u));
                        bh[2 * h4 + q] = hi_b;
                        bl[2 * h4 + q] = pack_bf16x2(b[2 * q] - __uint_as_float(hi_b << 16),
                                                     b[2 * q + 1] - __uint_as_float(hi_b & 0xffff0000u));
                    }
                }
                w[ct][ks][0] = __builtin_bit_cast(bf16x8, ah);
                w[ct][ks][1] = __builtin_bit_cast(bf16x8, al);
                w[ct][ks][2] = __builtin_bit_cast(bf16x8, bh);
                w[ct][ks][3] = __builtin_bit_cast(bf16x8, bl);
            }
            // all CPR chunk sums of component k: lanes j and j + 32 hold the two halves
            float chunk[CPR];
#pragma unroll
            for (int i = 0; i < 2 * KS; ++i) {
                const float mine = part[i], other = __shfl_xor(part[i], 32, kWave);
                const int ks = i >> 1, h4 = i & 1;
                chunk[4 * ks + 0 + h4] = lh == 0 ? mine : other;
                chunk[4 * ks + 2 + h4] = lh == 0 ? other : mine;
            }
            // the tree of PlaneBuilder's butterfly: level o adds chunk i + o into chunk i
#pragma unroll
            for (int o = CPR / 2; o >= 1; o >>= 1)
#pragma unroll
                for (int i = 0; i < o; ++i) chunk[i] = chunk[i] + chunk[i + o];
            const float ck = valid ? __builtin_amdgcn_logf(r.pk[ct]) - 0.5f * chunk[0] : -INFINITY;
            // D rows of this lane: components 8 q + 4 lh + i of the tile
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) c[ct][4 * q + i] = __shfl(ck, 8 * q + 4 * lh + i);
        }
    }

    __device__ __forceinline__ void compute(const Mixture& mx, int h, int ct0) {
        Raw r;
        fetch(mx, h, ct0, r);
        build(r, mx.K, ct0);
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

// B fragments of the 32-token subtile at row `row0` of a buffer resource over a
// row-major [rows][DR] bf16 tile; rows past the resource's end read as zero.
template <int DR>
__device__ __forceinline__ void load_x_buf(__amdgpu_buffer_rsrc_t rs, int64_t row0, bf16x8 (&xs)[DR / 16]) {
    const int l = threadIdx.x & 63, lh = l >> 5, j = l & 31;
    const uint32_t off = uint32_t(((row0 + j) * DR + 8 * lh) * 2);
#pragma unroll
    for (int ks = 0; ks < DR / 16; ++ks) xs[ks] = __builtin_bit_cast(bf16x8, buf_load16(rs, off + 32 * ks));
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

// Scores of token subtile ts from an XTile in LDS.
template <int DR, int CTW>
__device__ __forceinline__ void scores_lds(const WaveParams<DR, CTW>& P, const u32x4* xt, int ts, f32x16 (&acc)[CTW]) {
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ct][r] = P.c[ct][r];
#pragma unroll
    for (int ks = 0; ks < DR / 16; ++ks) {
        bf16x8 x, x2h, x2l;
        xtile_frags<DR>(xt, ts, ks, x, x2h, x2l);
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
    // a wave whose components are all padding (score -inf) has m = -inf: subtract 0 instead, so
    // that its terms are exp2(-inf) = 0 (and L = 0) rather than NaN; the combine across waves
    // then weighs it by exp2(-inf - m_total) = 0
    const float mref = m == -INFINITY ? 0.0f : m;
    L = 0.0f;
    D = 0.0f;
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float e = __builtin_amdgcn_exp2f(acc[ct][r] - mref);
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

// ---- 16x16x32 MFMA pieces shared by the causal scans (lane l, g = l / 16): A row i = l % 16,
// k = 8 g + v; B col j = l % 16, k = 8 g + v; D row i = 4 g + r, col j = l % 16.
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 fragment with k down a column of a row-major LDS tile:
// lane (g, i) gets tile[row0 + 8 g + v][col0 + i], v = 0..7.  Within each 16-lane group
// the transposing read hands output lane q, element v, the value at offset q % 4 of the
// 8 bytes addressed by source lane 4 v + q / 4; source lane m therefore addresses row
// (m / 4), columns 4 (m % 4) .. + 3.
__device__ __forceinline__ bf16x8 read_colfrag16(const uint16_t* tile, int ld, int row0, int col0) {
    const int l = threadIdx.x & 63;
    const int g = l >> 4, m = l & 15;
    const uint16_t* base = tile + (row0 + 8 * g + (m >> 2)) * ld + col0 + 4 * (m & 3);
    i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
    i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 4 * ld));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

struct ScanStats {
    float m, L, D;
};

// The scans keep the memory as 16x16 MFMA accumulators: mem[cc][kt] holds Vt[k][c] for value
// column c = 16 (wave + cc NW) + l % 16 and components k = 16 kt + 4 (l / 16) + r, r = 0..3
// (Vt^T's D layout), and Z in LDS.  The carried memory of gma_forward_causal_state is
// [K][DV + 1] fp32 (row k: Vt_k then Z_k); components k >= K (padding) are zero.  Thread t
// initialises Z entries ZV t .. ZV t + ZV - 1 (+ ZV NT, ...): the same entries it later adds
// the earlier segments' aggregates to, so no barrier is needed in between.
template <int CPW, int KT16, int NW, int DV, int ZV>
__device__ __forceinline__ void init_memory(f32x4 (&mem)[CPW][KT16], float* Zs, int Kp, int NT,
                                            const float* __restrict__ state, int K) {
    const int l = threadIdx.x & 63, g4 = l >> 4, i16 = l & 15, wave = wave_id();
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt) {
            const int c = (wave + cc * NW) * 16 + i16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = kt * 16 + 4 * g4 + r;
                mem[cc][kt][r] = (state && c < DV && k < K) ? state[size_t(k) * (DV + 1) + c] : 0.0f;
            }
        }
    for (int k0 = threadIdx.x * ZV; k0 < Kp; k0 += NT * ZV)
#pragma unroll
        for (int r = 0; r < ZV; ++r) {
            const int k = k0 + r;
            Zs[k] = (state && k < K) ? state[size_t(k) * (DV + 1) + DV] : 0.0f;
        }
}

// Writes the memory back in the carried layout; Zs must be complete (after a barrier).
template <int CPW, int KT16, int NW, int DV>
__device__ __forceinline__ void store_memory(const f32x4 (&mem)[CPW][KT16], const float* Zs, float* __restrict__ state,
                                             int K) {
    const int l = threadIdx.x & 63, g4 = l >> 4, i16 = l & 15, wave = wave_id();
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt) {
            const int c = (wave + cc * NW) * 16 + i16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = kt * 16 + 4 * g4 + r;
                if (c < DV && k < K) state[size_t(k) * (DV + 1) + c] = mem[cc][kt][r];
            }
        }
    for (int k = threadIdx.x; k < K; k += int(blockDim.x)) state[size_t(k) * (DV + 1) + DV] = Zs[k];
}

}  // namespace bf
}  // namespace gma
