// Short causal calls (decoding): a few positions per (batch, head), continued from a carried
// memory.  Sec. 3.5 of "Gaussian Mixture Attention" defines the prefix memory (Eq. 6b) and the
// output (Eq. 8b); read as a recurrence, the memory after position i is the memory after
// position i-1 plus gammaK_i [V_i | 1].  One workgroup per problem walks its positions in order:
//   s_k   = log pi_k - 1/2 sum_d ( log sigma2_kd + (x_d - mu_kd)^2 / sigma2_kd )   (Eq. 16, direct form,
//                                                                                  fp64 accumulation)
//   gamma = softmax_k(s)                                                          (Eq. 3b)
//   M_k  += gammaK_k [V | 1]   (row k of the memory: Vt_k then Z_k, fp32)         (Eq. 6b)
//   O     = gammaQ Vt / (gammaQ Z + eps)                                           (Eq. 8b)
// The memory stays in LDS between positions.  With a handful of positions there is no tile to
// keep the matrix cores busy; the work per position is a few thousand multiply-adds, so the
// kernel is bound by latency and the score arithmetic is kept exact enough for fp32 I/O.
#include <cmath>
#include <cstdint>

#include "gma_device.h"
#include "gma_internal.h"

namespace gma {

namespace dec {

constexpr int kDecodeThreads = 256;  // >= K (at least one lane per component) and >= d_v + 1

template <typename T>
__device__ __forceinline__ float load_io(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_io<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_io<uint16_t>(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

__device__ __forceinline__ void store_io(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_io(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16_bits(v); }

// Wave-wide reduction of a float through DPP lane moves (VALU, no LDS round trip): pairs and
// quads (quad_perm), then the two halves of each row of 8 and of 16 lanes (half-mirror,
// mirror) combine, so every lane of a row holds the row's result; the four rows are then read
// with readlane and combined in a fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
    v = op(v, dpp<0xB1>(v));   // quad_perm [1, 0, 3, 2]
    v = op(v, dpp<0x4E>(v));   // quad_perm [2, 3, 0, 1]
    v = op(v, dpp<0x141>(v));  // row_half_mirror
    v = op(v, dpp<0x140>(v));  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return op(op(r0, r1), op(r2, r3));
}

// Lanes per component: a power of two, so a component's lanes are consecutive lanes of one
// wave; each takes every TPC-th dim of the score sums.
__host__ __device__ constexpr int lanes_per_component(int K) {
    int k2 = 1;
    while (k2 < K) k2 <<= 1;
    const int tpc = kDecodeThreads / k2;
    return tpc > 64 ? 64 : (tpc < 1 ? 1 : tpc);
}

// Grid (P): problem p = b H + h.  Dynamic LDS: decode_lds_bytes().
template <typename T>
__global__ void __launch_bounds__(kDecodeThreads)
    decode_kernel(const T* __restrict__ XQ, const T* __restrict__ XK, const T* __restrict__ V, int64_t N, int H, int dr,
                  int dv, int K, const float* __restrict__ mu, const float* __restrict__ s2,
                  const float* __restrict__ pi, float eps, const float* __restrict__ state_in,
                  float* __restrict__ state_out, T* __restrict__ O) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    const int64_t p = blockIdx.x;
    const int h = int(p % H), t = threadIdx.x, E = K * (dv + 1);
    float* mem = reinterpret_cast<float*>(lds_raw + 8 * (kDecodeThreads / 64));  // [K][dv + 1] (after 32 spare bytes)
    float* xq = mem + E;                                                     // [dr]
    float* xk = xq + dr;                                                     // [dr]
    float* vv = xk + dr;                                                     // [dv]
    float* gq = vv + dv;                                                     // [K]
    float* gk = gq + K;                                                      // [K]
    float* den = gk + K;                                                     // [1]
    double* sc = reinterpret_cast<double*>(lds_raw + 8 * (kDecodeThreads / 64) +
                                           4 * ((size_t(E) + 2 * dr + dv + 2 * K + 2) & ~size_t(1)));  // [2][K]

    // every first load in flight at once: this thread's element of position 0's routing vectors
    // and values, the carried memory, and its lane's dims of the component's parameters
    float rq = 0.0f, rk = 0.0f, rvv = 0.0f;
    auto fetch = [&](int64_t i) {
        if (t < dr) {
            rq = load_io(XQ, (size_t(p) * N + i) * dr + t);
            rk = load_io(XK, (size_t(p) * N + i) * dr + t);
        }
        if (t < dv) rvv = load_io(V, (size_t(p) * N + i) * dv + t);
    };
    fetch(0);
    // the carried memory: 16-byte pieces, eight of a thread's loads in flight before the first is
    // stored, where the problem's memory starts on a 16-byte boundary (E a multiple of 4)
    const bool vec = (E & 3) == 0;
    if (!state_in) {
        for (int e = t; e < E; e += kDecodeThreads) mem[e] = 0.0f;
    } else if (vec) {
        const float4* sp = reinterpret_cast<const float4*>(state_in + size_t(p) * E);
#pragma unroll 8
        for (int e4 = t; e4 < E / 4; e4 += kDecodeThreads) reinterpret_cast<float4*>(mem)[e4] = sp[e4];
    } else {
#pragma unroll 8
        for (int e = t; e < E; e += kDecodeThreads) mem[e] = state_in[size_t(p) * E + e];
    }

    // component k = t / TPC; its lane j = t % TPC takes dims j, j + TPC, ... (the first MAXD of
    // them kept in registers)
    const int TPC = lanes_per_component(K);
    const int k = t / TPC, j = t - k * TPC;
    const bool comp = k < K;
    const float* mk = mu + (size_t(h) * K + (comp ? k : 0)) * dr;
    const float* vk = s2 + (size_t(h) * K + (comp ? k : 0)) * dr;
    constexpr int MAXD = 16;
    const float pik = comp ? pi[size_t(h) * K + k] : 1.0f;
    float pm[MAXD], pv[MAXD];
#pragma unroll
    for (int u = 0; u < MAXD; ++u) {
        const int d = j + u * TPC;
        const bool in = comp && d < dr;
        pm[u] = in ? mk[d] : 0.0f;
        pv[u] = in ? vk[d] : 1.0f;
    }
    // score constant of component k (fp64): log pi_k - 1/2 sum_d log sigma2_kd, with the sum of
    // logs taken as one log of the product of the significands (each in [0.5, 1), so no
    // underflow for d_r <= 128 per lane) plus the sum of the binary exponents
    double mant = 1.0;
    int ex = 0;
#pragma unroll
    for (int u = 0; u < MAXD; ++u) {
        if (comp && j + u * TPC < dr) {
            int e;
            mant *= frexp(double(pv[u]), &e);
            ex += e;
        }
    }
    if (comp)
        for (int d = j + MAXD * TPC; d < dr; d += TPC) {
            int e;
            mant *= frexp(double(vk[d]), &e);
            ex += e;
        }
    for (int o = TPC / 2; o >= 1; o >>= 1) {
        mant *= __shfl_xor(mant, o, kWave);
        ex += __shfl_xor(ex, o, kWave);
    }
    const double ck =
        comp ? log(double(pik)) - 0.5 * (log(mant) + double(ex) * 0.69314718055994530942) : 0.0;

    for (int64_t i = 0; i < N; ++i) {
        const size_t rv = (size_t(p) * N + i) * dv;
        __syncthreads();  // the previous position is done with xq, xk, vv, gq, gk
        if (t < dr) {
            xq[t] = rq;
            xk[t] = rk;
        }
        if (t < dv) vv[t] = rvv;
        __syncthreads();
        if (i + 1 < N) fetch(i + 1);  // next position's inputs in flight during this one
        // Eq. 16 for the query and the key routing vector against component k
        double aq = 0.0, ak = 0.0;
        auto term = [&](int d, float mf, float vf) {
            const double m = double(mf), sv = double(vf);
            const double r0 = double(__builtin_amdgcn_rcpf(vf));
            const double iv = fma(r0, fma(-sv, r0, 1.0), r0);  // 1 / sigma2 to fp64 accuracy
            const double dq = double(xq[d]) - m, dk = double(xk[d]) - m;
            aq = fma(dq * dq, iv, aq);
            ak = fma(dk * dk, iv, ak);
        };
#pragma unroll
        for (int u = 0; u < MAXD; ++u)
            if (comp && j + u * TPC < dr) term(j + u * TPC, pm[u], pv[u]);
        if (comp)
            for (int d = j + MAXD * TPC; d < dr; d += TPC) term(d, mk[d], vk[d]);
        for (int o = TPC / 2; o >= 1; o >>= 1) {
            aq += __shfl_xor(aq, o, kWave);
            ak += __shfl_xor(ak, o, kWave);
        }
        if (comp && j == 0) {
            sc[k] = ck - 0.5 * aq;
            sc[K + k] = ck - 0.5 * ak;
        }
        __syncthreads();
        // Eq. 3b: softmax over the components in wave 0 (largest score subtracted; the exponent
        // of a difference <= 0 needs no more than fp32).  Lane l holds components l, l + 64, ...
        if (t < 64) {
            constexpr int PER = kDecodeThreads / 64;
            const float L2E = 1.4426950408889634f;
            float mq = -INFINITY, mkx = -INFINITY;
#pragma unroll
            for (int u = 0; u < PER; ++u)
                if (t + 64 * u < K) {
                    mq = fmaxf(mq, float(sc[t + 64 * u]));
                    mkx = fmaxf(mkx, float(sc[K + t + 64 * u]));
                }
            auto mx = [](float a, float b) { return fmaxf(a, b); };
            mq = wave_reduce(mq, mx);
            mkx = wave_reduce(mkx, mx);
            float eq[PER], ek[PER], lq = 0.0f, lk = 0.0f;
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const bool in = t + 64 * u < K;
                eq[u] = in ? __builtin_amdgcn_exp2f(float(sc[t + 64 * u] - double(mq)) * L2E) : 0.0f;
                ek[u] = in ? __builtin_amdgcn_exp2f(float(sc[K + t + 64 * u] - double(mkx)) * L2E) : 0.0f;
                lq += eq[u];
                lk += ek[u];
            }
            auto add = [](float a, float b) { return a + b; };
            const float rq_ = 1.0f / wave_reduce(lq, add), rk_ = 1.0f / wave_reduce(lk, add);
#pragma unroll
            for (int u = 0; u < PER; ++u)
                if (t + 64 * u < K) {
                    gq[t + 64 * u] = eq[u] * rq_;
                    gk[t + 64 * u] = ek[u] * rk_;
                }
        }
        __syncthreads();
        // Eq. 6b: memory += gammaK [V | 1]; Eq. 8b: numerator and denominator from the updated
        // memory.  Thread c owns memory column c (c < dv: Vt, c = dv: Z), components in order.
        float num = 0.0f;
        if (t <= dv) {
            const float add = t < dv ? vv[t] : 1.0f;
            for (int k0 = 0; k0 < K; k0 += 8) {  // 8 rows in flight at a time
                float m[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) m[u] = k0 + u < K ? mem[(k0 + u) * (dv + 1) + t] : 0.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (k0 + u < K) {
                        m[u] = fmaf(gk[k0 + u], add, m[u]);
                        num = fmaf(gq[k0 + u], m[u], num);
                        mem[(k0 + u) * (dv + 1) + t] = m[u];
                    }
                }
            }
            if (t == dv) den[0] = num + eps;
        }
        __syncthreads();
        if (t < dv) store_io(O, rv + t, num / den[0]);  // rv: this position's output row
    }
    __syncthreads();
    if (state_out) {
        if (vec) {
            float4* sp = reinterpret_cast<float4*>(state_out + size_t(p) * E);
            for (int e4 = t; e4 < E / 4; e4 += kDecodeThreads) sp[e4] = reinterpret_cast<const float4*>(mem)[e4];
        } else {
            for (int e = t; e < E; e += kDecodeThreads) state_out[size_t(p) * E + e] = mem[e];
        }
    }
}

size_t decode_lds_bytes(const Plan& p) {
    const size_t E = size_t(p.K) * size_t(p.dv + 1);
    // spare bytes, the memory, x_q, x_k, v, gamma_q, gamma_k, the denominator (float count padded
    // to even), then the fp64 scores [2][K]
    return 8 * (kDecodeThreads / 64) + ((E + 2 * size_t(p.dr) + size_t(p.dv) + 2 * size_t(p.K) + 2) & ~size_t(1)) * 4 +
           2 * size_t(p.K) * 8;
}

}  // namespace dec

using dec::decode_kernel;
using dec::decode_lds_bytes;
using dec::kDecodeThreads;

bool decode_applies(const Plan& p) {
    return p.op == GMA_OP_CAUSAL && p.N >= 1 && p.N <= kDecodeMaxPositions && p.K <= kDecodeThreads &&
           p.dv + 1 <= kDecodeThreads && decode_lds_bytes(p) <= 160 * 1024;
}

hipError_t causal_decode(const Plan& p, const void* XQ, const void* XK, const void* V, const float* mu,
                         const float* s2, const float* pi, float eps, void* O, hipStream_t st,
                         const float* state_in, float* state_out) {
    const size_t lds = decode_lds_bytes(p);
    const dim3 grid(unsigned(p.P)), block(kDecodeThreads);
    if (p.io == GMA_BF16) {
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_kernel<uint16_t>),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (attr != hipSuccess) return attr;
        GMA_LAUNCH("bf16_decode", decode_kernel<uint16_t>, grid, block, lds, st, static_cast<const uint16_t*>(XQ),
                   static_cast<const uint16_t*>(XK), static_cast<const uint16_t*>(V), p.N, int(p.H), int(p.dr),
                   int(p.dv), int(p.K), mu, s2, pi, eps, state_in, state_out, static_cast<uint16_t*>(O));
    } else {
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_kernel<float>),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (attr != hipSuccess) return attr;
        GMA_LAUNCH("f32_decode", decode_kernel<float>, grid, block, lds, st, static_cast<const float*>(XQ),
                   static_cast<const float*>(XK), static_cast<const float*>(V), p.N, int(p.H), int(p.dr), int(p.dv),
                   int(p.K), mu, s2, pi, eps, state_in, state_out, static_cast<float*>(O));
    }
    return hipGetLastError();
}

}  // namespace gma
