// Pieces of the fp32 path that the forward (gma_f32.hip) and the backward
// (gma_f32_backward.hip) share: block size and LDS limit, the fp64 score tables of every
// head, responsibility tiles in the direct form of Sec. 4.1 Eq. 16 of "Gaussian Mixture
// Attention", and the split write, combine and segment-prefix kernels of Sec. 3.3 Eq. 5-6
// and Sec. 3.5 Eq. 6b.  The kernels have internal linkage: each translation unit that
// includes this header launches its own copy.
#pragma once

#include <cmath>
#include <cstdint>

#include "gma_device.h"
#include "gma_internal.h"

namespace gma {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;  // tokens per tile
constexpr size_t kMaxLds = 160 * 1024;

struct F32Params {
    const double* c;    // [H][K]
    const double* inv;  // [H][K][dr]   1 / sigma2
};

F32Params f32_params_view(const Plan& p, char* ws) {
    F32Params v;
    v.c = reinterpret_cast<const double*>(ws + p.off_params);
    v.inv = reinterpret_cast<const double*>(ws + p.off_params + round_up(size_t(p.H * p.K) * 8, 256));
    return v;
}

// Grid (H, ceil(K / 4)): wave w of block (h, b) takes component k = 4 b + w of head h, its lanes
// over d: c_k = log pi_k - 1/2 sum_d log sigma2_kd in fp64 and the table of 1 / sigma2_kd.
__global__ void __launch_bounds__(kThreads) f32_params_kernel(const float* __restrict__ s2,
                                                              const float* __restrict__ pi, int K,
                                                              int dr, double* __restrict__ c_out,
                                                              double* __restrict__ inv_out) {
    const int h = blockIdx.x;
    const int lane = threadIdx.x & 63, k = blockIdx.y * (kThreads / kWave) + (threadIdx.x >> 6);
    if (k >= K) return;  // the whole wave
    const float* s2k = s2 + (size_t(h) * K + k) * dr;
    double acc = 0.0;
    for (int d = lane; d < dr; d += kWave) {
        const double v = double(s2k[d]);
        acc += log(v);
        inv_out[(size_t(h) * K + k) * dr + d] = 1.0 / v;
    }
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, kWave);
    if (lane == 0) c_out[size_t(h) * K + k] = log(double(pi[size_t(h) * K + k])) - 0.5 * acc;
}

// Grid (H): c_k of head h shifted by its maximum over k (a k-independent shift, exact in the
// softmax), so the fp32 value the score loops take is small.
__global__ void __launch_bounds__(kThreads) f32_params_shift_kernel(int K, double* __restrict__ c) {
    __shared__ double red[kThreads / kWave];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double* ch = c + size_t(blockIdx.x) * K;
    double m = -INFINITY;
    for (int k = threadIdx.x; k < K; k += kThreads) m = fmax(m, ch[k]);
    for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, kWave));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = red[0];
    for (int w = 1; w < kThreads / kWave; ++w) m = fmax(m, red[w]);
    for (int k = threadIdx.x; k < K; k += kThreads) ch[k] -= m;
}

// Responsibilities of rows [n0, n0 + rows) of one problem into LDS g[T][K]; xs is LDS
// scratch of T*dr floats.  Rows at or beyond `rows` are zero in g.  One wave owns a
// row at a time: each lane evaluates up to K/64 <= 4 scores in fp64 registers, the
// row maximum is subtracted in fp64, and only then is the softmax (Eq. 3b) taken in fp32.
__device__ void gamma_tile(const float* __restrict__ X, int64_t n0, int rows, int T, int dr, int K,
                           const double* __restrict__ c_h, const double* __restrict__ inv_h,
                           const float* __restrict__ mu_h, float* xs, float* g) {
    for (int i = threadIdx.x; i < T * dr; i += kThreads) {
        int t = i / dr;
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
        double sc[4];
        double m = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = lane + j * kWave;
            sc[j] = -INFINITY;
            if (k < K) {
                const float* mk = mu_h + size_t(k) * dr;
                const double* ik = inv_h + size_t(k) * dr;
                double q = 0.0;
                for (int d = 0; d < dr; ++d) {
                    double diff = double(xt[d]) - double(mk[d]);
                    q = fma(diff * diff, ik[d], q);
                }
                sc[j] = c_h[k] - 0.5 * q;
                m = fmax(m, sc[j]);
            }
        }
        for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, kWave));
        float ev[4];
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ev[j] = (lane + j * kWave < K) ? expf(float(sc[j] - m)) : 0.0f;
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

// Partial latent memory of one split: mem[k*dv + c] = sum_t gammaK_tk V_tc and
// mem[K*dv + k] = sum_t gammaK_tk over tokens [g*seg, min((g+1)*seg, N)).
__global__ void __launch_bounds__(kThreads) f32_write_kernel(const float* __restrict__ XK,
                                                             const float* __restrict__ V, int64_t N,
                                                             int H, int dr, int dv, int K, int64_t seg,
                                                             int G, const double* c, const double* inv,
                                                             const float* mu, float* partials) {
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int g_idx = blockIdx.x;
    const int h = int(p % H);
    float* xs = lds;
    float* g = xs + kTile * dr;
    float* vs = g + kTile * K;
    float* mem = partials + (size_t(p) * G + g_idx) * size_t(K) * (dv + 1);
    const int64_t lo = int64_t(g_idx) * seg, hi = min<int64_t>(lo + seg, N);
    const int E = K * (dv + 1);
    bool first = true;
    for (int64_t n0 = lo; n0 < hi; n0 += kTile) {
        const int rows = int(min<int64_t>(kTile, hi - n0));
        gamma_tile(XK + p * N * dr, n0, rows, kTile, dr, K, c + size_t(h) * K,
                   inv + size_t(h) * K * dr, mu + size_t(h) * K * dr, xs, g);
        for (int i = threadIdx.x; i < rows * dv; i += kThreads) vs[i] = V[(p * N + n0) * dv + i];
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += kThreads) {
            float acc = 0.0f;
            if (e < K * dv) {
                int k = e / dv, cc = e - k * dv;
                for (int t = 0; t < rows; ++t) acc = fmaf(g[t * K + k], vs[t * dv + cc], acc);
            } else {
                int k = e - K * dv;
                for (int t = 0; t < rows; ++t) acc += g[t * K + k];
            }
            mem[e] = first ? acc : mem[e] + acc;
        }
        first = false;
        __syncthreads();
    }
    if (first)  // empty split (cannot happen with the host plan, kept for safety)
        for (int e = threadIdx.x; e < E; e += kThreads) mem[e] = 0.0f;
}

// Bidirectional: out[p][e] = sum_g partials[p][g][e] in increasing g.
__global__ void __launch_bounds__(kThreads) f32_combine_kernel(const float* __restrict__ partials,
                                                               int G, int E, float* __restrict__ out) {
    const int64_t p = blockIdx.y;
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= E) return;
    const float* src = partials + size_t(p) * G * E + e;
    float acc = 0.0f;
    for (int g = 0; g < G; ++g) acc += src[size_t(g) * E];
    out[size_t(p) * E + e] = acc;
}

// Index of partial-layout element e (Vt [K][dv] then Z [K]) in the carried-memory layout
// [K][dv + 1] (row k: Vt_k then Z_k).
__device__ __forceinline__ int state_index(int e, int K, int dv) {
    return e < K * dv ? (e / dv) * (dv + 1) + e % dv : (e - K * dv) * (dv + 1) + dv;
}

// Causal: exclusive prefix over segments in place; segment g then holds the memory
// accumulated over all positions before it, starting from the carried memory state_in
// ([P][K][dv+1], or zero when NULL).
__global__ void __launch_bounds__(kThreads) f32_prefix_kernel(float* __restrict__ partials, int G, int E,
                                                              const float* __restrict__ state_in, int K, int dv) {
    const int64_t p = blockIdx.y;
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= E) return;
    float* src = partials + size_t(p) * G * E + e;
    float run = state_in ? state_in[size_t(p) * E + state_index(e, K, dv)] : 0.0f;
    for (int g = 0; g < G; ++g) {
        float a = src[size_t(g) * E];
        src[size_t(g) * E] = run;
        run += a;
    }
}

// The score tables of every head (f32_params_kernel, then the shift of c) into the workspace.
inline hipError_t launch_param_tables(const Plan& p, const float* s2, const float* pi, char* ws, hipStream_t st) {
    F32Params v = f32_params_view(p, ws);
    GMA_LAUNCH("f32_params", f32_params_kernel,
               dim3(unsigned(p.H), unsigned((p.K + kThreads / kWave - 1) / (kThreads / kWave))), dim3(kThreads), 0, st,
               s2, pi, int(p.K), int(p.dr), const_cast<double*>(v.c), const_cast<double*>(v.inv));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GMA_LAUNCH("f32_params_shift", f32_params_shift_kernel, dim3(unsigned(p.H)), dim3(kThreads), 0, st, int(p.K),
               const_cast<double*>(v.c));
    return hipGetLastError();
}

}  // namespace
}  // namespace gma
