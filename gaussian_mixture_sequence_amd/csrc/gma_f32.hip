// fp32 I/O path of the GMA forward: VALU kernels, direct-form scores.
//
// Scores follow Sec. 4.1 Eq. 16 of "Gaussian Mixture Attention" in the direct form
//   s_k = c_k - 1/2 sum_d (x_d - mu_kd)^2 / sigma2_kd,   c_k = log pi_k - 1/2 sum_d log sigma2_kd
// (the k-independent -(d_r/2) log 2 pi and any k-independent shift of c cancel in the
// softmax of Eq. 3b).  Scores are accumulated in fp64: with d_r = 128 the Mahalanobis
// sum reaches several hundred, where one fp32 ulp already moves a responsibility by
// ~1e-4, above the fp32 tolerance.  On gfx950 an fp64 FMA issues at the same rate as a
// non-packed fp32 FMA, so this costs no VALU throughput.  The softmax, the latent memory
// and the read run in fp32.  The bf16 path uses the expanded form on MFMA instead.
//
// Kernel sequence (each kernel one launch on the caller's stream):
//   params   c_k (computed in fp64, shifted by max_k c_k) and 1/sigma2 per head
//   write    per (problem, split g): partial [Vt | Z] = Gamma_K^T [V | 1] over the split's
//            tokens (Sec. 3.3 Eq. 5-6), tile by tile
//   combine  bidirectional: fixed-order sum of the partials; causal: exclusive prefix of
//            the segment aggregates, i.e. each segment's starting memory (Eq. 6b)
//   read     bidirectional: O = Gamma_Q Vt / (Gamma_Q Z + eps) (Eq. 7-8)
//   scan     causal: chunked scan of Eq. 6b/8b inside each segment
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

// One block per head.  c_k = log pi_k - 1/2 sum_d log sigma2_kd in fp64, then shifted by
// its maximum over k (a k-independent shift, exact in the softmax) so the fp32 value is small.
__global__ void __launch_bounds__(kThreads) f32_params_kernel(const float* __restrict__ s2,
                                                              const float* __restrict__ pi, int K,
                                                              int dr, double* __restrict__ c_out,
                                                              double* __restrict__ inv_out) {
    const int h = blockIdx.x;
    __shared__ double cd[256];
    __shared__ double red[kThreads / kWave];
    const float* s2h = s2 + size_t(h) * K * dr;
    double local_max = -INFINITY;
    for (int k = threadIdx.x; k < K; k += kThreads) {
        double acc = log(double(pi[size_t(h) * K + k]));
        for (int d = 0; d < dr; ++d) {
            double v = double(s2h[size_t(k) * dr + d]);
            acc -= 0.5 * log(v);
            inv_out[(size_t(h) * K + k) * dr + d] = 1.0 / v;
        }
        cd[k] = acc;
        local_max = fmax(local_max, acc);
    }
    // block max
    for (int o = 32; o >= 1; o >>= 1) local_max = fmax(local_max, __shfl_xor(local_max, o, kWave));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = local_max;
    __syncthreads();
    double m = red[0];
    for (int w = 1; w < kThreads / kWave; ++w) m = fmax(m, red[w]);
    for (int k = threadIdx.x; k < K; k += kThreads) c_out[size_t(h) * K + k] = cd[k] - m;
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

__global__ void __launch_bounds__(kThreads) f32_resp_kernel(const float* __restrict__ X, int64_t N,
                                                            int H, int dr, int K, const double* c,
                                                            const double* inv, const float* mu,
                                                            void* Gamma, int gamma_bf16) {
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int h = int(p % H);
    const int64_t n0 = int64_t(blockIdx.x) * kTile;
    const int rows = int(min<int64_t>(kTile, N - n0));
    float* xs = lds;
    float* g = lds + kTile * dr;
    gamma_tile(X + p * N * dr, n0, rows, kTile, dr, K, c + size_t(h) * K, inv + size_t(h) * K * dr,
               mu + size_t(h) * K * dr, xs, g);
    const size_t base = (size_t(p) * N + n0) * K;
    for (int i = threadIdx.x; i < rows * K; i += kThreads) {
        if (gamma_bf16)
            static_cast<uint16_t*>(Gamma)[base + i] = f32_to_bf16_bits(g[i]);
        else
            static_cast<float*>(Gamma)[base + i] = g[i];
    }
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

// Eq. 7-8 for one tile of queries.
__global__ void __launch_bounds__(kThreads) f32_read_kernel(const float* __restrict__ XQ, int64_t N,
                                                            int H, int dr, int dv, int K, const double* c,
                                                            const double* inv, const float* mu,
                                                            const float* __restrict__ memory, float eps,
                                                            float* __restrict__ O) {
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int h = int(p % H);
    const int64_t n0 = int64_t(blockIdx.x) * kTile;
    const int rows = int(min<int64_t>(kTile, N - n0));
    float* xs = lds;
    float* g = xs + kTile * dr;
    float* den = g + kTile * K;
    gamma_tile(XQ + p * N * dr, n0, rows, kTile, dr, K, c + size_t(h) * K, inv + size_t(h) * K * dr,
               mu + size_t(h) * K * dr, xs, g);
    const float* Vt = memory + size_t(p) * K * (dv + 1);
    const float* Z = Vt + size_t(K) * dv;
    for (int t = threadIdx.x; t < rows; t += kThreads) {
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) acc = fmaf(g[t * K + k], Z[k], acc);
        den[t] = acc + eps;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < rows * dv; i += kThreads) {
        int t = i / dv, cc = i - t * dv;
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) acc = fmaf(g[t * K + k], Vt[size_t(k) * dv + cc], acc);
        O[(p * N + n0) * dv + i] = acc / den[t];
    }
}

// Causal scan of one segment (Eq. 6b/8b).  `state` starts as the segment's prefix memory
// and is advanced chunk by chunk: for a chunk with responsibilities Gq, Gk and values Vc,
//   A_tj = sum_k Gq_tk Gk_jk  for j <= t (0 otherwise)
//   O_t  = (sum_j A_tj Vc_j + Gq_t Vt) / (sum_j A_tj + Gq_t Z + eps)
//   Vt  += Gk^T Vc,  Z += Gk^T 1
__global__ void __launch_bounds__(kThreads) f32_scan_kernel(const float* __restrict__ XQ,
                                                            const float* __restrict__ XK,
                                                            const float* __restrict__ V, int64_t N, int H,
                                                            int dr, int dv, int K, int64_t seg, int G,
                                                            int C, const double* c, const double* inv,
                                                            const float* mu, float* partials, float eps,
                                                            float* __restrict__ O, float* __restrict__ state_out) {
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int g_idx = blockIdx.x;
    const int h = int(p % H);
    float* xs = lds;              // C*dr
    float* gq = xs + C * dr;      // C*K
    float* gk = gq + C * K;       // C*K
    float* vs = gk + C * K;       // C*dv
    float* A = vs + C * dv;       // C*C
    float* den = A + C * C;       // C
    float* Vt = partials + (size_t(p) * G + g_idx) * size_t(K) * (dv + 1);
    float* Z = Vt + size_t(K) * dv;
    const double *ch = c + size_t(h) * K, *ih = inv + size_t(h) * K * dr;
    const float* mh = mu + size_t(h) * K * dr;
    const int64_t lo = int64_t(g_idx) * seg, hi = min<int64_t>(lo + seg, N);
    for (int64_t n0 = lo; n0 < hi; n0 += C) {
        const int rows = int(min<int64_t>(C, hi - n0));
        gamma_tile(XQ + p * N * dr, n0, rows, C, dr, K, ch, ih, mh, xs, gq);
        gamma_tile(XK + p * N * dr, n0, rows, C, dr, K, ch, ih, mh, xs, gk);
        for (int i = threadIdx.x; i < rows * dv; i += kThreads) vs[i] = V[(p * N + n0) * dv + i];
        for (int i = threadIdx.x; i < C * C; i += kThreads) {
            int t = i / C, j = i - t * C;
            float acc = 0.0f;
            if (t < rows && j <= t)
                for (int k = 0; k < K; ++k) acc = fmaf(gq[t * K + k], gk[j * K + k], acc);
            A[i] = acc;
        }
        __syncthreads();
        for (int t = threadIdx.x; t < rows; t += kThreads) {
            float acc = 0.0f;
            for (int j = 0; j <= t; ++j) acc += A[t * C + j];
            for (int k = 0; k < K; ++k) acc = fmaf(gq[t * K + k], Z[k], acc);
            den[t] = acc + eps;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < rows * dv; i += kThreads) {
            int t = i / dv, cc = i - t * dv;
            float acc = 0.0f;
            for (int j = 0; j <= t; ++j) acc = fmaf(A[t * C + j], vs[j * dv + cc], acc);
            for (int k = 0; k < K; ++k) acc = fmaf(gq[t * K + k], Vt[size_t(k) * dv + cc], acc);
            O[(p * N + n0) * dv + i] = acc / den[t];
        }
        __syncthreads();  // every read of the state for this chunk is done
        for (int e = threadIdx.x; e < K * (dv + 1); e += kThreads) {
            float acc = 0.0f;
            if (e < K * dv) {
                int k = e / dv, cc = e - k * dv;
                for (int t = 0; t < rows; ++t) acc = fmaf(gk[t * K + k], vs[t * dv + cc], acc);
            } else {
                int k = e - K * dv;
                for (int t = 0; t < rows; ++t) acc += gk[t * K + k];
            }
            Vt[e] += acc;  // Z is contiguous after Vt, so one index covers both
        }
        __syncthreads();  // state update visible to the whole block before the next chunk
    }
    // the last segment's memory is the memory after the last position
    if (state_out && g_idx == G - 1)
        for (int e = threadIdx.x; e < K * (dv + 1); e += kThreads)
            state_out[size_t(p) * K * (dv + 1) + state_index(e, K, dv)] = Vt[e];
}

__global__ void __launch_bounds__(kThreads) state_copy_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                              int E) {
    const size_t i = size_t(blockIdx.y) * E + size_t(blockIdx.x) * kThreads + threadIdx.x;
    if (int(blockIdx.x) * kThreads + int(threadIdx.x) < E) out[i] = in ? in[i] : 0.0f;
}

size_t scan_lds_bytes(int C, int dr, int dv, int K) {
    return size_t(C) * (dr + 2 * K + dv + C + 1) * sizeof(float);
}

// Kernels below may take more than 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU).
hipError_t allow_lds() {
    static hipError_t status = [] {
        const void* fns[] = {(const void*)f32_resp_kernel, (const void*)f32_write_kernel,
                             (const void*)f32_read_kernel, (const void*)f32_scan_kernel};
        for (const void* f : fns) {
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxLds));
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }();
    return status;
}

hipError_t launch_params(const Plan& p, const float* s2, const float* pi, char* ws, hipStream_t st) {
    hipError_t e0 = allow_lds();
    if (e0 != hipSuccess) return e0;
    F32Params v = f32_params_view(p, ws);
    GMA_LAUNCH("f32_params", f32_params_kernel, dim3(unsigned(p.H)), dim3(kThreads), 0, st, s2, pi, int(p.K),
                       int(p.dr), const_cast<double*>(v.c), const_cast<double*>(v.inv));
    return hipGetLastError();
}

}  // namespace

hipError_t f32_responsibilities(const Plan& p, const float* X, const float* mu, const float* s2,
                                const float* pi, void* Gamma, gma_dtype_t gamma_dtype, char* ws,
                                hipStream_t st) {
    hipError_t e = launch_params(p, s2, pi, ws, st);
    if (e != hipSuccess) return e;
    F32Params v = f32_params_view(p, ws);
    size_t lds = size_t(kTile) * (p.dr + p.K) * sizeof(float);
    dim3 grid(unsigned((p.N + kTile - 1) / kTile), unsigned(p.P));
    GMA_LAUNCH("f32_resp", f32_resp_kernel, grid, dim3(kThreads), lds, st, X, p.N, int(p.H), int(p.dr),
                       int(p.K), v.c, v.inv, mu, Gamma, gamma_dtype == GMA_BF16 ? 1 : 0);
    return hipGetLastError();
}

hipError_t f32_bidir(const Plan& p, const float* XQ, const float* XK, const float* V, const float* mu,
                     const float* s2, const float* pi, float eps, float* O, char* ws, hipStream_t st) {
    hipError_t e = launch_params(p, s2, pi, ws, st);
    if (e != hipSuccess) return e;
    F32Params v = f32_params_view(p, ws);
    float* partials = reinterpret_cast<float*>(ws + p.off_partials);
    float* memory = reinterpret_cast<float*>(ws + p.off_memory);
    const int E = int(p.K * (p.dv + 1));
    size_t lds_w = size_t(kTile) * (p.dr + p.K + p.dv) * sizeof(float);
    GMA_LAUNCH(p.cross ? "f32_cross_write" : "f32_write", f32_write_kernel, dim3(unsigned(p.G), unsigned(p.P)), dim3(kThreads), lds_w, st, XK, V,
                       p.N, int(p.H), int(p.dr), int(p.dv), int(p.K), p.seg, int(p.G), v.c, v.inv, mu,
                       partials);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GMA_LAUNCH(p.cross ? "f32_cross_combine" : "f32_combine", f32_combine_kernel, dim3(unsigned((E + kThreads - 1) / kThreads), unsigned(p.P)),
                       dim3(kThreads), 0, st, partials, int(p.G), E, memory);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    size_t lds_r = size_t(kTile) * (p.dr + p.K + 1) * sizeof(float);
    GMA_LAUNCH(p.cross ? "f32_cross_read" : "f32_read", f32_read_kernel, dim3(unsigned((p.Nq + kTile - 1) / kTile), unsigned(p.P)),
                       dim3(kThreads), lds_r, st, XQ, p.Nq, int(p.H), int(p.dr), int(p.dv), int(p.K), v.c,
                       v.inv, mu, memory, eps, O);
    return hipGetLastError();
}

hipError_t copy_state(const Plan& p, const float* state_in, float* state_out, hipStream_t st) {
    const int E = int(p.K * (p.dv + 1));
    GMA_LAUNCH("state_copy", state_copy_kernel, dim3(unsigned((E + kThreads - 1) / kThreads), unsigned(p.P)),
               dim3(kThreads), 0, st, state_in, state_out, E);
    return hipGetLastError();
}

hipError_t f32_causal(const Plan& p, const float* XQ, const float* XK, const float* V, const float* mu,
                      const float* s2, const float* pi, float eps, float* O, char* ws, hipStream_t st,
                      const float* state_in, float* state_out) {
    hipError_t e = launch_params(p, s2, pi, ws, st);
    if (e != hipSuccess) return e;
    F32Params v = f32_params_view(p, ws);
    float* partials = reinterpret_cast<float*>(ws + p.off_partials);
    const int E = int(p.K * (p.dv + 1));
    if (p.G > 1) {
        size_t lds_w = size_t(kTile) * (p.dr + p.K + p.dv) * sizeof(float);
        GMA_LAUNCH("f32_causal_aggregate", f32_write_kernel, dim3(unsigned(p.G), unsigned(p.P)), dim3(kThreads), lds_w, st, XK,
                           V, p.N, int(p.H), int(p.dr), int(p.dv), int(p.K), p.seg, int(p.G), v.c, v.inv, mu,
                           partials);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // With one segment the aggregate pass is skipped: the prefix kernel writes the
    // starting memory of segment 0 as zeros without reading the aggregate.
    GMA_LAUNCH("f32_prefix", f32_prefix_kernel, dim3(unsigned((E + kThreads - 1) / kThreads), unsigned(p.P)),
                       dim3(kThreads), 0, st, partials, int(p.G), E, state_in, int(p.K), int(p.dv));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // The chunk length is a tiling choice; halve it until the chunk's tiles fit in LDS.
    int C = p.chunk;
    while (C > 8 && scan_lds_bytes(C, int(p.dr), int(p.dv), int(p.K)) > kMaxLds) C /= 2;
    GMA_LAUNCH("f32_scan", f32_scan_kernel, dim3(unsigned(p.G), unsigned(p.P)), dim3(kThreads),
                       scan_lds_bytes(C, int(p.dr), int(p.dv), int(p.K)), st, XQ, XK, V, p.N, int(p.H),
                       int(p.dr), int(p.dv), int(p.K), p.seg, int(p.G), C, v.c, v.inv, mu, partials, eps, O,
                       state_out);
    return hipGetLastError();
}

// ============================================================================ backward
// Gradients of <dO, O> for the bidirectional forward (Sec. 4.1 of "Gaussian Mixture
// Attention": the softmax Jacobian of Eq. 17, the centred score gradient of Eq. 18 and the
// chain rule of Eq. 19-20 through the direct-form score of Eq. 16), fp32 with the fp64 score
// tables of the forward.  With a_i = dO_i . O_i and D_i = gamma^Q_i . Z + eps:
//   g^Q_ik = (dO_i . Vt_k - a_i Z_k) / D_i,      dVt_k = sum_i gamma^Q_ik dO_i / D_i,
//   dZ_k = -sum_i gamma^Q_ik a_i / D_i,          dV_j = sum_k gamma^K_jk dVt_k,
//   g^K_jk = dVt_k . V_j + dZ_k,                  ds_ik = gamma_ik (g_ik - sum_l gamma_il g_il),
//   dx_id = -sum_k ds_ik (x_id - mu_kd) / sigma2_kd,
//   dmu_kd += ds_ik (x_id - mu_kd) / sigma2_kd,   dsigma2_kd += ds_ik ((x_id - mu_kd)^2 / sigma2_kd^2
//   - 1 / sigma2_kd) / 2,                         dpi_k += ds_ik / pi_k.
namespace {

// LDS floats of one side's tile of T rows.
size_t bwd_lds_bytes(int T, int dr, int dv, int K) { return size_t(T) * (dr + 2 * K + dv + 2) * sizeof(float); }

// Grid (G, P): rows [g seg, (g + 1) seg) of problem p in tiles of T.  QUERY: the query side
// (reads the memory mem = [Vt | Z], writes dX_Q and the partial [dVt | dZ] of its rows);
// otherwise the key side (reads dmem = [dVt | dZ], writes dV and dX_K).  Both add their rows'
// parameter gradients into the block's partial record pp = [dmu (K dr) | dsigma2 (K dr) | dpi
// (K)] (first tile writes, later tiles add: each entry has one owner thread).
template <bool QUERY>
__global__ void __launch_bounds__(kThreads)
    f32_bwd_side_kernel(const float* __restrict__ X, const float* __restrict__ Y, int64_t N, int H, int dr, int dv,
                        int K, int64_t seg, int G, int T, const double* c, const double* inv, const float* mu,
                        const float* __restrict__ pi, const float* __restrict__ mem, float eps,
                        float* __restrict__ dX, float* __restrict__ dY, float* __restrict__ mem_part,
                        float* __restrict__ param_part) {
    extern __shared__ float lds[];
    const int64_t p = blockIdx.y;
    const int gi = blockIdx.x, h = int(p % H);
    float* xs = lds;          // T*dr: the tile's routing vectors (left by gamma_tile)
    float* gm = xs + T * dr;  // T*K: responsibilities
    float* gg = gm + T * K;   // T*K: upstream gradient, then the score gradient
    float* ys = gg + T * K;   // T*dv: dO (query side) or V (key side)
    float* dd = ys + T * dv;  // T: D_i
    float* aa = dd + T;       // T: a_i
    const double *ch = c + size_t(h) * K, *ih = inv + size_t(h) * K * dr;
    const float* mh = mu + size_t(h) * K * dr;
    const float* Vt = mem + size_t(p) * K * (dv + 1);  // [K][dv], then Z (or dVt, dZ)
    const float* Z = Vt + size_t(K) * dv;
    const int E = K * (dv + 1), PE = 2 * K * dr + K;
    float* mp = mem_part ? mem_part + (size_t(p) * G + gi) * E : nullptr;
    float* pp = param_part + (size_t(p) * G + gi) * PE;
    const int64_t lo = int64_t(gi) * seg, hi = min<int64_t>(lo + seg, N);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    bool first = true;
    for (int64_t n0 = lo; n0 < hi; n0 += T) {
        const int rows = int(min<int64_t>(T, hi - n0));
        gamma_tile(X + p * N * dr, n0, rows, T, dr, K, ch, ih, mh, xs, gm);
        for (int i = threadIdx.x; i < T * dv; i += kThreads) {
            const int t = i / dv;
            ys[i] = t < rows ? Y[(p * N + n0) * dv + i] : 0.0f;
        }
        __syncthreads();
        if (QUERY) {  // D_t and a_t = dO_t . O_t, one wave per row
            for (int t = wave; t < rows; t += kThreads / kWave) {
                float d = 0.0f;
                for (int k = lane; k < K; k += kWave) d = fmaf(gm[t * K + k], Z[k], d);
                d = wave_sum(d) + eps;
                float a = 0.0f;
                for (int cc = lane; cc < dv; cc += kWave) {
                    float nn = 0.0f;
                    for (int k = 0; k < K; ++k) nn = fmaf(gm[t * K + k], Vt[size_t(k) * dv + cc], nn);
                    a = fmaf(ys[t * dv + cc], nn / d, a);
                }
                a = wave_sum(a);
                if (lane == 0) {
                    dd[t] = d;
                    aa[t] = a;
                }
            }
            __syncthreads();
        } else {  // dV_tc = sum_k gamma^K_tk dVt_kc
            for (int i = threadIdx.x; i < rows * dv; i += kThreads) {
                const int t = i / dv, cc = i - t * dv;
                float acc = 0.0f;
                for (int k = 0; k < K; ++k) acc = fmaf(gm[t * K + k], Vt[size_t(k) * dv + cc], acc);
                dY[(p * N + n0) * dv + i] = acc;
            }
        }
        // upstream gradient at the responsibilities
        for (int i = threadIdx.x; i < T * K; i += kThreads) {
            const int t = i / K, k = i - t * K;
            float acc = 0.0f;
            if (t < rows) {
                for (int cc = 0; cc < dv; ++cc) acc = fmaf(ys[t * dv + cc], Vt[size_t(k) * dv + cc], acc);
                acc = QUERY ? (acc - aa[t] * Z[k]) / dd[t] : acc + Z[k];
            }
            gg[i] = acc;
        }
        __syncthreads();
        // Eq. 18: ds = gamma (g - gamma . g), one wave per row
        for (int t = wave; t < T; t += kThreads / kWave) {
            float w = 0.0f;
            for (int k = lane; k < K; k += kWave) w = fmaf(gm[t * K + k], gg[t * K + k], w);
            w = wave_sum(w);
            for (int k = lane; k < K; k += kWave) gg[t * K + k] = gm[t * K + k] * (gg[t * K + k] - w);
        }
        __syncthreads();
        // routing-vector gradient
        for (int i = threadIdx.x; i < rows * dr; i += kThreads) {
            const int t = i / dr, d = i - t * dr;
            float acc = 0.0f;
            for (int k = 0; k < K; ++k)
                acc = fmaf(gg[t * K + k], float((double(xs[t * dr + d]) - double(mh[size_t(k) * dr + d])) * ih[size_t(k) * dr + d]), acc);
            dX[(p * N + n0) * dr + i] = -acc;
        }
        // parameter gradients of these rows (Eq. 19-20)
        for (int e = threadIdx.x; e < K * dr; e += kThreads) {
            const int k = e / dr, d = e - k * dr;
            const double m = double(mh[e]), iv = ih[e];
            double am = 0.0, as = 0.0;
            for (int t = 0; t < rows; ++t) {
                const double df = double(xs[t * dr + d]) - m, s = double(gg[t * K + k]);
                am += s * df * iv;
                as += s * 0.5 * (df * df * iv * iv - iv);
            }
            pp[e] = first ? float(am) : pp[e] + float(am);
            pp[K * dr + e] = first ? float(as) : pp[K * dr + e] + float(as);
        }
        for (int k = threadIdx.x; k < K; k += kThreads) {
            float acc = 0.0f;
            for (int t = 0; t < rows; ++t) acc += gg[t * K + k];
            acc /= pi[size_t(h) * K + k];
            pp[2 * K * dr + k] = first ? acc : pp[2 * K * dr + k] + acc;
        }
        if (QUERY) {  // partial [dVt | dZ] of these rows, in the memory's layout
            for (int e = threadIdx.x; e < E; e += kThreads) {
                float acc = 0.0f;
                if (e < K * dv) {
                    const int k = e / dv, cc = e - k * dv;
                    for (int t = 0; t < rows; ++t) acc = fmaf(gm[t * K + k], ys[t * dv + cc] / dd[t], acc);
                } else {
                    const int k = e - K * dv;
                    for (int t = 0; t < rows; ++t) acc -= gm[t * K + k] * aa[t] / dd[t];
                }
                mp[e] = first ? acc : mp[e] + acc;
            }
        }
        first = false;
        __syncthreads();  // the tile's LDS is free
    }
    if (first) {  // empty block
        for (int e = threadIdx.x; e < PE; e += kThreads) pp[e] = 0.0f;
        if (QUERY)
            for (int e = threadIdx.x; e < E; e += kThreads) mp[e] = 0.0f;
    }
}

// Grid (ceil(PE / kThreads), H): the parameter gradients of head h, one entry per thread, summed
// over the query and key sides, the batch and the splits in that fixed order.  With B == 0 it
// writes zeros (no rows, no gradient).
__global__ void __launch_bounds__(kThreads)
    f32_bwd_param_reduce_kernel(const float* __restrict__ param_part, int B, int H, int G, int K, int dr,
                                float* __restrict__ dmu, float* __restrict__ ds2, float* __restrict__ dpi) {
    const int h = blockIdx.y, PE = 2 * K * dr + K;
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= PE) return;
    const size_t P = size_t(B) * H;
    float acc = 0.0f;
    for (int side = 0; side < 2; ++side)
        for (int b = 0; b < B; ++b)
            for (int g = 0; g < G; ++g) acc += param_part[((side * P + size_t(b) * H + h) * G + g) * PE + e];
    if (e < K * dr) dmu[size_t(h) * K * dr + e] = acc;
    else if (e < 2 * K * dr) ds2[size_t(h) * K * dr + e - K * dr] = acc;
    else dpi[size_t(h) * K + e - 2 * K * dr] = acc;
}

}  // namespace

size_t f32_backward_extra_bytes(const Plan& p) {
    const size_t E = size_t(p.K) * size_t(p.dv + 1);
    return round_up(size_t(p.P * p.G) * E * 4, 256) + round_up(size_t(p.P) * E * 4, 256) +
           round_up(2 * size_t(p.P * p.G) * size_t(2 * p.K * p.dr + p.K) * 4, 256);
}

namespace {
hipError_t reduce_params(const Plan& p, const float* ppart, int B, float* dmu, float* ds2, float* dpi, hipStream_t st) {
    const int PE = int(2 * p.K * p.dr + p.K);
    GMA_LAUNCH("f32_bwd_params", f32_bwd_param_reduce_kernel, dim3(unsigned((PE + kThreads - 1) / kThreads), unsigned(p.H)),
               dim3(kThreads), 0, st, ppart, B, int(p.H), int(p.G), int(p.K), int(p.dr), dmu, ds2, dpi);
    return hipGetLastError();
}
}  // namespace

hipError_t f32_backward_bidir(const Plan& p, const float* XQ, const float* XK, const float* V, const float* mu,
                              const float* s2, const float* pi, float eps, const float* dO, float* dXQ, float* dXK,
                              float* dV, float* dmu, float* ds2, float* dpi, char* ws, hipStream_t st) {
    if (p.H == 0) return hipSuccess;
    if (p.P == 0 || p.N == 0) return reduce_params(p, nullptr, 0, dmu, ds2, dpi, st);  // zero gradients
    static const hipError_t attr = [] {
        const void* fns[] = {(const void*)f32_bwd_side_kernel<true>, (const void*)f32_bwd_side_kernel<false>};
        for (const void* f : fns) {
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxLds));
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }();
    if (attr != hipSuccess) return attr;
    hipError_t e = launch_params(p, s2, pi, ws, st);
    if (e != hipSuccess) return e;
    F32Params v = f32_params_view(p, ws);
    float* partials = reinterpret_cast<float*>(ws + p.off_partials);
    float* memory = reinterpret_cast<float*>(ws + p.off_memory);
    const size_t E = size_t(p.K) * size_t(p.dv + 1);
    char* extra = ws + p.total - f32_backward_extra_bytes(p);
    float* dpart = reinterpret_cast<float*>(extra);
    float* dmem = reinterpret_cast<float*>(extra + round_up(size_t(p.P * p.G) * E * 4, 256));
    float* ppart = reinterpret_cast<float*>(extra + round_up(size_t(p.P * p.G) * E * 4, 256) + round_up(size_t(p.P) * E * 4, 256));
    // the forward's memory
    size_t lds_w = size_t(kTile) * (p.dr + p.K + p.dv) * sizeof(float);
    GMA_LAUNCH("f32_bwd_write", f32_write_kernel, dim3(unsigned(p.G), unsigned(p.P)), dim3(kThreads), lds_w, st, XK, V,
               p.N, int(p.H), int(p.dr), int(p.dv), int(p.K), p.seg, int(p.G), v.c, v.inv, mu, partials);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int Ei = int(E);
    GMA_LAUNCH("f32_bwd_combine", f32_combine_kernel, dim3(unsigned((Ei + kThreads - 1) / kThreads), unsigned(p.P)),
               dim3(kThreads), 0, st, partials, int(p.G), Ei, memory);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    int T = kTile;
    while (T > 8 && bwd_lds_bytes(T, int(p.dr), int(p.dv), int(p.K)) > kMaxLds) T /= 2;
    const size_t lds = bwd_lds_bytes(T, int(p.dr), int(p.dv), int(p.K));
    GMA_LAUNCH("f32_bwd_query", f32_bwd_side_kernel<true>, dim3(unsigned(p.G), unsigned(p.P)), dim3(kThreads), lds, st,
               XQ, dO, p.N, int(p.H), int(p.dr), int(p.dv), int(p.K), p.seg, int(p.G), T, v.c, v.inv, mu, pi, memory,
               eps, dXQ, static_cast<float*>(nullptr), dpart, ppart);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GMA_LAUNCH("f32_bwd_combine", f32_combine_kernel, dim3(unsigned((Ei + kThreads - 1) / kThreads), unsigned(p.P)),
               dim3(kThreads), 0, st, dpart, int(p.G), Ei, dmem);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GMA_LAUNCH("f32_bwd_key", f32_bwd_side_kernel<false>, dim3(unsigned(p.G), unsigned(p.P)), dim3(kThreads), lds, st,
               XK, V, p.N, int(p.H), int(p.dr), int(p.dv), int(p.K), p.seg, int(p.G), T, v.c, v.inv, mu, pi, dmem,
               eps, dXK, dV, static_cast<float*>(nullptr), ppart + size_t(p.P * p.G) * size_t(2 * p.K * p.dr + p.K));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return reduce_params(p, ppart, int(p.B), dmu, ds2, dpi, st);
}

}  // namespace gma
