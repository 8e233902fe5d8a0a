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
#include "gma_f32_common.h"

namespace gma {
namespace {

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
    return launch_param_tables(p, s2, pi, ws, st);
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

// The chunk length is a tiling choice: the requested one, halved until the chunk's tiles fit in LDS.
int64_t f32_causal_chunk(const Plan& p) {
    int C = p.chunk;
    while (C > 8 && scan_lds_bytes(C, int(p.dr), int(p.dv), int(p.K)) > kMaxLds) C /= 2;
    return C;
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
    const int C = int(f32_causal_chunk(p));
    GMA_LAUNCH("f32_scan", f32_scan_kernel, dim3(unsigned(p.G), unsigned(p.P)), dim3(kThreads),
                       scan_lds_bytes(C, int(p.dr), int(p.dv), int(p.K)), st, XQ, XK, V, p.N, int(p.H),
                       int(p.dr), int(p.dv), int(p.K), p.seg, int(p.G), C, v.c, v.inv, mu, partials, eps, O,
                       state_out);
    return hipGetLastError();
}

}  // namespace gma
