// Internal interface between the C-ABI front end (gma_api.cpp) and the kernel
// launchers (gma_f32.hip, gma_bf16.hip).  Not installed; the public ABI is
// include/gma.h.
#pragma once

#include <cstddef>
#include <cstdint>
#include <hip/hip_runtime.h>

#include "gma.h"

namespace gma {

// Rounded-up size of one workspace region (256-byte granules keep every region
// aligned for vector loads).
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Where each piece of scratch lives inside the caller's workspace, and how the
// sequence is split.  Computed on the host from the shape alone (never from the
// device), so workspace sizes and reduction orders are the same on every GPU.
struct Plan {
    gma_op_t op;
    gma_dtype_t io;
    int64_t B, H, N, dr, dv, K;
    int64_t Nq;           // query rows: N, except for cross-attention (N is then the context length)
    bool cross;           // cross-attention plan (queries and keys from different sequences)
    int64_t P;            // B * H independent (batch, head) problems
    int64_t Kp;           // K padded to the MFMA component tile (bf16) or K (f32)
    int64_t G;            // sequence splits per problem (write partials / causal segments)
    int64_t seg;          // tokens per split (multiple of the token tile)
    int64_t seg_q;        // query rows per split of the read (seg, except for cross-attention)
    int32_t chunk;        // causal chunk length
    // byte offsets into the workspace
    size_t off_params, off_partials, off_memory, off_flags, off_gk, total;
    size_t off_stage;     // backward: end of the fp32 passes' regions; bf16 I/O is staged in fp32 after it
    size_t params_bytes, partials_bytes, memory_bytes, flags_bytes;
    size_t gk_bytes;      // bf16 causal with 256 components: the keys' responsibilities [P][N][256] bf16
};

// A fresh 64-bit value per launch that hands data between workgroups (bf16 fused kernels):
// flag words left in a workspace by earlier calls never equal it.
uint64_t launch_token();

// Polls a workgroup of the fused bf16 kernels makes before it gives up on a hand-off
// (gma_set_wait_limit).
uint32_t wait_limit();

// Bits of the per-device error word that kernels raise (atomic OR) and gma_device_status
// takes: a hand-off wait of a single-launch forward ran out.
// Splits per problem up to which the bf16 bidirectional forward runs as one launch; beyond,
// its write, combine and read launches measure faster (the single launch waits on more
// workgroups per problem and holds both phases' registers).
constexpr int64_t kBidirSingleMaxSplits = 8;
constexpr uint32_t kDevErrTimeout = 1u;
// Address of the error word on the current device (resolved once per device).
hipError_t device_error_word(uint32_t** word);

// Whether the bf16 forwards may hand data between workgroups inside one launch
// (gma_set_single_launch).
bool single_launch_enabled();
// Workgroups of `kernel` (launched with `threads` threads and no dynamic LDS) that the current
// device keeps resident at once: the runtime's occupancy per CU times the CU count (cached).
hipError_t resident_workgroups(const void* kernel, int threads, int64_t* out);

// Kernel timing hooks (see gma_profiling in gma.h).  Launchers bracket each launch with
// trace_begin / trace_end; both are no-ops unless profiling is enabled.
void trace_begin(hipStream_t st, const char* name);
void trace_end(hipStream_t st);

// hipLaunchKernelGGL bracketed by the timing hooks; `name` must be a static string.
#define GMA_LAUNCH(name, kernel, grid, block, lds, stream, ...)                   \
    do {                                                                         \
        ::gma::trace_begin(stream, name);                                        \
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);       \
        ::gma::trace_end(stream);                                                \
    } while (0)

// Fills `plan`; returns GMA_OK or the validation error for unsupported sizes.
gma_status_t make_plan(gma_op_t op, const gma_shape_t& s, gma_dtype_t io, int32_t chunk, Plan* plan);
// Cross-attention plan: a bidirectional plan over the context (N = N_k) whose read covers
// N_q query rows in the same number of splits.
gma_status_t make_cross_plan(const gma_cross_shape_t& s, gma_dtype_t io, Plan* plan);
// Backward of cross-attention: the cross plan (fp32) with the backward's scratch and staging.
gma_status_t make_backward_cross_plan(const gma_cross_shape_t& s, gma_dtype_t io, Plan* plan);

// ---- fp32 path (gma_f32.hip) ---------------------------------------------------
hipError_t f32_responsibilities(const Plan& p, const float* X, const float* mu, const float* s2,
                                const float* pi, void* Gamma, gma_dtype_t gamma_dtype, char* ws,
                                hipStream_t st);
hipError_t f32_bidir(const Plan& p, const float* XQ, const float* XK, const float* V,
                     const float* mu, const float* s2, const float* pi, float eps, float* O,
                     char* ws, hipStream_t st);
// state_in / state_out: [P][K][d_v+1] fp32 carried memory (gma_forward_causal_state), or NULL.
// Positions per chunk the fp32 causal scan runs for the plan's requested chunk.
int64_t f32_causal_chunk(const Plan& p);
hipError_t f32_causal(const Plan& p, const float* XQ, const float* XK, const float* V,
                      const float* mu, const float* s2, const float* pi, float eps, float* O,
                      char* ws, hipStream_t st, const float* state_in, float* state_out);
// state_out = state_in (zeros if state_in is NULL) for the P problems of `p`: the carried
// memory of a call without positions.
hipError_t copy_state(const Plan& p, const float* state_in, float* state_out, hipStream_t st);

// Backward of the bidirectional forward (fp32): workspace beyond the bidirectional plan's
// own (placed at its end), and the launcher.
size_t f32_backward_extra_bytes(const Plan& p);
hipError_t f32_backward_bidir(const Plan& p, const float* XQ, const float* XK, const float* V, const float* mu,
                              const float* s2, const float* pi, float eps, const float* dO, float* dXQ, float* dXK,
                              float* dV, float* dmu, float* ds2, float* dpi, char* ws, hipStream_t st);

// Backward of the causal forward (fp32): workspace beyond the causal plan's own, and the launcher.
size_t f32_backward_causal_extra_bytes(const Plan& p);
// state_in: the carried memory before the call, dstate_out: the gradient of the memory after it,
// dstate_in: the gradient of state_in (all [P][K][d_v+1] fp32, NULL for none).
hipError_t f32_backward_causal(const Plan& p, const float* XQ, const float* XK, const float* V, const float* mu,
                               const float* s2, const float* pi, float eps, const float* dO, float* dXQ, float* dXK,
                               float* dV, float* dmu, float* ds2, float* dpi, char* ws, hipStream_t st,
                               const float* state_in = nullptr, const float* dstate_out = nullptr,
                               float* dstate_in = nullptr);

// bf16 <-> fp32 copies of n elements (the staging of the backward's bf16 I/O).
hipError_t widen_bf16(const void* src, float* dst, size_t n, hipStream_t st);
hipError_t narrow_to_bf16(const float* src, void* dst, size_t n, hipStream_t st);

// ---- responsibility diagnostics (gma_diag.hip) ---------------------------------
// Workspace: Gamma [B][H][N][K] fp32, then per-block partial sums, then the responsibilities
// plan's own workspace.
size_t diag_gamma_bytes(const Plan& p);
size_t diag_partials_bytes(const Plan& p);
hipError_t diagnostics(const Plan& p, const Plan& resp, const void* X, const float* mu, const float* s2,
                       const float* pi, float* usage, float* stats, int32_t* argmax, float* gbar, char* ws,
                       hipStream_t st);

// ---- short causal calls (gma_decode.hip) --------------------------------------
// Causal calls of at most this many positions (decoding steps) run one workgroup per problem
// that walks its positions in order, instead of the chunked scan.
constexpr int64_t kDecodeMaxPositions = 8;
bool decode_applies(const Plan& p);
hipError_t causal_decode(const Plan& p, const void* XQ, const void* XK, const void* V, const float* mu,
                         const float* s2, const float* pi, float eps, void* O, hipStream_t st,
                         const float* state_in, float* state_out);

// ---- bf16 MFMA path (gma_bf16.hip) ---------------------------------------------
hipError_t bf16_responsibilities(const Plan& p, const void* X, const float* mu, const float* s2,
                                 const float* pi, void* Gamma, gma_dtype_t gamma_dtype, char* ws,
                                 hipStream_t st);
// Threads and static LDS bytes of one workgroup of the single-launch bidirectional kernel for
// these dims (d_r, component tiles of 32, value tiles of 32); zeros for unsupported dims.
void bf16_bidir_geometry(int64_t dr, int64_t kt, int64_t vt, int* threads, int64_t* lds_bytes);
// Workgroups of that kernel a CU keeps resident by its LDS and its declared waves per SIMD
// (every MI355X CU has 160 KiB of LDS and 4 SIMDs); at least 1.
int64_t bf16_bidir_per_cu(int64_t dr, int64_t kt, int64_t vt);
hipError_t bf16_bidir(const Plan& p, const void* XQ, const void* XK, const void* V,
                      const float* mu, const float* s2, const float* pi, float eps, void* O,
                      char* ws, hipStream_t st);
// Positions per chunk the bf16 causal scan runs for the plan's requested chunk.
int64_t bf16_causal_chunk(const Plan& p);
hipError_t bf16_causal(const Plan& p, const void* XQ, const void* XK, const void* V,
                       const float* mu, const float* s2, const float* pi, float eps, void* O,
                       char* ws, hipStream_t st, const float* state_in, float* state_out);
// Causal forward for 256 padded components with d_r <= 64 (gma_bf16_wide.hip): one launch of
// 8-wave workgroups, the memory spread over the waves' registers.
bool bf16_causal_wide_applies(const Plan& p);
hipError_t bf16_causal_wide(const Plan& p, const void* XQ, const void* XK, const void* V, const float* mu,
                            const float* s2, const float* pi, float eps, void* O, char* ws, hipStream_t st,
                            const float* state_in, float* state_out);
// Segment aggregates (the first `splits` segments) into the partials region: the first
// launch of the causal path for shapes the fused causal kernel does not take.
hipError_t bf16_write_partials(const Plan& p, const void* XK, const void* V, const float* mu, const float* s2,
                               const float* pi, char* ws, hipStream_t st, int64_t splits);

}  // namespace gma
