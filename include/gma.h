/*
 * gma.h -- C ABI of libgma.so, the MI355X (gfx950) forward pass of Gaussian
 * Mixture Attention (GMA), after "Gaussian Mixture Attention: Linear-Time Sequence
 * Mixing via Probabilistic Latent Routing" (Huang & Raza).
 *
 * Problem statement (Sec. 3.2-3.5 of that paper).  For every batch entry b and head h
 * there are N routing vectors of dimension d_r for queries (X_Q) and keys (X_K), N
 * value vectors of dimension d_v (V), and one diagonal Gaussian mixture with K
 * components shared by queries and keys of that head (Fig. 1, "Shared GMM
 * Parameters"): means mu, variances sigma2 (the diagonal of Sigma_k) and priors pi.
 *   responsibilities   Gamma = softmax_k(s),  s_k = log pi_k + log N(x | mu_k, Sigma_k)
 *                      (Sec. 3.2 Eq. 2-3, Sec. 4.1 Eq. 16 and Eq. 3b)
 *   bidirectional      Vt = Gamma_K^T V,  Z = Gamma_K^T 1           (Sec. 3.3 Eq. 5-6)
 *                      O  = Gamma_Q Vt / (Gamma_Q Z + eps)           (Eq. 7-8)
 *   causal             Vt, Z replaced by prefix sums over j <= i     (Sec. 3.5 Eq. 6b, 8b)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout      All tensors are dense, contiguous and row-major:
 *               X, X_Q, X_K [B, H, N, d_r]   V, O [B, H, N, d_v]   Gamma [B, H, N, K]
 *               mu, sigma2  [H, K, d_r]      pi   [H, K]
 *             Parameters are per head and broadcast over the batch.
 * Dtypes      X_Q, X_K, V and O share one I/O dtype (GMA_F32 or GMA_BF16).  The
 *             parameters mu, sigma2, pi are always fp32.  eps is fp32.
 * Memory      Every pointer is a device pointer (HBM) owned by the caller.  The library
 *             never allocates or frees device memory and keeps no state between calls
 *             apart from the optional kernel-timing record (gma_profiling) and one
 *             device error word per device (gma_device_status); scratch space is the
 *             caller's workspace (size from gma_workspace_size).
 *             O and Gamma must not overlap any input or the workspace.
 * Alignment   Tensor pointers and the workspace must be 16-byte aligned
 *             (GMA_ERR_MISALIGNED otherwise).
 * Streams     Work is enqueued on `stream` (NULL = the device's null stream) and the call
 *             returns without waiting.  Calls on different streams must use different
 *             workspaces.  The single-launch bf16 forwards (gma_forward_bidir,
 *             gma_forward_cross, gma_forward_causal and gma_forward_causal_state) hand data
 *             between the workgroups of one launch and rely on the device dispatching them
 *             (bidirectional: all of the launch's workgroups resident at once; the host
 *             checks the grid against the device's occupancy and otherwise runs the phases
 *             as separate launches, as it also does with more than 8 splits per problem,
 *             where the separate launches measure faster).  A kernel running concurrently on another stream can
 *             hold the compute units those workgroups need; a hand-off wait then runs out
 *             after a bounded time, the affected output rows are NaN and gma_device_status
 *             reports GMA_ERR_TIMEOUT.  Callers that run forwards concurrently on one device
 *             turn the single launches off with gma_set_single_launch(0).
 * Pointers    A tensor pointer may be NULL when the tensor has no elements (e.g. N = 0);
 *             the parameters, the shape and a workspace of nonzero size may not.
 * Errors      Arguments are validated on the host before any HIP call; a non-OK status
 *             means nothing was enqueued.  GMA_ERR_HIP reports a failed launch.  Faults
 *             inside a kernel surface at the caller's next synchronisation.  Device-side
 *             preconditions that are not checked: sigma2 > 0, pi > 0, finite inputs
 *             (violations propagate NaN or infinities into the outputs).
 * Sizes       B, H, N >= 0; a problem with B*H*N == 0 is valid and enqueues nothing.
 *             d_r, d_v, K must lie in the supported set (GMA_ERR_UNSUPPORTED otherwise):
 *               GMA_F32  : 1 <= d_r <= 128, 1 <= d_v <= 128, 1 <= K <= 256
 *               GMA_BF16 : d_r in {16, 32, 64, 128}, d_v in {32, 64, 128}, 1 <= K <= 256
 * Numerics    Scores and softmax in fp32, accumulations in fp32.  bf16 I/O uses bf16
 *             MFMA with split (hi + lo) operands for the scores and for the latent
 *             memory, and rounds O to bf16 (nearest-even).  Results are bitwise
 *             reproducible for a fixed shape and chunk length: reductions run in a fixed
 *             order, and the only atomics are the hand-off words between the phases of
 *             one launch (see gma_set_wait_limit).
 */
#ifndef GMA_H
#define GMA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GMA_OK = 0,
    GMA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL                        */
    GMA_ERR_BAD_SHAPE = 2,           /* negative size                                     */
    GMA_ERR_BAD_VALUE = 3,           /* eps <= 0 or not finite; unknown dtype or op       */
    GMA_ERR_UNSUPPORTED = 4,         /* d_r, d_v, K or chunk outside the supported set    */
    GMA_ERR_MISALIGNED = 5,          /* pointer not 16-byte aligned                       */
    GMA_ERR_WORKSPACE_TOO_SMALL = 6, /* workspace_bytes < gma_workspace_size(...)         */
    GMA_ERR_HIP = 7,                 /* a HIP runtime call or kernel launch failed        */
    GMA_ERR_TIMEOUT = 8              /* gma_device_status: a hand-off wait inside a
                                        single-launch forward ran out (see there)         */
} gma_status_t;

typedef enum { GMA_F32 = 0, GMA_BF16 = 1 } gma_dtype_t;

typedef enum {
    GMA_OP_RESPONSIBILITIES = 0,
    GMA_OP_BIDIR = 1,
    GMA_OP_CAUSAL = 2,
    GMA_OP_DIAGNOSTICS = 3,
    GMA_OP_BACKWARD_BIDIR = 4,
    GMA_OP_BACKWARD_CAUSAL = 5
} gma_op_t;

/* Problem sizes: batch B, heads H, sequence length N, routing dim d_r, value dim d_v,
 * number of mixture components K (Sec. 3.2-3.3 notation). */
typedef struct {
    int64_t B, H, N, d_r, d_v, K;
} gma_shape_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* gma_status_string(gma_status_t status);

/*
 * Workspace bytes that `op` needs for `shape` with I/O dtype `io_dtype` (and causal
 * chunk length `chunk`, ignored for other ops).  Depends only on its arguments, never
 * on the device.  For GMA_OP_RESPONSIBILITIES d_v is ignored.  Writes *bytes_out on
 * success; same validation and error codes as the op itself.
 */
gma_status_t gma_workspace_size(gma_op_t op, const gma_shape_t* shape, gma_dtype_t io_dtype,
                                int32_t chunk, size_t* bytes_out);

/*
 * Responsibilities Gamma[b,h,n,:] of every routing vector X[b,h,n,:] under head h's
 * mixture: Sec. 3.2 Eq. 3, evaluated as the softmax of Eq. 3b over the scores of
 * Sec. 4.1 Eq. 16 (the k-independent -(d_r/2) log 2 pi is dropped; it cancels).
 *   X       [B,H,N,d_r] in x_dtype          mu, sigma2 [H,K,d_r] fp32, pi [H,K] fp32
 *   Gamma   [B,H,N,K] out, in gamma_dtype (GMA_F32 or GMA_BF16)
 * shape->d_v is ignored.  Every output row is non-negative and sums to 1 up to the
 * output rounding.
 */
gma_status_t gma_responsibilities(const void* X, gma_dtype_t x_dtype,
                                  const float* mu, const float* sigma2, const float* pi,
                                  void* Gamma, gma_dtype_t gamma_dtype,
                                  const gma_shape_t* shape,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Bidirectional GMA forward, Sec. 3.3 Eq. 5-8:
 *   Vt = Gamma_K^T V,  Z = Gamma_K^T 1_N,  O_i = (Gamma_Q Vt)_i / ((Gamma_Q Z)_i + eps)
 * with Gamma_Q, Gamma_K the responsibilities of X_Q and X_K (see gma_responsibilities).
 * eps > 0 is added once to each row denominator (footnote 4 of Sec. 3.3).  Gamma is
 * never written to memory; Vt and Z live in the workspace.
 *   XQ, XK [B,H,N,d_r], V [B,H,N,d_v], O [B,H,N,d_v] out, all in io_dtype.
 * With bf16 I/O the whole forward is one kernel launch whose workgroups hand the split
 * partials and the combined memory to one another through the workspace (flag words
 * compared with a fresh per-call value, so the workspace may hold anything on entry).
 */
gma_status_t gma_forward_bidir(const void* XQ, const void* XK, const void* V,
                               gma_dtype_t io_dtype,
                               const float* mu, const float* sigma2, const float* pi,
                               float eps, void* O, const gma_shape_t* shape,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gma_forward_bidir without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It makes no allocation of any kind: its scratch is a static device array of
 * GMA_STATIC_SCRATCH_BYTES inside the library, one per device, resolved when the first call on
 * that device (or gma_device_status) runs there and held until the process ends.  Shapes whose
 * workspace (gma_workspace_size(GMA_OP_BIDIR, ...)) exceeds that size are rejected with
 * GMA_ERR_WORKSPACE_TOO_SMALL before any HIP call.  Every call on a device shares that device's
 * array and the kernels leave their contents in it: calls that overlap on one device (several
 * streams, several host threads) race and must be serialised by the caller.  The kernels never
 * read scratch they did not write in the same call, so no clearing is needed.  Arguments, results
 * (bitwise those of gma_forward_bidir), dtypes and errors otherwise as for gma_forward_bidir.
 */
#define GMA_STATIC_SCRATCH_BYTES (32u << 20)
gma_status_t gma_forward_bidir_noalloc(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                       const float* mu, const float* sigma2, const float* pi, float eps, void* O,
                                       const gma_shape_t* shape, hipStream_t stream);

/*
 * Causal GMA forward, Sec. 3.5 Eq. 6b and 8b:
 *   Vt^(i) = sum_{j<=i} gammaK_j V_j^T,  Z^(i) = sum_{j<=i} gammaK_j   (inclusive of i)
 *   O_i    = gammaQ_i Vt^(i) / (gammaQ_i Z^(i) + eps)
 * computed as a chunked scan: the sequence is cut into chunks of `chunk` positions;
 * inside a chunk the masked product (Gamma_Q Gamma_K^T restricted to j <= i) is formed
 * on chip and the K x (d_v+1) running memory carries the prefix across chunks.
 * `chunk` must be 16, 32, 64 or 128 (GMA_ERR_UNSUPPORTED otherwise; with bf16 I/O 16 is
 * unsupported too, as the bf16 scans form their scores on 32-position tiles).  It is the most
 * positions a step takes on chip: each kernel runs the largest power of two not above it that
 * its tiles allow in LDS and registers (64 at most on the bf16 path, 32 for 256 components);
 * gma_plan_info reports the length used.  Only the order of the sums depends on it.  Output row i depends
 * only on inputs at positions <= i.  Arguments as for gma_forward_bidir.  With bf16 I/O,
 * K <= 128 (d_r * K <= 8192) or 256 padded components with d_r <= 64, the forward is one
 * launch: each segment's workgroup publishes its segment aggregate in the workspace and
 * waits for those of the segments before it (same flag scheme as gma_forward_bidir); other
 * shapes take two launches.  The 256-component form also keeps the keys' responsibilities
 * of every position in the workspace (B*H*N*512 bytes) between its key pass and its scan.
 */
gma_status_t gma_forward_causal(const void* XQ, const void* XK, const void* V,
                                gma_dtype_t io_dtype,
                                const float* mu, const float* sigma2, const float* pi,
                                float eps, void* O, const gma_shape_t* shape, int32_t chunk,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Causal GMA with a carried memory: Sec. 3.5 Eq. 6b read as a recurrence, the prefix memory
 * after position i being the memory after position i-1 plus gammaK_i [V_i | 1].  A call
 * continues the sequence from the memory of all positions before its first one:
 *   state_in   [B,H,K,d_v+1] fp32, row k = Vt_k (d_v values) then Z_k: the memory before
 *              position 0 of this call.  NULL means an empty memory (then this is
 *              gma_forward_causal).
 *   state_out  [B,H,K,d_v+1] fp32, same layout: the memory after this call's last position,
 *              i.e. state_in plus gammaK_j [V_j | 1] summed over every position j of the call.
 *              NULL skips it.  Must not overlap state_in.
 *   O_i = gammaQ_i (Vt_in + sum_{j<=i} gammaK_j V_j^T) / (gammaQ_i (Z_in + sum_{j<=i} gammaK_j) + eps)
 * Processing a sequence in consecutive pieces, each call's state_out being the next call's
 * state_in, gives the outputs of one call over the whole sequence (up to the order of the
 * sums); pieces of N = 1 are single-token decoding.  With N = 0 state_out receives state_in
 * (zeros if state_in is NULL).  All other arguments, errors and the workspace (size from
 * gma_workspace_size with GMA_OP_CAUSAL) are those of gma_forward_causal.  state_in and
 * state_out must be 16-byte aligned.
 */
gma_status_t gma_forward_causal_state(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                      const float* mu, const float* sigma2, const float* pi, float eps,
                                      void* O, const gma_shape_t* shape, int32_t chunk,
                                      const float* state_in, float* state_out,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Cross-attention (Sec. 3, "Cross-attention"): queries are formed from a query-side
 * sequence X and keys and values from a separate context sequence Y; the routing of
 * Sec. 3.3 is applied with Gamma^Q of X and Gamma^K of Y, through the same mixture:
 *   Vt = Gamma_K^T V,  Z = Gamma_K^T 1_{Nk},  O_i = (Gamma_Q Vt)_i / ((Gamma_Q Z)_i + eps)
 * Sizes are given by gma_cross_shape_t: N_q query rows, N_k context rows.
 *   XQ [B,H,N_q,d_r], XK [B,H,N_k,d_r], V [B,H,N_k,d_v], O [B,H,N_q,d_v] out, in io_dtype.
 * N_q, N_k >= 0.  An empty context (N_k = 0, N_q > 0) is valid: Vt = 0 and Z = 0, so every
 * output row is 0.  XK and V may be NULL when N_k = 0, XQ and O when N_q = 0.  With N_q = N_k = N this is gma_forward_bidir.  Conventions, dtypes,
 * supported d_r, d_v, K, errors and the workspace contract are those of gma_forward_bidir;
 * the workspace size comes from gma_cross_workspace_size.  With bf16 I/O the forward is one
 * launch (same hand-off scheme as gma_forward_bidir).
 */
typedef struct {
    int64_t B, H, N_q, N_k, d_r, d_v, K;
} gma_cross_shape_t;

gma_status_t gma_cross_workspace_size(const gma_cross_shape_t* shape, gma_dtype_t io_dtype, size_t* bytes_out);

gma_status_t gma_forward_cross(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                               const float* mu, const float* sigma2, const float* pi, float eps,
                               void* O, const gma_cross_shape_t* shape,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Responsibility diagnostics (Sec. 5.4, Eq. 24-29) of routing vectors X [B,H,N,d_r] of B
 * sequences of N positions (for instance the query projections of a layer), each head with
 * its own mixture; T = B N token occurrences t = (b, n):
 *   gbar[t,k] = (1/H) sum_h gamma[b,h,n,k]                       head-averaged responsibility (Eq. 24)
 *   usage[k]  = (1/T) sum_t gbar[t,k]                            marginal component usage    (Eq. 25)
 *   stats[0]  = H_usage = -sum_k usage_k log usage_k / log K     usage entropy               (Eq. 26)
 *   stats[1]  = H_token = (1/T) sum_t (-sum_k gbar log gbar) / log K   mean token entropy    (Eq. 27)
 *   stats[2]  = R_max   = (1/T) sum_t max_k gbar[t,k]            mean maximum responsibility (Eq. 28)
 *   argmax[t] = argmax_k gbar[t,k], the lowest k among equal maxima      hard assignment     (Eq. 29)
 * with gamma the responsibilities of gma_responsibilities.  0 log 0 is 0; with K = 1 both
 * normalised entropies are reported as 0; T = 0 gives zeros.
 *   usage  [K] fp32 out, stats [3] fp32 out (required);
 *   argmax [B,N] int32 out and gbar [B,N,K] fp32 out (optional, NULL to skip).
 * Workspace: gma_workspace_size(GMA_OP_DIAGNOSTICS, shape, x_dtype, 0, ...) (shape->d_v is
 * ignored): per-block partial sums, and for fp32 input the responsibilities of every head
 * (B H N K fp32); bf16 input (except d_r = 128 with K > 128) is processed by one fused kernel that
 * needs only per-head operand tables.  Sums run in a fixed order (bitwise reproducible).  Sizes, dtypes and errors as
 * for gma_responsibilities.
 */
gma_status_t gma_responsibility_diagnostics(const void* X, gma_dtype_t x_dtype, const float* mu, const float* sigma2,
                                            const float* pi, const gma_shape_t* shape, float* usage, float* stats,
                                            int32_t* argmax, float* gbar, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/*
 * Backward pass of the bidirectional forward (gma_forward_bidir) for the loss gradient dO:
 * the gradients of <dO, O> with respect to every input, Sec. 4.1 Eq. 17-20.  With the
 * forward's Vt, Z, D_i = (Gamma_Q Z)_i + eps and a_i = dO_i . O_i, the upstream gradients at
 * the responsibilities are
 *   g^Q_ik = (dO_i . Vt_k - a_i Z_k) / D_i                 (query side)
 *   g^K_jk = dVt_k . V_j + dZ_k                            (key side)
 * with dVt_k = sum_i Gamma_Q[i,k] dO_i / D_i and dZ_k = -sum_i Gamma_Q[i,k] a_i / D_i; they pass
 * the softmax Jacobian as ds_ik = gamma_ik (g_ik - sum_l gamma_il g_il) (Eq. 18) and reach the
 * routing vectors and the mixture parameters through the score of Eq. 16 (Eq. 19-20):
 *   dX[i,d] = -sum_k ds_ik (x_id - mu_kd) / sigma2_kd, dmu[k,d] = sum_i ds_ik (x_id - mu_kd) / sigma2_kd,
 *   dsigma2[k,d] = sum_i ds_ik ((x_id - mu_kd)^2 / sigma2_kd^2 - 1 / sigma2_kd) / 2,
 *   dpi[k] = sum_i ds_ik / pi_k      (pi as passed in; its parameterisation lies upstream),
 * the parameter sums running over both sides, every sequence and every position.  Also
 *   dV[j,:] = sum_k Gamma_K[j,k] dVt_k.
 *   XQ, XK, dXQ, dXK [B,H,N,d_r]; V, dO, dV [B,H,N,d_v] in io_dtype (GMA_F32 or GMA_BF16);
 *   mu, sigma2, dmu, dsigma2 [H,K,d_r] and pi, dpi [H,K] fp32.  The arithmetic is fp32 at either
 *   I/O dtype; bf16 inputs are widened exactly and bf16 outputs rounded to nearest even.  The
 *   gradient outputs are overwritten, not accumulated into.
 * Workspace: gma_workspace_size(GMA_OP_BACKWARD_BIDIR, shape, io_dtype, 0, ...): the forward's
 * memory and its split partials, the same for (dVt, dZ), and per-split parameter partials,
 * reduced in a fixed order (bitwise reproducible); for K, d_r, d_v <= 64 (multiples of 4) the
 * responsibilities of the keys, which the key pass reads back (B H N K fp32); for 64 < K <= 256
 * with d_r, d_v <= 64 (multiples of 4) the responsibilities of both sides (2 B H N K fp32), three
 * fp32 values per row and the component blocks' shares of dX (ceil(K / 64) B H N d_r fp32); with
 * bf16 I/O also
 * fp32 copies of the four inputs and three outputs (O(B H N (d_r + d_v)) bytes).  Sizes as for
 * the fp32 forward (d_r, d_v <= 128, K <= 256 at either I/O dtype); alignment and errors as for
 * gma_forward_bidir; with no rows (B N = 0) the parameter gradients are zeros.
 */
gma_status_t gma_backward_bidir(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                const float* mu, const float* sigma2, const float* pi, float eps,
                                const void* dO, void* dXQ, void* dXK, void* dV, float* dmu, float* dsigma2,
                                float* dpi, const gma_shape_t* shape, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Backward pass of the causal forward (gma_forward_causal): the gradients of <dO, O> with
 * respect to every input, Sec. 4.1 Eq. 17-20 through the prefix memory of Sec. 3.5 Eq. 6b, 8b.
 * Position i reads Vt^(i), Z^(i) over j <= i, so with D_i = (Gamma_Q Z^(i))_i + eps and
 * a_i = dO_i . O_i the query side is
 *   g^Q_ik = (dO_i . Vt^(i)_k - a_i Z^(i)_k) / D_i,
 * and key position j receives the suffix sums over the positions that read it:
 *   dVt_j = sum_{i>=j} Gamma_Q[i,:]^T dO_i / D_i,  dZ_j = -sum_{i>=j} Gamma_Q[i,:] a_i / D_i,
 *   dV[j,:] = sum_k Gamma_K[j,k] dVt_j[k,:],        g^K_jk = dVt_j[k,:] . V_j + dZ_j[k];
 * the softmax Jacobian, the routing-vector and the parameter gradients are those of
 * gma_backward_bidir.  Shapes, dtypes, outputs, workspace
 * (gma_workspace_size(GMA_OP_BACKWARD_CAUSAL, shape, io_dtype, 0, ...), which also holds D_i and
 * a_i of every position and, where the register-tiled passes apply, the responsibilities of both
 * sides, 2 B H N K fp32; where the K-blocked causal passes apply (K <= 256, d_r, d_v <= 64, not
 * within the register-tiled passes' LDS), the same, the memory before and what the later
 * positions send for every tile of 64 positions (2 B H ceil(N / 64) K (d_v + 1) fp32), the
 * in-tile products (B H ceil(N / 64) 64 64 fp32), three fp32 values per row and the component
 * blocks' shares of dX (ceil(K / 64) B H N d_r fp32)) and errors as for gma_backward_bidir.
 */
gma_status_t gma_backward_causal(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                 const float* mu, const float* sigma2, const float* pi, float eps,
                                 const void* dO, void* dXQ, void* dXK, void* dV, float* dmu, float* dsigma2,
                                 float* dpi, const gma_shape_t* shape, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Backward pass of a causal call continued from a carried memory (gma_forward_causal_state):
 * the gradients of <dO, O> + <dstate_out, state_out>.  Every prefix memory of the call includes
 * state_in, and the memory after the call depends on every key position with weight one, so
 * dstate_out is added to every key position's memory gradient (dVt_j, dZ_j of
 * gma_backward_causal), and
 *   dstate_in[k, :d_v] = dstate_out[k, :d_v] + sum_i Gamma_Q[i,k] dO_i / D_i,
 *   dstate_in[k, d_v]  = dstate_out[k, d_v]  - sum_i Gamma_Q[i,k] a_i / D_i
 * (sum over every position of the call).  Chained over calls (each call's dstate_in passed as the
 * previous call's dstate_out) this is the backward of one pass over the whole sequence.
 *   state_in, dstate_out: [B,H,K,d_v+1] fp32 (row k: Vt_k, then Z_k), NULL for zeros;
 *   dstate_in: [B,H,K,d_v+1] fp32 out, NULL to skip; it must not overlap state_in or dstate_out.
 * A call without positions returns dstate_in = dstate_out and zero parameter gradients.  Other
 * arguments, the workspace (GMA_OP_BACKWARD_CAUSAL) and errors as for gma_backward_causal.
 */
gma_status_t gma_backward_causal_state(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                       const float* mu, const float* sigma2, const float* pi, float eps,
                                       const void* dO, const float* state_in, const float* dstate_out, void* dXQ,
                                       void* dXK, void* dV, float* dmu, float* dsigma2, float* dpi,
                                       float* dstate_in, const gma_shape_t* shape, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * Backward pass of cross-attention (gma_forward_cross): the gradients of <dO, O> with the
 * formulas of gma_backward_bidir, Gamma_Q taken over the N_q query rows and Gamma_K over the N_k
 * context rows (Sec. 3 "Cross-attention"; Sec. 4.1 Eq. 17-20).
 *   XQ, dXQ [B,H,N_q,d_r]; dO [B,H,N_q,d_v]; XK, dXK [B,H,N_k,d_r]; V, dV [B,H,N_k,d_v] in io_dtype;
 *   mu, sigma2, pi and their gradients fp32, as for gma_backward_bidir.
 * An empty context (N_k = 0) gives O = 0, so dXQ and the parameter gradients are zeros; no queries
 * (N_q = 0) give zeros everywhere.  A side without rows may come without storage.
 * Workspace: gma_backward_cross_workspace_size (same validation and errors as the call).  With
 * N_q = N_k it equals the bidirectional backward on the same tensors.
 */
gma_status_t gma_backward_cross_workspace_size(const gma_cross_shape_t* shape, gma_dtype_t io_dtype,
                                               size_t* bytes_out);
gma_status_t gma_backward_cross(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                const float* mu, const float* sigma2, const float* pi, float eps,
                                const void* dO, void* dXQ, void* dXK, void* dV, float* dmu, float* dsigma2,
                                float* dpi, const gma_cross_shape_t* shape, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Kernel timing (optional tracing).  While enabled, every kernel the library launches is
 * bracketed by a pair of hipEvents recorded on the launch stream; gma_profiling_collect
 * waits for the recorded events, adds each launch's elapsed time to a per-kernel total,
 * writes up to `capacity` entries (kernel name, launches, total milliseconds) and
 * clears the record.  Names are static strings owned by the library.  Events are host
 * objects created and destroyed by the library (no device memory).  Recording adds one
 * event packet before and after each launch.  Not thread-safe against concurrent calls
 * from other host threads while enabled.
 *   gma_profiling(1) enables, gma_profiling(0) disables and drops anything uncollected.
 */
typedef struct {
    const char* name;
    int64_t launches;
    double total_ms;
} gma_kernel_stat_t;

gma_status_t gma_profiling(int enable);
gma_status_t gma_profiling_collect(gma_kernel_stat_t* stats, int capacity, int* count);

/*
 * Bound on the hand-off waits of the single-launch bf16 forwards.  Each of those launches
 * runs several phases, and a workgroup waits for data that other workgroups of the same
 * launch publish (the split partials and memory slices of a bidirectional problem; the
 * aggregates of the earlier segments of a causal problem).  The waits poll at most `polls`
 * times (each poll is a device-wide load followed by a short sleep).  A workgroup whose
 * wait exceeds the bound stops waiting, publishes nothing further, writes NaN over its
 * output rows (and the carried memory, if it produces it) and raises the device error that
 * gma_device_status reports, so a launch always terminates and a failure is never silent.  The default, GMA_WAIT_LIMIT_DEFAULT polls, is far above any wait of
 * a healthy launch (well under a second in total).  0 makes every such wait fail at
 * once.  That setting exists so that tests can exercise the failure path.  The value is
 * process-wide and read when a forward is enqueued.
 */
#define GMA_WAIT_LIMIT_DEFAULT (1u << 18)
gma_status_t gma_set_wait_limit(uint32_t polls);

/*
 * Device-side failures of earlier calls on the current device.  Waits for `stream`, then
 * returns GMA_ERR_TIMEOUT if, since the previous gma_device_status on this device, a
 * single-launch forward's hand-off wait ran out (gma_set_wait_limit; its output rows, and
 * the carried memory of a causal call, were then written as NaN), GMA_OK if not, and
 * GMA_ERR_HIP if the query itself failed.  Taking the status clears it.  The library keeps
 * one error word per device (a static device variable, the only state it keeps besides the
 * profiling record); kernels raise it with an atomic OR, and this call exchanges it with
 * zero on the device, so a failure raised meanwhile by work on another stream is reported
 * by this call or the next one, never lost.
 */
gma_status_t gma_device_status(hipStream_t stream);

/*
 * Whether the bf16 forwards may run as single launches whose workgroups hand data to one
 * another (1, the default) or must run their phases as separate launches in which no
 * workgroup waits for another (0): bidirectional and cross-attention forwards as write,
 * combine and read launches; causal forwards as the segment aggregates followed by the
 * scan.  Results are bitwise identical in both modes.  0 is for callers that run several
 * forwards concurrently on one device (see Streams above).  Process-wide, read when a
 * forward is enqueued.
 */
gma_status_t gma_set_single_launch(int enable);

/*
 * How a forward of `op` (GMA_OP_BIDIR or GMA_OP_CAUSAL) on `shape` is split, for inspection
 * and tests; device-independent, like the workspace size.  Same validation and errors as
 * gma_workspace_size.  GMA_OP_BACKWARD_BIDIR and GMA_OP_BACKWARD_CAUSAL give the backward's
 * splits (`chunk` ignored; the fields below the first three are then 0).
 *   splits                 sequence splits (bidirectional) or segments (causal) per problem
 *   rows_per_split         positions per split (the last may be shorter)
 *   workgroups             B H splits: the grid of the single launch (backward: of the row passes)
 *   threads_per_workgroup  }  bf16 bidirectional only (0 otherwise): the single-launch
 *   lds_bytes              }  kernel's workgroup size and static LDS,
 *   waits_on_all_splits    }  1 if the single launch is planned (2 to 8 splits per problem)
 *                              and its workgroups wait on every split of their problem,
 *   resident_bound         }  and the workgroups that the kernel's LDS and declared waves
 *                              per SIMD let a 256-CU MI355X keep resident at once
 *                              (workgroups <= resident_bound whenever waits_on_all_splits)
 *   chunk_used             causal only (0 otherwise): the positions per chunk the scan runs for
 *                          the requested `chunk` (see gma_forward_causal)
 */
typedef struct {
    int64_t splits, rows_per_split, workgroups;
    int64_t threads_per_workgroup, lds_bytes, waits_on_all_splits, resident_bound;
    int64_t chunk_used;
} gma_plan_info_t;

gma_status_t gma_plan_info(gma_op_t op, const gma_shape_t* shape, gma_dtype_t io_dtype, int32_t chunk,
                           gma_plan_info_t* info);

#ifdef __cplusplus
}
#endif

#endif /* GMA_H */
