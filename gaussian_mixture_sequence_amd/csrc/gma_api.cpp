// C-ABI front end of libgma.so: argument validation, workspace planning and
// dispatch to the fp32 (VALU) or bf16 (MFMA) kernel launchers.  Declarations and
// the contract of every entry point are in include/gma.h.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <random>
#include <string>
#include <vector>

#include "gma_internal.h"

namespace gma {

namespace {

constexpr int64_t kTokenTile = 64;      // tokens per tile in every kernel family
constexpr int64_t kBidirBlocks = 512;   // target workgroups for the split-N write and the read
                                        // (two resident per CU: one wave of workgroups)
constexpr int64_t kCausalBlocks = 512;  // target workgroups for the segmented scan
constexpr int64_t kBackwardBlocks = 2048;       // target workgroups of the causal backward's segments
constexpr int64_t kBackwardBidirBlocks = 512;   // ... and of the bidirectional backward's splits
constexpr int64_t kDeviceCUs = 256;        // compute units of an MI355X (planning is device-independent)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tiles of 32 components the bf16 kernels are compiled for: the smallest of 1, 2, 4, 8 that
// holds K (K <= 256 is checked before).
int64_t bf16_component_tiles(int64_t K) {
    const int64_t t = cdiv(std::max<int64_t>(K, 1), 32);
    return t <= 1 ? 1 : t <= 2 ? 2 : t <= 4 ? 4 : 8;
}

gma_status_t check_dims(gma_op_t op, const gma_shape_t& s, gma_dtype_t io) {
    if (s.B < 0 || s.H < 0 || s.N < 0) return GMA_ERR_BAD_SHAPE;
    if (s.d_r < 1 || s.K < 1) return GMA_ERR_UNSUPPORTED;
    const bool has_values = op == GMA_OP_BIDIR || op == GMA_OP_CAUSAL || op == GMA_OP_BACKWARD_BIDIR ||
                            op == GMA_OP_BACKWARD_CAUSAL;
    if (has_values && s.d_v < 1) return GMA_ERR_UNSUPPORTED;
    if (s.K > 256) return GMA_ERR_UNSUPPORTED;
    if (io == GMA_F32) {
        if (s.d_r > 128) return GMA_ERR_UNSUPPORTED;
        if (has_values && s.d_v > 128) return GMA_ERR_UNSUPPORTED;
    } else {
        if (s.d_r != 16 && s.d_r != 32 && s.d_r != 64 && s.d_r != 128) return GMA_ERR_UNSUPPORTED;
        if (has_values && s.d_v != 32 && s.d_v != 64 && s.d_v != 128)
            return GMA_ERR_UNSUPPORTED;
    }
    // guard the int64 products used for sizes
    const int64_t lim = int64_t(1) << 40;
    if (s.B > lim || s.H > lim || s.N > lim || (s.B * s.H) > lim || (s.B * s.H > 0 && s.N > lim / (s.B * s.H)))
        return GMA_ERR_BAD_SHAPE;
    return GMA_OK;
}

}  // namespace

void layout(Plan* pl);

// Splits of the backward passes, which walk each split's rows in tiles of kTokenTile and keep
// one workgroup per split (and component block): about `blocks` workgroups in all, each split a
// multiple of the tile (the forwards' splits follow their own kernels' occupancy, and at B8 H8
// N1024 the bidirectional one left half the CUs idle).  The causal passes walk their segments
// in order and take finer ones; each bidirectional split also writes partial records, so those
// stay coarser.  Both sides take the same count of splits; the regions are laid out again.
void backward_split(Plan* pl, int64_t blocks) {
    const int64_t n = std::max(pl->N, pl->Nq);
    if (pl->P <= 0 || n <= 0) return;
    const int64_t g = std::max<int64_t>(1, std::min(cdiv(blocks, pl->P), cdiv(n, kTokenTile)));
    pl->seg = round_up(size_t(cdiv(std::max<int64_t>(pl->N, 1), g)), kTokenTile);
    pl->seg_q = round_up(size_t(cdiv(std::max<int64_t>(pl->Nq, 1), g)), kTokenTile);
    pl->G = std::max<int64_t>(1, std::max(cdiv(pl->N, pl->seg), cdiv(pl->Nq, pl->seg_q)));
    layout(pl);
}

// Workgroups the bidirectional split aims at.  The bf16 forward runs as one launch whose
// workgroups wait on every other workgroup of their problem, so there the whole grid must be
// resident at once: P G stays within what the kernel's LDS and declared waves let every CU
// of a 256-CU MI355X hold (for P beyond that, one split per problem, which waits on nothing
// else).  The fp32 forward runs its phases as separate launches and takes two per CU.
int64_t bidir_split_target(const Plan& p) {
    if (p.io != GMA_BF16) return kBidirBlocks;
    return kDeviceCUs * bf16_bidir_per_cu(p.dr, p.Kp / 32, p.dv / 32);
}

// fp32 copies of X_Q, X_K, V, dO (inputs) and dX_Q, dX_K, dV (outputs) for a bf16 backward, in
// that order after the fp32 passes' regions (query-side arrays of N_q rows, key-side of N).
struct StageLayout {
    size_t off[7];  // XQ, XK, V, dO, dXQ, dXK, dV
    size_t total;
};
StageLayout stage_layout(const Plan& p) {
    const size_t rq = round_up(size_t(p.P * p.Nq * p.dr) * 4, 256), rk = round_up(size_t(p.P * p.N * p.dr) * 4, 256);
    const size_t vq = round_up(size_t(p.P * p.Nq * p.dv) * 4, 256), vk = round_up(size_t(p.P * p.N * p.dv) * 4, 256);
    const size_t sz[7] = {rq, rk, vk, vq, rq, rk, vk};
    StageLayout l{};
    for (int i = 0; i < 7; ++i) l.off[i] = l.total, l.total += sz[i];
    return l;
}
size_t backward_stage_bytes(const Plan& p) { return stage_layout(p).total; }

gma_status_t make_plan(gma_op_t op, const gma_shape_t& s, gma_dtype_t io, int32_t chunk, Plan* pl) {
    if (op != GMA_OP_RESPONSIBILITIES && op != GMA_OP_BIDIR && op != GMA_OP_CAUSAL && op != GMA_OP_DIAGNOSTICS &&
        op != GMA_OP_BACKWARD_BIDIR && op != GMA_OP_BACKWARD_CAUSAL)
        return GMA_ERR_BAD_VALUE;
    if (io != GMA_F32 && io != GMA_BF16) return GMA_ERR_BAD_VALUE;
    // the backward computes in fp32 at either I/O dtype, so it takes the fp32 size limits
    const bool backward = op == GMA_OP_BACKWARD_BIDIR || op == GMA_OP_BACKWARD_CAUSAL;
    gma_status_t st = check_dims(op, s, backward ? GMA_F32 : io);
    if (st != GMA_OK) return st;
    if (op == GMA_OP_BACKWARD_BIDIR || op == GMA_OP_BACKWARD_CAUSAL) {
        // the fp32 forward's plan, then the gradient scratch; bf16 I/O adds fp32 copies of the
        // inputs and outputs
        const bool causal = op == GMA_OP_BACKWARD_CAUSAL;
        if ((st = make_plan(causal ? GMA_OP_CAUSAL : GMA_OP_BIDIR, s, GMA_F32, causal ? 64 : 0, pl)) != GMA_OK)
            return st;
        backward_split(pl, causal ? kBackwardBlocks : kBackwardBidirBlocks);
        pl->op = op;
        pl->chunk = 0;
        pl->total += causal ? f32_backward_causal_extra_bytes(*pl) : f32_backward_extra_bytes(*pl);
        pl->off_stage = pl->total;
        if (io == GMA_BF16) {
            pl->io = io;
            pl->total += backward_stage_bytes(*pl);
        }
        return GMA_OK;
    }
    // causal chunk lengths 16, 32, 64 and 128; the bf16 scans form scores on 32-position subtiles
    if (op == GMA_OP_CAUSAL && chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return GMA_ERR_UNSUPPORTED;
    if (op == GMA_OP_CAUSAL && io == GMA_BF16 && chunk == 16) return GMA_ERR_UNSUPPORTED;

    Plan p{};
    p.op = op;
    p.io = io;
    p.B = s.B; p.H = s.H; p.N = s.N; p.dr = s.d_r;
    p.dv = (op == GMA_OP_BIDIR || op == GMA_OP_CAUSAL) ? s.d_v : 0;
    p.K = s.K;
    p.P = s.B * s.H;
    // bf16: K padded to 1, 2, 4 or 8 tiles of 32 components (the compiled MFMA tilings);
    // padded components get a score of -inf and so a responsibility of exactly 0
    p.Kp = (io == GMA_BF16) ? 32 * bf16_component_tiles(s.K) : s.K;
    p.chunk = (op == GMA_OP_CAUSAL) ? chunk : 0;

    // parameter tables: the fp32 path keeps 1/sigma2 and the score constant in fp64; the bf16
    // kernels build their operands from mu, sigma2 and pi in registers and keep none.
    if (io == GMA_F32)
        p.params_bytes = round_up(size_t(p.H * p.K) * 8, 256) + round_up(size_t(p.H * p.K * p.dr) * 8, 256);
    else
        p.params_bytes = 0;

    p.G = 1;
    p.seg = round_up(size_t(std::max<int64_t>(p.N, 1)), kTokenTile);
    if (op == GMA_OP_BIDIR && p.P > 0 && p.N > 0) {
        int64_t g = std::min(bidir_split_target(p) / p.P, cdiv(p.N, 512));
        g = std::max<int64_t>(g, 1);
        p.seg = round_up(size_t(cdiv(p.N, g)), kTokenTile);
        p.G = cdiv(p.N, p.seg);
    } else if (op == GMA_OP_CAUSAL && p.P > 0 && p.N > 0) {
        // segments per problem: every workgroup resident at once (two per CU), and the
        // busiest CU's share of positions (ceil(P g / 256) segments of `seg`) smallest;
        // ties go to fewer segments (less aggregate work)
        int64_t best_g = 1, best_cost = -1;
        for (int64_t g = 1; g <= std::min<int64_t>(16, cdiv(p.N, kTokenTile)); ++g) {
            if (g > 1 && p.P * g > kCausalBlocks) break;
            const int64_t seg = int64_t(round_up(size_t(cdiv(p.N, g)), kTokenTile));
            const int64_t cost = cdiv(p.P * g, 256) * seg;
            if (best_cost < 0 || cost < best_cost) best_cost = cost, best_g = g;
        }
        p.seg = round_up(size_t(cdiv(p.N, best_g)), kTokenTile);
        p.G = cdiv(p.N, p.seg);
    }
    p.Nq = p.N;
    p.seg_q = p.seg;
    layout(&p);
    if (op == GMA_OP_DIAGNOSTICS) {  // responsibilities of every head, partial sums, and their plan's scratch
        Plan r;
        st = make_plan(GMA_OP_RESPONSIBILITIES, s, io, 0, &r);
        if (st != GMA_OK) return st;
        p.partials_bytes = p.memory_bytes = p.flags_bytes = 0;
        p.total = diag_gamma_bytes(p) + diag_partials_bytes(p) + r.total;
    }
    *pl = p;
    return GMA_OK;
}

// Workspace regions of a plan whose op, sizes and split are set.
void layout(Plan* pl) {
    Plan& p = *pl;
    const gma_op_t op = p.op;
    const gma_dtype_t io = p.io;
    const size_t mem_elems = size_t(p.Kp) * size_t(p.dv + 1);
    p.partials_bytes = (op == GMA_OP_BIDIR || op == GMA_OP_CAUSAL) ? round_up(size_t(p.P * p.G) * mem_elems * 4, 256) : 0;
    p.memory_bytes = (op == GMA_OP_BIDIR) ? round_up(size_t(p.P) * mem_elems * 4, 256) : 0;
    p.off_params = 0;
    p.off_partials = p.off_params + p.params_bytes;
    // hand-off words of the fused bf16 kernels: [P][2][G] (bidirectional), [P][G] (causal)
    p.flags_bytes = 0;
    if (io == GMA_BF16 && op == GMA_OP_BIDIR) p.flags_bytes = round_up(size_t(p.P * 2 * p.G) * 8, 256);
    if (io == GMA_BF16 && op == GMA_OP_CAUSAL) p.flags_bytes = round_up(size_t(p.P * p.G) * 8, 256);
    p.off_memory = p.off_partials + p.partials_bytes;
    p.off_flags = p.off_memory + p.memory_bytes;
    // the 256-component causal scan reads back the keys' responsibilities of its key pass
    p.gk_bytes = (io == GMA_BF16 && op == GMA_OP_CAUSAL && bf16_causal_wide_applies(p))
                     ? round_up(size_t(p.P) * size_t(p.N) * size_t(p.Kp) * 2, 256)
                     : 0;
    p.off_gk = p.off_flags + p.flags_bytes;
    p.total = p.off_gk + p.gk_bytes;
}

gma_status_t make_cross_plan(const gma_cross_shape_t& s, gma_dtype_t io, Plan* pl) {
    const gma_shape_t sk{s.B, s.H, s.N_k, s.d_r, s.d_v, s.K};
    Plan p;
    gma_status_t st = make_plan(GMA_OP_BIDIR, sk, io, 0, &p);
    if (st != GMA_OK) return st;
    const int64_t lim = int64_t(1) << 40;
    if (s.N_q < 0) return GMA_ERR_BAD_SHAPE;
    if (s.N_q > lim || (p.P > 0 && s.N_q > lim / p.P)) return GMA_ERR_BAD_SHAPE;
    // one split count for both sides, from the longer one; a split may be empty on one side
    p.Nq = s.N_q;
    p.cross = true;
    p.G = 1;
    if (p.P > 0) {
        const int64_t n = std::max(p.N, p.Nq);
        p.G = std::max<int64_t>(1, std::min(bidir_split_target(p) / p.P, cdiv(std::max<int64_t>(n, 1), 512)));
    }
    p.seg = round_up(size_t(cdiv(std::max<int64_t>(p.N, 1), p.G)), kTokenTile);
    p.seg_q = round_up(size_t(cdiv(std::max<int64_t>(p.Nq, 1), p.G)), kTokenTile);
    // no split that is empty on both sides (with N_q = N_k this is the bidirectional plan)
    p.G = std::max<int64_t>(1, std::max(cdiv(p.N, p.seg), cdiv(p.Nq, p.seg_q)));
    layout(&p);
    *pl = p;
    return GMA_OK;
}

// Backward of cross-attention: the cross plan in fp32 (split partials and memory over the
// context), then the bidirectional backward's scratch, then the bf16 staging if any.
gma_status_t make_backward_cross_plan(const gma_cross_shape_t& s, gma_dtype_t io, Plan* pl) {
    if (io != GMA_F32 && io != GMA_BF16) return GMA_ERR_BAD_VALUE;
    gma_status_t st = make_cross_plan(s, GMA_F32, pl);
    if (st != GMA_OK) return st;
    backward_split(pl, kBackwardBidirBlocks);
    pl->op = GMA_OP_BACKWARD_BIDIR;
    pl->total += f32_backward_extra_bytes(*pl);
    pl->off_stage = pl->total;
    if (io == GMA_BF16) {
        pl->io = io;
        pl->total += backward_stage_bytes(*pl);
    }
    return GMA_OK;
}

// ---- launch tokens ----------------------------------------------------------------

uint64_t launch_token() {
    // splitmix64 over a per-process random seed plus a launch counter
    static std::atomic<uint64_t> counter{0};
    static const uint64_t seed = [] {
        std::random_device rd;
        return (uint64_t(rd()) << 32) ^ uint64_t(rd()) ^
               uint64_t(std::chrono::high_resolution_clock::now().time_since_epoch().count());
    }();
    uint64_t z = seed + 0x9e3779b97f4a7c15ull * (counter.fetch_add(1, std::memory_order_relaxed) + 1);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

namespace {
std::atomic<uint32_t> g_wait_limit{GMA_WAIT_LIMIT_DEFAULT};
std::atomic<int> g_single_launch{1};
}  // namespace

uint32_t wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }
bool single_launch_enabled() { return g_single_launch.load(std::memory_order_relaxed) != 0; }

// ---- per-device error word ----------------------------------------------------------
// Kernels OR kDevErrTimeout into d_error_word when a hand-off wait runs out;
// gma_device_status moves it into d_error_taken (an atomic exchange on the device, so no
// bit raised meanwhile is lost) and copies that to the host.  Each device has its own
// copy of both words; their addresses are resolved once per device, with it current.
__device__ uint32_t d_error_word;
__device__ uint32_t d_error_taken;

// Scratch of gma_forward_bidir_noalloc (the workspace it does not take): one per device, held
// until the process ends.  In host code the name is only a handle for hipGetSymbolAddress;
// kernels receive the device address it resolves to.
constexpr size_t kStaticScratchBytes = size_t(GMA_STATIC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

__global__ void take_error_kernel(uint32_t* word, uint32_t* taken) {
    if (threadIdx.x == 0) *taken = atomicExch(word, 0u);
}

namespace {
constexpr int kMaxDevices = 64;
struct DeviceWords {
    std::once_flag once;
    hipError_t status = hipSuccess;
    uint32_t* word = nullptr;
    uint32_t* taken = nullptr;
    void* scratch = nullptr;  // this device's copy of `scratch`
};
DeviceWords g_words[kMaxDevices];

hipError_t device_words(DeviceWords** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    DeviceWords& w = g_words[dev];
    std::call_once(w.once, [&w] {
        w.status = hipGetSymbolAddress(reinterpret_cast<void**>(&w.word), HIP_SYMBOL(d_error_word));
        if (w.status == hipSuccess)
            w.status = hipGetSymbolAddress(reinterpret_cast<void**>(&w.taken), HIP_SYMBOL(d_error_taken));
        if (w.status == hipSuccess) w.status = hipGetSymbolAddress(&w.scratch, HIP_SYMBOL(scratch));
    });
    *out = &w;
    return w.status;
}

std::mutex g_resident_mu;
std::map<std::pair<int, const void*>, int64_t> g_resident;
}  // namespace

hipError_t device_error_word(uint32_t** word) {
    DeviceWords* w = nullptr;
    hipError_t e = device_words(&w);
    *word = e == hipSuccess ? w->word : nullptr;
    return e;
}

hipError_t resident_workgroups(const void* kernel, int threads, int64_t* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    {
        std::lock_guard<std::mutex> lk(g_resident_mu);
        auto it = g_resident.find({dev, kernel});
        if (it != g_resident.end()) {
            *out = it->second;
            return hipSuccess;
        }
    }
    int per_cu = 0, cus = 0;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int64_t n = int64_t(std::max(per_cu, 0)) * int64_t(std::max(cus, 0));
    std::lock_guard<std::mutex> lk(g_resident_mu);
    g_resident[{dev, kernel}] = n;
    *out = n;
    return hipSuccess;
}

// ---- kernel timing ----------------------------------------------------------------

namespace {

struct PendingLaunch {
    const char* name;
    hipEvent_t start, stop;
};

std::mutex g_trace_mu;
bool g_trace_on = false;
std::vector<PendingLaunch> g_pending;
PendingLaunch g_open{nullptr, nullptr, nullptr};

void drop_pending() {
    for (auto& p : g_pending) {
        (void)hipEventDestroy(p.start);
        (void)hipEventDestroy(p.stop);
    }
    g_pending.clear();
}

}  // namespace

void trace_begin(hipStream_t st, const char* name) {
    std::lock_guard<std::mutex> lk(g_trace_mu);
    if (!g_trace_on) return;
    PendingLaunch p{name, nullptr, nullptr};
    if (hipEventCreate(&p.start) != hipSuccess) return;
    if (hipEventCreate(&p.stop) != hipSuccess) {
        (void)hipEventDestroy(p.start);
        return;
    }
    (void)hipEventRecord(p.start, st);
    g_open = p;
}

void trace_end(hipStream_t st) {
    std::lock_guard<std::mutex> lk(g_trace_mu);
    if (!g_trace_on || !g_open.name) return;
    (void)hipEventRecord(g_open.stop, st);
    g_pending.push_back(g_open);
    g_open = PendingLaunch{nullptr, nullptr, nullptr};
}

}  // namespace gma

using gma::Plan;

extern "C" {

const char* gma_status_string(gma_status_t s) {
    switch (s) {
        case GMA_OK: return "GMA_OK";
        case GMA_ERR_NULL_POINTER: return "GMA_ERR_NULL_POINTER";
        case GMA_ERR_BAD_SHAPE: return "GMA_ERR_BAD_SHAPE";
        case GMA_ERR_BAD_VALUE: return "GMA_ERR_BAD_VALUE";
        case GMA_ERR_UNSUPPORTED: return "GMA_ERR_UNSUPPORTED";
        case GMA_ERR_MISALIGNED: return "GMA_ERR_MISALIGNED";
        case GMA_ERR_WORKSPACE_TOO_SMALL: return "GMA_ERR_WORKSPACE_TOO_SMALL";
        case GMA_ERR_HIP: return "GMA_ERR_HIP";
        case GMA_ERR_TIMEOUT: return "GMA_ERR_TIMEOUT";
    }
    return "GMA_ERR_UNKNOWN";
}

gma_status_t gma_workspace_size(gma_op_t op, const gma_shape_t* shape, gma_dtype_t io_dtype,
                                int32_t chunk, size_t* bytes_out) {
    if (!shape || !bytes_out) return GMA_ERR_NULL_POINTER;
    Plan p;
    gma_status_t st = gma::make_plan(op, *shape, io_dtype, chunk, &p);
    if (st != GMA_OK) return st;
    *bytes_out = p.total;
    return GMA_OK;
}

static gma_status_t check_ws(const Plan& p, const void* ws, size_t ws_bytes) {
    if (p.total > 0 && !ws) return GMA_ERR_NULL_POINTER;
    if (ws_bytes < p.total) return GMA_ERR_WORKSPACE_TOO_SMALL;
    if (ws && !gma::aligned16(ws)) return GMA_ERR_MISALIGNED;
    return GMA_OK;
}

static gma_status_t launch_status(hipError_t e) { return e == hipSuccess ? GMA_OK : GMA_ERR_HIP; }

gma_status_t gma_responsibilities(const void* X, gma_dtype_t x_dtype, const float* mu,
                                  const float* sigma2, const float* pi, void* Gamma,
                                  gma_dtype_t gamma_dtype, const gma_shape_t* shape,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!X || !mu || !sigma2 || !pi || !Gamma || !shape) return GMA_ERR_NULL_POINTER;
    if (gamma_dtype != GMA_F32 && gamma_dtype != GMA_BF16) return GMA_ERR_BAD_VALUE;
    Plan p;
    gma_status_t st = gma::make_plan(GMA_OP_RESPONSIBILITIES, *shape, x_dtype, 0, &p);
    if (st != GMA_OK) return st;
    for (const void* q : {X, (const void*)mu, (const void*)sigma2, (const void*)pi, (const void*)Gamma})
        if (!gma::aligned16(q)) return GMA_ERR_MISALIGNED;
    if ((st = check_ws(p, workspace, workspace_bytes)) != GMA_OK) return st;
    if (p.P == 0 || p.N == 0) return GMA_OK;
    char* ws = static_cast<char*>(workspace);
    if (x_dtype == GMA_F32)
        return launch_status(gma::f32_responsibilities(p, static_cast<const float*>(X), mu, sigma2, pi,
                                                       Gamma, gamma_dtype, ws, stream));
    return launch_status(gma::bf16_responsibilities(p, X, mu, sigma2, pi, Gamma, gamma_dtype, ws, stream));
}

static gma_status_t forward_common(gma_op_t op, const void* XQ, const void* XK, const void* V,
                                   gma_dtype_t io, const float* mu, const float* sigma2,
                                   const float* pi, float eps, void* O, const gma_shape_t* shape,
                                   int32_t chunk, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream, const float* state_in = nullptr,
                                   float* state_out = nullptr) {
    if (!mu || !sigma2 || !pi || !shape) return GMA_ERR_NULL_POINTER;
    Plan p;
    gma_status_t st = gma::make_plan(op, *shape, io, chunk, &p);
    if (st != GMA_OK) return st;
    if ((!XQ || !XK || !V || !O) && p.P > 0 && p.N > 0) return GMA_ERR_NULL_POINTER;  // tensors with elements
    if (!(eps > 0.0f) || !std::isfinite(eps)) return GMA_ERR_BAD_VALUE;
    for (const void* q : {XQ, XK, V, (const void*)mu, (const void*)sigma2, (const void*)pi, (const void*)O})
        if (!gma::aligned16(q)) return GMA_ERR_MISALIGNED;
    if ((st = check_ws(p, workspace, workspace_bytes)) != GMA_OK) return st;
    if (state_out) {  // carried memory (causal only): aligned and not overlapping its input
        const size_t sb = size_t(p.P) * size_t(p.K) * size_t(p.dv + 1) * 4;
        if (!gma::aligned16(state_out) || (state_in && !gma::aligned16(state_in))) return GMA_ERR_MISALIGNED;
        const char *a = reinterpret_cast<const char*>(state_in), *b = reinterpret_cast<const char*>(state_out);
        if (state_in && sb > 0 && a < b + sb && b < a + sb) return GMA_ERR_BAD_VALUE;
    } else if (state_in && !gma::aligned16(state_in)) {
        return GMA_ERR_MISALIGNED;
    }
    if (p.P == 0) return GMA_OK;
    if (p.N == 0) return state_out ? launch_status(gma::copy_state(p, state_in, state_out, stream)) : GMA_OK;
    if (gma::decode_applies(p))
        return launch_status(gma::causal_decode(p, XQ, XK, V, mu, sigma2, pi, eps, O, stream, state_in, state_out));
    char* ws = static_cast<char*>(workspace);
    if (io == GMA_F32) {
        const float *q = static_cast<const float*>(XQ), *k = static_cast<const float*>(XK),
                    *v = static_cast<const float*>(V);
        float* o = static_cast<float*>(O);
        if (op == GMA_OP_BIDIR) return launch_status(gma::f32_bidir(p, q, k, v, mu, sigma2, pi, eps, o, ws, stream));
        return launch_status(gma::f32_causal(p, q, k, v, mu, sigma2, pi, eps, o, ws, stream, state_in, state_out));
    }
    if (op == GMA_OP_BIDIR) return launch_status(gma::bf16_bidir(p, XQ, XK, V, mu, sigma2, pi, eps, O, ws, stream));
    return launch_status(gma::bf16_causal(p, XQ, XK, V, mu, sigma2, pi, eps, O, ws, stream, state_in, state_out));
}

gma_status_t gma_forward_bidir(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                               const float* mu, const float* sigma2, const float* pi, float eps,
                               void* O, const gma_shape_t* shape, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    return forward_common(GMA_OP_BIDIR, XQ, XK, V, io_dtype, mu, sigma2, pi, eps, O, shape, 0,
                          workspace, workspace_bytes, stream);
}

gma_status_t gma_forward_bidir_noalloc(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                       const float* mu, const float* sigma2, const float* pi, float eps, void* O,
                                       const gma_shape_t* shape, hipStream_t stream) {
    if (!shape) return GMA_ERR_NULL_POINTER;
    size_t need = 0;
    gma_status_t st = gma_workspace_size(GMA_OP_BIDIR, shape, io_dtype, 0, &need);
    if (st != GMA_OK) return st;
    if (need > gma::kStaticScratchBytes) return GMA_ERR_WORKSPACE_TOO_SMALL;  // before any HIP call
    if (!mu || !sigma2 || !pi) return GMA_ERR_NULL_POINTER;
    gma::DeviceWords* w = nullptr;
    if (gma::device_words(&w) != hipSuccess) return GMA_ERR_HIP;
    return forward_common(GMA_OP_BIDIR, XQ, XK, V, io_dtype, mu, sigma2, pi, eps, O, shape, 0, w->scratch,
                          gma::kStaticScratchBytes, stream);
}

gma_status_t gma_forward_causal(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                const float* mu, const float* sigma2, const float* pi, float eps,
                                void* O, const gma_shape_t* shape, int32_t chunk, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    return forward_common(GMA_OP_CAUSAL, XQ, XK, V, io_dtype, mu, sigma2, pi, eps, O, shape, chunk,
                          workspace, workspace_bytes, stream);
}

gma_status_t gma_forward_causal_state(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                      const float* mu, const float* sigma2, const float* pi, float eps,
                                      void* O, const gma_shape_t* shape, int32_t chunk,
                                      const float* state_in, float* state_out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    return forward_common(GMA_OP_CAUSAL, XQ, XK, V, io_dtype, mu, sigma2, pi, eps, O, shape, chunk,
                          workspace, workspace_bytes, stream, state_in, state_out);
}

gma_status_t gma_responsibility_diagnostics(const void* X, gma_dtype_t x_dtype, const float* mu, const float* sigma2,
                                            const float* pi, const gma_shape_t* shape, float* usage, float* stats,
                                            int32_t* argmax, float* gbar, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
    if (!mu || !sigma2 || !pi || !shape || !usage || !stats) return GMA_ERR_NULL_POINTER;
    Plan p, r;
    gma_status_t st = gma::make_plan(GMA_OP_DIAGNOSTICS, *shape, x_dtype, 0, &p);
    if (st != GMA_OK) return st;
    if ((st = gma::make_plan(GMA_OP_RESPONSIBILITIES, *shape, x_dtype, 0, &r)) != GMA_OK) return st;
    if (!X && p.P > 0 && p.N > 0) return GMA_ERR_NULL_POINTER;
    for (const void* q : {X, (const void*)mu, (const void*)sigma2, (const void*)pi, (const void*)usage, (const void*)stats,
                          (const void*)argmax, (const void*)gbar})
        if (!gma::aligned16(q)) return GMA_ERR_MISALIGNED;
    if ((st = check_ws(p, workspace, workspace_bytes)) != GMA_OK) return st;
    return launch_status(gma::diagnostics(p, r, X, mu, sigma2, pi, usage, stats, argmax, gbar,
                                          static_cast<char*>(workspace), stream));
}

// Validation, bf16 staging and dispatch of the three backward entry points; `p` is their plan
// (query-side arrays have p.Nq rows, key-side arrays p.N).
static gma_status_t backward_run(const Plan& p, const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                 const float* mu, const float* sigma2, const float* pi, float eps, const void* dO,
                                 void* dXQ, void* dXK, void* dV, float* dmu, float* dsigma2, float* dpi,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream,
                                 const float* state_in = nullptr, const float* dstate_out = nullptr,
                                 float* dstate_in = nullptr) {
    if ((!dmu || !dsigma2 || !dpi) && p.H > 0) return GMA_ERR_NULL_POINTER;
    for (const void* q : {(const void*)state_in, (const void*)dstate_out, (const void*)dstate_in})
        if (!gma::aligned16(q)) return GMA_ERR_MISALIGNED;
    if (dstate_in) {  // written while the others are read: no overlap
        const size_t sb = size_t(p.P) * size_t(p.K) * size_t(p.dv + 1) * 4;
        const char* b = reinterpret_cast<const char*>(dstate_in);
        for (const float* other : {state_in, dstate_out}) {
            const char* a = reinterpret_cast<const char*>(other);
            if (other && sb > 0 && a < b + sb && b < a + sb) return GMA_ERR_BAD_VALUE;
        }
    }
    if ((!XQ || !dO || !dXQ) && p.P > 0 && p.Nq > 0) return GMA_ERR_NULL_POINTER;  // tensors with elements
    if ((!XK || !V || !dXK || !dV) && p.P > 0 && p.N > 0) return GMA_ERR_NULL_POINTER;
    if (!(eps > 0.0f) || !std::isfinite(eps)) return GMA_ERR_BAD_VALUE;
    for (const void* q : {XQ, XK, V, (const void*)mu, (const void*)sigma2, (const void*)pi, dO, (const void*)dXQ,
                          (const void*)dXK, (const void*)dV, (const void*)dmu, (const void*)dsigma2, (const void*)dpi})
        if (!gma::aligned16(q)) return GMA_ERR_MISALIGNED;
    gma_status_t st = check_ws(p, workspace, workspace_bytes);
    if (st != GMA_OK) return st;
    const float *q = static_cast<const float*>(XQ), *k = static_cast<const float*>(XK),
                *v = static_cast<const float*>(V), *d = static_cast<const float*>(dO);
    float *dq = static_cast<float*>(dXQ), *dk = static_cast<float*>(dXK), *dvv = static_cast<float*>(dV);
    char* ws = static_cast<char*>(workspace);
    const bool staged = io_dtype == GMA_BF16 && p.P > 0 && (p.N > 0 || p.Nq > 0);
    const size_t nrq = size_t(p.P * p.Nq * p.dr), nrk = size_t(p.P * p.N * p.dr);
    const size_t nvq = size_t(p.P * p.Nq * p.dv), nvk = size_t(p.P * p.N * p.dv);
    hipError_t e = hipSuccess;
    if (staged) {  // fp32 copies of the inputs; the passes write fp32 outputs next to them
        const gma::StageLayout l = gma::stage_layout(p);
        char* sg = ws + p.off_stage;
        float *q32 = reinterpret_cast<float*>(sg + l.off[0]), *k32 = reinterpret_cast<float*>(sg + l.off[1]),
              *v32 = reinterpret_cast<float*>(sg + l.off[2]), *d32 = reinterpret_cast<float*>(sg + l.off[3]);
        dq = reinterpret_cast<float*>(sg + l.off[4]);
        dk = reinterpret_cast<float*>(sg + l.off[5]);
        dvv = reinterpret_cast<float*>(sg + l.off[6]);
        if ((e = gma::widen_bf16(XQ, q32, nrq, stream)) != hipSuccess || (e = gma::widen_bf16(XK, k32, nrk, stream)) != hipSuccess ||
            (e = gma::widen_bf16(V, v32, nvk, stream)) != hipSuccess || (e = gma::widen_bf16(dO, d32, nvq, stream)) != hipSuccess)
            return launch_status(e);
        q = q32, k = k32, v = v32, d = d32;
    }
    if (p.op == GMA_OP_BACKWARD_CAUSAL)
        e = gma::f32_backward_causal(p, q, k, v, mu, sigma2, pi, eps, d, dq, dk, dvv, dmu, dsigma2, dpi, ws, stream,
                                     state_in, dstate_out, dstate_in);
    else
        e = gma::f32_backward_bidir(p, q, k, v, mu, sigma2, pi, eps, d, dq, dk, dvv, dmu, dsigma2, dpi, ws, stream);
    if (e != hipSuccess || !staged) return launch_status(e);
    if ((e = gma::narrow_to_bf16(dq, dXQ, nrq, stream)) != hipSuccess || (e = gma::narrow_to_bf16(dk, dXK, nrk, stream)) != hipSuccess)
        return launch_status(e);
    return launch_status(gma::narrow_to_bf16(dvv, dV, nvk, stream));
}

static gma_status_t backward_common(gma_op_t op, const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                    const float* mu, const float* sigma2, const float* pi, float eps, const void* dO,
                                    void* dXQ, void* dXK, void* dV, float* dmu, float* dsigma2, float* dpi,
                                    const gma_shape_t* shape, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    if (!mu || !sigma2 || !pi || !shape) return GMA_ERR_NULL_POINTER;
    Plan p;
    gma_status_t st = gma::make_plan(op, *shape, io_dtype, 0, &p);
    if (st != GMA_OK) return st;
    return backward_run(p, XQ, XK, V, io_dtype, mu, sigma2, pi, eps, dO, dXQ, dXK, dV, dmu, dsigma2, dpi, workspace,
                        workspace_bytes, stream);
}

gma_status_t gma_backward_bidir(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                const float* mu, const float* sigma2, const float* pi, float eps, const void* dO,
                                void* dXQ, void* dXK, void* dV, float* dmu, float* dsigma2, float* dpi,
                                const gma_shape_t* shape, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return backward_common(GMA_OP_BACKWARD_BIDIR, XQ, XK, V, io_dtype, mu, sigma2, pi, eps, dO, dXQ, dXK, dV, dmu,
                           dsigma2, dpi, shape, workspace, workspace_bytes, stream);
}

gma_status_t gma_backward_causal(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                 const float* mu, const float* sigma2, const float* pi, float eps, const void* dO,
                                 void* dXQ, void* dXK, void* dV, float* dmu, float* dsigma2, float* dpi,
                                 const gma_shape_t* shape, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return backward_common(GMA_OP_BACKWARD_CAUSAL, XQ, XK, V, io_dtype, mu, sigma2, pi, eps, dO, dXQ, dXK, dV, dmu,
                           dsigma2, dpi, shape, workspace, workspace_bytes, stream);
}

gma_status_t gma_backward_causal_state(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                                       const float* mu, const float* sigma2, const float* pi, float eps,
                                       const void* dO, const float* state_in, const float* dstate_out, void* dXQ,
                                       void* dXK, void* dV, float* dmu, float* dsigma2, float* dpi, float* dstate_in,
                                       const gma_shape_t* shape, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    if (!mu || !sigma2 || !pi || !shape) return GMA_ERR_NULL_POINTER;
    Plan p;
    gma_status_t st = gma::make_plan(GMA_OP_BACKWARD_CAUSAL, *shape, io_dtype, 0, &p);
    if (st != GMA_OK) return st;
    return backward_run(p, XQ, XK, V, io_dtype, mu, sigma2, pi, eps, dO, dXQ, dXK, dV, dmu, dsigma2, dpi, workspace,
                        workspace_bytes, stream, state_in, dstate_out, dstate_in);
}

gma_status_t gma_backward_cross_workspace_size(const gma_cross_shape_t* shape, gma_dtype_t io_dtype, size_t* bytes_out) {
    if (!shape || !bytes_out) return GMA_ERR_NULL_POINTER;
    Plan p;
    gma_status_t st = gma::make_backward_cross_plan(*shape, io_dtype, &p);
    if (st != GMA_OK) return st;
    *bytes_out = p.total;
    return GMA_OK;
}

gma_status_t gma_backward_cross(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype, const float* mu,
                                const float* sigma2, const float* pi, float eps, const void* dO, void* dXQ, void* dXK,
                                void* dV, float* dmu, float* dsigma2, float* dpi, const gma_cross_shape_t* shape,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!mu || !sigma2 || !pi || !shape) return GMA_ERR_NULL_POINTER;
    Plan p;
    gma_status_t st = gma::make_backward_cross_plan(*shape, io_dtype, &p);
    if (st != GMA_OK) return st;
    return backward_run(p, XQ, XK, V, io_dtype, mu, sigma2, pi, eps, dO, dXQ, dXK, dV, dmu, dsigma2, dpi, workspace,
                        workspace_bytes, stream);
}

gma_status_t gma_cross_workspace_size(const gma_cross_shape_t* shape, gma_dtype_t io_dtype, size_t* bytes_out) {
    if (!shape || !bytes_out) return GMA_ERR_NULL_POINTER;
    Plan p;
    gma_status_t st = gma::make_cross_plan(*shape, io_dtype, &p);
    if (st != GMA_OK) return st;
    *bytes_out = p.total;
    return GMA_OK;
}

gma_status_t gma_forward_cross(const void* XQ, const void* XK, const void* V, gma_dtype_t io_dtype,
                               const float* mu, const float* sigma2, const float* pi, float eps, void* O,
                               const gma_cross_shape_t* shape, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    if (!mu || !sigma2 || !pi || !shape) return GMA_ERR_NULL_POINTER;
    Plan p;
    gma_status_t st = gma::make_cross_plan(*shape, io_dtype, &p);
    if (st != GMA_OK) return st;
    // a side without rows may come without storage
    if ((!XQ || !O) && p.P > 0 && p.Nq > 0) return GMA_ERR_NULL_POINTER;
    if ((!XK || !V) && p.P > 0 && p.N > 0) return GMA_ERR_NULL_POINTER;
    if (!(eps > 0.0f) || !std::isfinite(eps)) return GMA_ERR_BAD_VALUE;
    for (const void* q : {XQ, XK, V, (const void*)mu, (const void*)sigma2, (const void*)pi, (const void*)O})
        if (!gma::aligned16(q)) return GMA_ERR_MISALIGNED;
    if ((st = check_ws(p, workspace, workspace_bytes)) != GMA_OK) return st;
    if (p.P == 0 || p.Nq == 0) return GMA_OK;  // no output rows (an empty context still yields zeros)
    char* ws = static_cast<char*>(workspace);
    if (io_dtype == GMA_F32)
        return launch_status(gma::f32_bidir(p, static_cast<const float*>(XQ), static_cast<const float*>(XK),
                                            static_cast<const float*>(V), mu, sigma2, pi, eps, static_cast<float*>(O),
                                            ws, stream));
    return launch_status(gma::bf16_bidir(p, XQ, XK, V, mu, sigma2, pi, eps, O, ws, stream));
}

gma_status_t gma_set_single_launch(int enable) {
    gma::g_single_launch.store(enable != 0 ? 1 : 0, std::memory_order_relaxed);
    return GMA_OK;
}

gma_status_t gma_device_status(hipStream_t stream) {
    gma::DeviceWords* w = nullptr;
    if (gma::device_words(&w) != hipSuccess) return GMA_ERR_HIP;
    hipLaunchKernelGGL(gma::take_error_kernel, dim3(1), dim3(64), 0, stream, w->word, w->taken);
    if (hipGetLastError() != hipSuccess) return GMA_ERR_HIP;
    uint32_t bits = 0;
    if (hipMemcpyAsync(&bits, w->taken, sizeof(bits), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return GMA_ERR_HIP;
    return (bits & gma::kDevErrTimeout) ? GMA_ERR_TIMEOUT : GMA_OK;
}

gma_status_t gma_plan_info(gma_op_t op, const gma_shape_t* shape, gma_dtype_t io_dtype, int32_t chunk,
                           gma_plan_info_t* info) {
    if (!shape || !info) return GMA_ERR_NULL_POINTER;
    const bool backward = op == GMA_OP_BACKWARD_BIDIR || op == GMA_OP_BACKWARD_CAUSAL;
    if (op != GMA_OP_BIDIR && op != GMA_OP_CAUSAL && !backward) return GMA_ERR_BAD_VALUE;
    Plan p;
    gma_status_t st = gma::make_plan(op, *shape, io_dtype, backward ? 0 : chunk, &p);
    if (st != GMA_OK) return st;
    *info = gma_plan_info_t{};
    info->splits = p.G;
    info->rows_per_split = int64_t(p.seg);
    info->workgroups = p.P * p.G;
    if (op == GMA_OP_CAUSAL) info->chunk_used = io_dtype == GMA_BF16 ? gma::bf16_causal_chunk(p) : gma::f32_causal_chunk(p);
    if (op == GMA_OP_BIDIR && io_dtype == GMA_BF16) {
        int threads = 0;
        int64_t lds = 0;
        gma::bf16_bidir_geometry(p.dr, p.Kp / 32, p.dv / 32, &threads, &lds);
        info->threads_per_workgroup = threads;
        info->lds_bytes = lds;
        info->waits_on_all_splits = p.G > 1 && p.G <= gma::kBidirSingleMaxSplits ? 1 : 0;
        info->resident_bound = gma::kDeviceCUs * gma::bf16_bidir_per_cu(p.dr, p.Kp / 32, p.dv / 32);
    }
    return GMA_OK;
}

gma_status_t gma_set_wait_limit(uint32_t polls) {
    gma::g_wait_limit.store(polls, std::memory_order_relaxed);
    return GMA_OK;
}

gma_status_t gma_profiling(int enable) {
    std::lock_guard<std::mutex> lk(gma::g_trace_mu);
    gma::g_trace_on = enable != 0;
    if (!gma::g_trace_on) gma::drop_pending();
    return GMA_OK;
}

gma_status_t gma_profiling_collect(gma_kernel_stat_t* stats, int capacity, int* count) {
    if (!count || (capacity > 0 && !stats)) return GMA_ERR_NULL_POINTER;
    std::lock_guard<std::mutex> lk(gma::g_trace_mu);
    std::map<std::string, std::pair<int64_t, double>> agg;
    std::vector<std::string> order;
    gma_status_t status = GMA_OK;
    for (auto& p : gma::g_pending) {
        float ms = 0.0f;
        if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
            status = GMA_ERR_HIP;
            continue;
        }
        auto it = agg.find(p.name);
        if (it == agg.end()) {
            order.push_back(p.name);
            agg[p.name] = {1, double(ms)};
        } else {
            it->second.first += 1;
            it->second.second += ms;
        }
    }
    // names are the launchers' string literals; map them back to those static pointers
    std::map<std::string, const char*> names;
    for (auto& p : gma::g_pending) names[p.name] = p.name;
    gma::drop_pending();
    int n = 0;
    for (const auto& name : order) {
        if (n < capacity) {
            stats[n].name = names[name];
            stats[n].launches = agg[name].first;
            stats[n].total_ms = agg[name].second;
        }
        ++n;
    }
    *count = n;
    return status;
}

}  // extern "C"
