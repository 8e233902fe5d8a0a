"""GPU parity of the backward passes of the bidirectional and causal forwards (Sec. 4.1, Eq.
17-20; Sec. 3.5 Eq. 6b, 8b) through the C ABI, against the fp64 oracle's backward on the same
seeded inputs and upstream gradient.

Error measure: per entry, |g - g*| / |g|_mag, where |g|_mag is the oracle's magnitude evaluation
of the same formulas (oracle.backward.backward_magnitudes: every input and intermediate replaced
by its absolute value, every difference by a sum), i.e. the size of the terms that form the
entry.  Every entry of every gradient is checked against its own scale: an entry that is small
because its terms cancel is allowed the error of those terms' rounding, and no more; an entry
that is simply wrong or zero fails.  Bound: the kernels evaluate the scores in fp32 (direct form,
absolute error ~u times the Mahalanobis sum, a few 1e-5 for the components that carry weight) and
everything after the softmax in fp32 sums over K, d_v and the positions of a split, each within a
few hundred roundings of its terms; 1e-4 of the magnitude leaves a margin of several times what
the shapes here (N up to 5000, K up to 256) accumulate.  bf16 outputs are then rounded to
nearest-even, 2^-9 of the entry at most, hence 5e-3 for them."""
import numpy as np
import pytest
import torch

import oracle.backward
from gaussian_mixture_sequence_amd import binding as gb
from gaussian_mixture_sequence_amd.inputs import WORKLOADS, Workload, head_slice, make_inputs
from gma_testutil import to_device, to_np

pytestmark = pytest.mark.gpu

TOL_BWD = 1e-4
KEYS = ("dXQ", "dXK", "dV", "dmu", "dsigma2", "dpi")


def upstream(w: Workload, seed: int) -> torch.Tensor:
    """dO [B,H,N,d_v]: standard normal, seeded (the loss gradient is an input of the pass)."""
    gen = torch.Generator().manual_seed(seed)
    return torch.randn(w.B, w.H, w.N, w.d_v, generator=gen, dtype=torch.float32)


# Below fp32's normal range the kernels' arithmetic has no relative precision: a responsibility
# under 2^-126 (about 1.2e-38; components a token is far from) is flushed to zero, and every term
# it forms (times factors g, (x - mu) / sigma2, ... of at most ~1e6, summed over ~1e3 positions)
# stays below 1e-28 in absolute value.  Magnitudes are floored there.
MAG_FLOOR = 1e-28


def entry_error(out, ref, mag) -> float:
    """max over entries of |out - ref| / max(mag, MAG_FLOOR) (mag: the magnitude evaluation of the
    entry's terms)."""
    out, ref, mag = (np.asarray(t, np.float64) for t in (out, ref, mag))
    if ref.size == 0:
        return 0.0
    assert (mag >= np.abs(ref) * (1 - 1e-12)).all()
    return float((np.abs(out - ref) / np.maximum(mag, MAG_FLOOR)).max())


def magnitudes(w: Workload, inp, d_o, causal=None, **kw):
    return oracle.backward.backward_magnitudes(inp["xq"], inp["xk"], inp["v"], inp["mu"], inp["sigma2"], inp["pi"],
                                               w.eps, d_o, causal=w.causal if causal is None else causal, **kw)


def check_all(got, ref, mag, keys=KEYS, tol=None, where=""):
    """Every entry of every gradient within its tolerance; prints the worst per tensor."""
    worst = {}
    for k in keys:
        g = np.asarray(got[k], np.float64)
        assert g.shape == ref[k].shape, k
        assert np.isfinite(g).all(), k
        t = tol(k) if callable(tol) else (tol or TOL_BWD)
        worst[k] = entry_error(g, ref[k], mag[k])
        assert worst[k] <= t, (where, k, worst[k])
    print("\n[bwd-err] %s %s" % (where, " ".join("%s=%.2e" % kv for kv in worst.items())))
    return worst


def run_gpu(w: Workload, inp, d_o):
    d = to_device(inp)
    g = gb.gma_backward_bidir(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], d_o.cuda(), w.eps)
    torch.cuda.synchronize()
    return {k: to_np(v) for k, v in g.items()}


def run_oracle(w: Workload, inp, d_o):
    return oracle.backward.backward_bidir(inp["xq"], inp["xk"], inp["v"], inp["mu"], inp["sigma2"], inp["pi"],
                                          w.eps, d_o)


def case(N, seed, **kw):
    base = WORKLOADS["bidir_small_f32"]
    return base.with_(name="bwd", N=N, seed=seed, **dict(dict(B=1, H=2), **kw))


def cid(w):
    return "B%dH%d-N%d-dr%d-dv%d-K%d" % (w.B, w.H, w.N, w.d_r, w.d_v, w.K)


CASES = [
    WORKLOADS["bidir_small_f32"],
    case(1000, 91, B=2, H=3, d_r=7, d_v=5, K=13),       # ragged dims and tail
    case(2, 92),                                        # two positions, one tile
    case(5000, 93, d_r=32, d_v=64, K=64),              # several splits per problem
    case(300, 94, B=1, H=1, d_r=128, d_v=128, K=256),  # maximum dims (half-height tiles)
    case(700, 95, B=3, H=2, d_r=64, d_v=32, K=128, mu_std=1.5),
    case(500, 96, B=1, H=2, d_r=64, d_v=64, K=256),     # K-blocked passes: four full blocks
    # K-blocked passes: a ragged last block and tail, several splits, small dims
    case(1500, 97, B=2, H=2, d_r=32, d_v=48, K=200),
    case(6000, 98, B=1, H=3, d_r=16, d_v=16, K=100, mu_std=1.5),
    # K-blocked passes with K not a multiple of 4 (per-element responsibility loads; the memory
    # rows of every problem after the first start off a 16-byte boundary), ragged tail
    case(900, 99, B=2, H=2, d_r=32, d_v=16, K=66),
]


@pytest.mark.parametrize("w", CASES, ids=cid)
def test_backward_parity(w):
    inp = make_inputs(w)
    d_o = upstream(w, w.seed + 1000)
    got, ref = run_gpu(w, inp, d_o), run_oracle(w, inp, d_o)
    check_all(got, ref, magnitudes(w, inp, d_o), where=cid(w))


def test_backward_single_position():
    """N = 1: the one key is the whole memory, so O = v r / (r + eps) with r = gamma_Q . gamma_K;
    the routing enters only through the eps term, so the routing and parameter gradients are
    O(eps / r) of their terms, obtained by cancellation.  Against the magnitude of those terms
    every gradient is still checked entry by entry."""
    w = case(1, 92)
    inp = make_inputs(w)
    d_o = upstream(w, 1092)
    got, ref = run_gpu(w, inp, d_o), run_oracle(w, inp, d_o)
    check_all(got, ref, magnitudes(w, inp, d_o), where="N1")


def test_backward_deterministic():
    """Fixed reduction orders: two calls give bit-identical gradients."""
    w = case(3000, 96, B=2, H=2)
    inp = make_inputs(w)
    d_o = upstream(w, 1096)
    a, b = run_gpu(w, inp, d_o), run_gpu(w, inp, d_o)
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k


def test_backward_no_rows_gives_zero_parameter_gradients():
    """N = 0: no term reaches the mixture parameters; their gradients are overwritten with 0."""
    w = case(0, 97)
    inp = make_inputs(w)
    d = to_device(inp)
    g = gb.gma_backward_bidir(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"],
                              torch.empty(w.B, w.H, 0, w.d_v, device="cuda"), w.eps)
    torch.cuda.synchronize()
    for k in ("dmu", "dsigma2", "dpi"):
        assert not to_np(g[k]).any(), k
    assert g["dXQ"].numel() == 0 and g["dV"].numel() == 0


# bf16 I/O: the inputs are bf16 values (exact in the fp64 oracle) and the per-position gradients
# come back rounded to bf16, at most 2^-9 of each entry; the parameter gradients stay fp32.
TOL_BWD_BF16 = 5e-3


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dims", [(1000, 7, 5, 13), (3000, 64, 64, 64), (500, 128, 128, 256), (1500, 64, 64, 32)],
                         ids=lambda d: "N%d-dr%d-dv%d-K%d" % d)
def test_backward_bf16_parity(causal, dims):
    N, dr, dv, K = dims
    w = case(N, 111 + N % 97, B=2, H=2, d_r=dr, d_v=dv, K=K, dtype="bf16", causal=causal)
    inp = make_inputs(w)
    d_o = upstream(w, w.seed + 1000).bfloat16()
    d = to_device(inp)
    fn = gb.gma_backward_causal if causal else gb.gma_backward_bidir
    g = fn(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], d_o.cuda(), w.eps)
    torch.cuda.synchronize()
    ref = (run_oracle_causal if causal else run_oracle)(w, inp, d_o)
    for k in KEYS:
        assert g[k].dtype == (torch.bfloat16 if k in ("dXQ", "dXK", "dV") else torch.float32), k
    check_all({k: to_np(v) for k, v in g.items()}, ref, magnitudes(w, inp, d_o),
              tol=lambda k: TOL_BWD_BF16 if k in ("dXQ", "dXK", "dV") else TOL_BWD,
              where="bf16-%s-%s" % ("causal" if causal else "bidir", cid(w)))


def head_column(inp, d_o, h):
    """The inputs of every batch entry of head h, as a B x 1 problem."""
    return ({"xq": inp["xq"][:, h:h + 1].contiguous(), "xk": inp["xk"][:, h:h + 1].contiguous(),
             "v": inp["v"][:, h:h + 1].contiguous(), "mu": inp["mu"][h:h + 1].contiguous(),
             "sigma2": inp["sigma2"][h:h + 1].contiguous(), "pi": inp["pi"][h:h + 1].contiguous()},
            d_o[:, h:h + 1].contiguous())


def full_size_check(w, got, inp, d_o, heads, causal):
    """Every gradient of the sampled heads, entry by entry: the oracle on all B sequences of a head
    gives that head's per-position gradients and its parameter gradients (which sum over every
    sequence and position of the head)."""
    fn = oracle.backward.backward_causal if causal else oracle.backward.backward_bidir
    for h in heads:
        sl, do_h = head_column(inp, d_o, h)
        ref = fn(sl["xq"], sl["xk"], sl["v"], sl["mu"], sl["sigma2"], sl["pi"], w.eps, do_h)
        mag = oracle.backward.backward_magnitudes(sl["xq"], sl["xk"], sl["v"], sl["mu"], sl["sigma2"], sl["pi"],
                                                  w.eps, do_h, causal=causal)
        g = {k: got[k][:, h:h + 1] for k in ("dXQ", "dXK", "dV")}
        g.update({k: got[k][h:h + 1] for k in ("dmu", "dsigma2", "dpi")})
        check_all(g, ref, mag, where="%s-full-h%d" % ("causal" if causal else "bidir", h))


def test_backward_full_size_sampled_heads():
    """The B=8, H=8, N=4096, d_r=d_v=K=64 dims in fp32 (the split plan of the bench's backward
    step): every gradient of two heads (all eight sequences each) against the oracle."""
    w = WORKLOADS["bidir_b8h8_n4096"].with_(dtype="f32", name="bwd_full")
    inp = make_inputs(w)
    d_o = upstream(w, 2001)
    got = run_gpu(w, inp, d_o)
    full_size_check(w, got, inp, d_o, (0, 5), causal=False)


# ---------------------------------------------------------------------------- causal


def run_gpu_causal(w: Workload, inp, d_o):
    d = to_device(inp)
    g = gb.gma_backward_causal(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], d_o.cuda(), w.eps)
    torch.cuda.synchronize()
    return {k: to_np(v) for k, v in g.items()}


def run_oracle_causal(w: Workload, inp, d_o):
    return oracle.backward.backward_causal(inp["xq"], inp["xk"], inp["v"], inp["mu"], inp["sigma2"], inp["pi"],
                                           w.eps, d_o)


CAUSAL_CASES = [
    WORKLOADS["bidir_small_f32"].with_(causal=True),
    case(1000, 101, B=2, H=3, d_r=7, d_v=5, K=13),       # ragged dims, 16 segments of one tile
    case(2, 102),                                        # two positions
    case(3000, 103, d_r=32, d_v=64, K=64),              # several tiles per segment, ragged tail
    case(300, 104, B=1, H=1, d_r=128, d_v=128, K=256),  # maximum dims (half-height tiles)
    case(700, 105, B=3, H=2, d_r=64, d_v=32, K=128, mu_std=1.5),
    # the register-tiled causal passes (K, d_r, d_v <= 64, multiples of 4, within LDS)
    case(1000, 108, B=2, H=2, d_r=32, d_v=32, K=32),
    case(333, 109, B=2, H=1, d_r=64, d_v=64, K=32),     # ragged tail, one tile per segment
    case(4100, 110, B=4, H=16, d_r=64, d_v=48, K=20),   # several tiles per segment, K below a row group
    case(500, 111, B=1, H=2, d_r=64, d_v=64, K=256),
    # the K-blocked causal passes (K <= 256; d_r, d_v <= 64, multiples of 4)
    case(1500, 113, B=2, H=2, d_r=32, d_v=48, K=200),    # a partial last component block
    case(130, 114, B=1, H=3, d_r=16, d_v=16, K=66),      # K not a multiple of 4, ragged tail
    case(1000, 115, B=1, H=2, d_r=64, d_v=64, K=64),     # one component block
    case(4500, 112, B=2, H=16, d_r=16, d_v=16, K=72),    # two tiles per segment, ragged tail
]


@pytest.mark.parametrize("w", CAUSAL_CASES, ids=cid)
def test_backward_causal_parity(w):
    inp = make_inputs(w)
    d_o = upstream(w, w.seed + 1000)
    got, ref = run_gpu_causal(w, inp, d_o), run_oracle_causal(w, inp, d_o)
    check_all(got, ref, magnitudes(w.with_(causal=True), inp, d_o), where="causal-" + cid(w))


def test_backward_causal_deterministic():
    w = case(3000, 106, B=2, H=2)
    inp = make_inputs(w)
    d_o = upstream(w, 1106)
    a, b = run_gpu_causal(w, inp, d_o), run_gpu_causal(w, inp, d_o)
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k


def test_backward_causal_no_rows_gives_zero_parameter_gradients():
    w = case(0, 107)
    inp = make_inputs(w)
    d = to_device(inp)
    g = gb.gma_backward_causal(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"],
                               torch.empty(w.B, w.H, 0, w.d_v, device="cuda"), w.eps)
    torch.cuda.synchronize()
    for k in ("dmu", "dsigma2", "dpi"):
        assert not to_np(g[k]).any(), k


def test_backward_causal_full_size_sampled_heads():
    """The B=8, H=12, N=2048, d_r=d_v=64, K=32 causal dims in fp32: every gradient of two heads
    (all eight sequences each) against the oracle."""
    w = WORKLOADS["causal_b8h12_n2048"].with_(dtype="f32", name="bwdc_full")
    inp = make_inputs(w)
    d_o = upstream(w, 2002)
    got = run_gpu_causal(w, inp, d_o)
    full_size_check(w, got, inp, d_o, (0, 11), causal=True)


@pytest.mark.parametrize("name,head", [("bwd_b8h8_n1024_k256_f32", 3), ("bwdc_b8h8_n1024_k256_f32", 6)],
                         ids=["bidir", "causal"])
def test_backward_kblocked_full_size_sampled_head(name, head):
    """B=8, H=8, N=1024, d_r=d_v=64 with K=256 components (the language-model setting of the
    paper's experiments), fp32, in the split plan the bench times (the K-blocked passes): every
    gradient of one head, all eight sequences, against the oracle."""
    w = WORKLOADS[name]
    inp = make_inputs(w)
    d_o = upstream(w, 2003)
    got = (run_gpu_causal if w.causal else run_gpu)(w, inp, d_o)
    full_size_check(w, got, inp, d_o, (head,), causal=w.causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dims", [(700, 16, 32, 8), (700, 7, 5, 13), (300, 32, 64, 64)],
                         ids=lambda d: "N%d-dr%d-dv%d-K%d" % d)
def test_backward_ignores_workspace_contents(causal, dims):
    """Every scratch value (split partials, segment memories and totals, per-position D and a,
    moments) is written before it is read: a workspace of NaN bytes, reused across calls, gives
    the same gradients bit for bit as a fresh one."""
    N, dr, dv, K = dims
    w = case(N, 120 + N % 89, B=2, H=3, d_r=dr, d_v=dv, K=K, causal=causal)
    inp = make_inputs(w)
    d = to_device(inp)
    d_o = upstream(w, 1120).cuda()
    fn = gb.gma_backward_causal if causal else gb.gma_backward_bidir
    op = gb.GMA_OP_BACKWARD_CAUSAL if causal else gb.GMA_OP_BACKWARD_BIDIR
    nbytes = gb.gma_workspace_size(op, w.B, w.H, w.N, w.d_r, w.d_v, w.K, gb.GMA_F32)
    args = (d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], d_o, w.eps)
    clean = fn(*args, workspace=torch.zeros(nbytes, dtype=torch.uint8, device="cuda"))
    dirty_ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        dirty = fn(*args, workspace=dirty_ws)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(clean[k], dirty[k]), k


# ---------------------------------------------------------------------------- cross-attention


def cross_case(Nq, Nk, seed, **kw):
    return WORKLOADS["bidir_small_f32"].with_(name="bwdx", N=Nq, n_ctx=Nk, seed=seed, **dict(dict(B=1, H=2), **kw))


def xid(w):
    return "%s-q%d-k%d-dr%d-dv%d-K%d" % (w.dtype, w.N, w.n_ctx, w.d_r, w.d_v, w.K)


CROSS_CASES = [
    cross_case(200, 333, 131),                                   # tiled
    cross_case(1000, 3000, 132, d_r=64, d_v=64, K=64),           # longer context, several splits
    cross_case(3000, 700, 133, d_r=32, d_v=64, K=64),            # more queries than keys
    cross_case(257, 100, 134, d_r=7, d_v=5, K=13),               # general kernels
    cross_case(130, 450, 135, B=1, H=1, d_r=128, d_v=128, K=256),
    cross_case(700, 1900, 140, d_r=64, d_v=64, K=128),          # K-blocked passes, longer context
    cross_case(2100, 300, 141, d_r=32, d_v=32, K=192),          # K-blocked passes, more queries
    cross_case(500, 800, 148, d_r=16, d_v=32, K=130),           # K-blocked, K not a multiple of 4
    cross_case(300, 0, 136),                                     # empty context
    cross_case(0, 300, 137),                                     # no queries
    cross_case(300, 0, 142, d_r=32, d_v=32, K=128),              # empty context, K-blocked passes
    cross_case(0, 300, 143, d_r=32, d_v=32, K=128),              # no queries, K-blocked passes
    cross_case(1000, 3000, 138, d_r=64, d_v=64, K=64, dtype="bf16"),
]


@pytest.mark.parametrize("w", CROSS_CASES, ids=xid)
def test_backward_cross_parity(w):
    inp = make_inputs(w)
    d_o = upstream(w, w.seed + 1000)
    if w.dtype == "bf16":
        d_o = d_o.bfloat16()
    d = to_device(inp)
    g = gb.gma_backward_cross(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], d_o.cuda(), w.eps)
    torch.cuda.synchronize()
    ref = run_oracle(w, inp, d_o)
    mag = magnitudes(w, inp, d_o, causal=False)
    for k in KEYS:
        got = to_np(g[k])
        assert got.shape == ref[k].shape and np.isfinite(got).all(), k
        tol = TOL_BWD_BF16 if (w.dtype == "bf16" and k in ("dXQ", "dXK", "dV")) else TOL_BWD
        if ref[k].size == 0:
            continue
        if np.abs(mag[k]).max() == 0.0:
            assert not got.any(), k   # exact zeros: an empty side
        else:
            err = entry_error(got, ref[k], mag[k])
            assert err <= tol, (k, err)


def test_backward_cross_equal_lengths_is_bidir_bitwise():
    """With N_q = N_k the cross backward runs the bidirectional backward's plan: identical bits."""
    w = cross_case(2900, 2900, 139, B=2, H=3, d_r=32, d_v=32, K=32)
    inp = make_inputs(w)
    d = to_device(inp)
    d_o = upstream(w, 1139).cuda()
    args = (d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], d_o, w.eps)
    a, b = gb.gma_backward_cross(*args), gb.gma_backward_bidir(*args)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(a[k], b[k]), k


# ---------------------------------------------------------------------------- carried memory


def carried(w, seed):
    """A carried memory (Z >= 0) and a gradient for the memory after the call, [B,H,K,d_v+1]."""
    gen = torch.Generator().manual_seed(seed)
    s = torch.randn(w.B, w.H, w.K, w.d_v + 1, generator=gen, dtype=torch.float32)
    s[..., -1] = s[..., -1].abs() * 3.0
    ds = torch.randn(w.B, w.H, w.K, w.d_v + 1, generator=gen, dtype=torch.float32)
    return s, ds


STATE_CASES = [
    case(700, 141),                                         # tiled causal passes
    case(1000, 142, B=2, H=2, d_r=64, d_v=64, K=32),
    case(500, 143, B=2, H=3, d_r=7, d_v=5, K=13),          # one element per thread (LDS tables)
    case(300, 144, d_r=32, d_v=64, K=64),                  # K-blocked, one component block
    case(200, 145, B=1, H=1, d_r=128, d_v=128, K=256),     # one element per thread (general)
    case(260, 147, B=1, H=2, d_r=64, d_v=64, K=200),       # K-blocked, four component blocks
]


@pytest.mark.parametrize("w", STATE_CASES, ids=cid)
def test_backward_causal_state_parity(w):
    w = w.with_(causal=True)
    inp = make_inputs(w)
    d_o = upstream(w, w.seed + 1000)
    s, ds = carried(w, w.seed + 2000)
    d = to_device(inp)
    g = gb.gma_backward_causal_state(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], d_o.cuda(), w.eps,
                                     state_in=s.cuda(), dstate_out=ds.cuda())
    torch.cuda.synchronize()
    ref = oracle.backward.backward_causal(inp["xq"], inp["xk"], inp["v"], inp["mu"], inp["sigma2"], inp["pi"], w.eps,
                                          d_o, state_in=s, dstate_out=ds)
    mag = magnitudes(w, inp, d_o, state_in=s, dstate_out=ds)
    check_all({k: to_np(v) for k, v in g.items()}, ref, mag, keys=KEYS + ("dstate_in",), where="state-" + cid(w))


@pytest.mark.parametrize("dims", [(32, 32, 32), (32, 32, 128)], ids=lambda d: "dr%d-dv%d-K%d" % d)
def test_backward_causal_state_chained_calls_equal_whole_sequence(dims):
    """Three calls over consecutive pieces, forward state carried and dstate_in fed back as the
    previous call's dstate_out, give the whole-sequence backward (register-tiled passes at K = 32,
    K-blocked at K = 128)."""
    dr, dv, K = dims
    w = case(1000, 146, B=2, H=2, d_r=dr, d_v=dv, K=K, causal=True)
    inp = make_inputs(w)
    d_o = upstream(w, 1146)
    d = to_device(inp)
    cuts = [0, 300, 301, 1000]
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    states = [None]
    for a, b in zip(cuts[:-1], cuts[1:]):  # forward: the memory before each piece
        _, so = gb.gma_forward_causal_state(sl(d["xq"], a, b), sl(d["xk"], a, b), sl(d["v"], a, b), d["mu"],
                                            d["sigma2"], d["pi"], w.eps, state_in=states[-1])
        states.append(so)
    grads, dso = [None] * 3, None
    for i in (2, 1, 0):
        a, b = cuts[i], cuts[i + 1]
        grads[i] = gb.gma_backward_causal_state(sl(d["xq"], a, b), sl(d["xk"], a, b), sl(d["v"], a, b), d["mu"],
                                                d["sigma2"], d["pi"], sl(d_o, a, b).cuda(), w.eps,
                                                state_in=states[i], dstate_out=dso)
        dso = grads[i]["dstate_in"]
    torch.cuda.synchronize()
    ref = oracle.backward.backward_causal(inp["xq"], inp["xk"], inp["v"], inp["mu"], inp["sigma2"], inp["pi"], w.eps,
                                          d_o)
    got = {k: np.concatenate([to_np(gr[k]) for gr in grads], axis=2) for k in ("dXQ", "dXK", "dV")}
    got.update({k: sum(to_np(gr[k]) for gr in grads) for k in ("dmu", "dsigma2", "dpi")})
    check_all(got, ref, magnitudes(w, inp, d_o), where="chained")


def test_backward_causal_state_empty_call():
    """No positions: dstate_in = dstate_out exactly, zero parameter gradients."""
    w = case(0, 147, causal=True)
    inp = make_inputs(w)
    d = to_device(inp)
    s, ds = carried(w, 2147)
    g = gb.gma_backward_causal_state(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"],
                                     torch.empty(w.B, w.H, 0, w.d_v, device="cuda"), w.eps, state_in=s.cuda(),
                                     dstate_out=ds.cuda())
    torch.cuda.synchronize()
    assert torch.equal(g["dstate_in"].cpu(), ds)
    for k in ("dmu", "dsigma2", "dpi"):
        assert not to_np(g[k]).any(), k


# ---------------------------------------------------------------------------- autograd


@pytest.mark.parametrize("variant", ["bidir", "causal", "cross"])
def test_autograd_functions_match_oracle(variant):
    """torch.autograd through gaussian_mixture_sequence_amd.autograd: the loss <dO, O> back-propagates
    to the oracle's gradients."""
    from gaussian_mixture_sequence_amd import autograd as ga
    if variant == "cross":
        w = cross_case(300, 500, 151, d_r=32, d_v=32, K=32)
    else:
        w = case(700, 152, B=2, H=2, d_r=32, d_v=32, K=32, causal=variant == "causal")
    inp = make_inputs(w)
    d_o = upstream(w, 1151)
    leaves = {k: t.cuda().requires_grad_(True) for k, t in inp.items()}
    fn = {"bidir": ga.gma_bidir, "causal": ga.gma_causal, "cross": ga.gma_cross}[variant]
    out = fn(leaves["xq"], leaves["xk"], leaves["v"], leaves["mu"], leaves["sigma2"], leaves["pi"], w.eps)
    (out * d_o.cuda()).sum().backward()
    torch.cuda.synchronize()
    ref_fn = oracle.backward.backward_causal if variant == "causal" else oracle.backward.backward_bidir
    ref = ref_fn(inp["xq"], inp["xk"], inp["v"], inp["mu"], inp["sigma2"], inp["pi"], w.eps, d_o)
    got = {k: to_np(leaves[name].grad) for k, name in zip(KEYS, ("xq", "xk", "v", "mu", "sigma2", "pi"))}
    check_all(got, ref, magnitudes(w, inp, d_o, causal=variant == "causal"), where="autograd-" + variant)
