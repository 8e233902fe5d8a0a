"""GPU parity of cross-attention (queries from one sequence, keys and values from a
separate context; Sec. 3 "Cross-attention", Eq. 5-8) through the C ABI, against the fp64
oracle on the same seeded inputs.  Tolerances as for the bidirectional forward."""
import numpy as np
import pytest
import torch

import oracle
from gaussian_mixture_sequence_amd import binding as gb
from gaussian_mixture_sequence_amd.inputs import WORKLOADS, Workload, head_slice, make_inputs
from gma_testutil import TOL, row_scaled_error, to_device, to_np

pytestmark = pytest.mark.gpu


def run_gpu(w: Workload, inp, workspace=None):
    d = to_device(inp)
    out = gb.gma_forward_cross(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps, workspace=workspace)
    torch.cuda.synchronize()
    return out


def run_oracle(w: Workload, inp):
    return oracle.forward_cross(inp["xq"], inp["xk"], inp["v"], inp["mu"], inp["sigma2"], inp["pi"], w.eps)


def case(dtype, Nq, Nk, seed, **kw):
    base = WORKLOADS["bidir_small_f32" if dtype == "f32" else "bidir_b8h8_n4096"]
    return base.with_(name="cross", N=Nq, n_ctx=Nk, seed=seed, **dict(dict(B=1, H=2), **kw))


def cid(w):
    return "%s-B%dH%d-q%d-k%d-dr%d-dv%d-K%d" % (w.dtype, w.B, w.H, w.N, w.n_ctx, w.d_r, w.d_v, w.K)


CASES = [
    case("f32", 200, 333, 71),
    case("f32", 1, 1000, 72, d_r=7, d_v=5, K=13),
    case("f32", 257, 1, 73),
    case("bf16", 1000, 3000, 74),                                        # longer context
    case("bf16", 3000, 700, 75),                                         # more queries than keys
    case("bf16", 1, 5000, 76),                                           # one query, many empty query splits
    case("bf16", 3000, 100, 77),                                         # empty key splits
    case("bf16", 777, 1, 78),
    case("bf16", 200, 129, 79, d_r=16, d_v=32, K=8),                     # K padded to 32
    case("bf16", 130, 450, 80, B=1, H=1, d_r=128, d_v=128, K=256),       # maximum dims
    case("bf16", 900, 2100, 81, d_r=32, d_v=64, K=128, mu_std=1.5),      # long-context dims
]


@pytest.mark.parametrize("w", CASES, ids=cid)
def test_cross_parity(w):
    inp = make_inputs(w)
    assert inp["xk"].shape[2] == w.n_ctx and inp["xq"].shape[2] == w.N
    out = run_gpu(w, inp)
    assert out.shape == (w.B, w.H, w.N, w.d_v) and out.dtype == inp["xq"].dtype
    err = row_scaled_error(to_np(out), run_oracle(w, inp))
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cross_empty_context_gives_zeros(dtype):
    """N_k = 0: the memory and normaliser are zero, so O = 0 / eps = 0 for every query."""
    w = case(dtype, 300, 0, 82)
    inp = make_inputs(w)
    d = to_device(inp)
    out = torch.full((w.B, w.H, w.N, w.d_v), 7.0, dtype=d["xq"].dtype, device="cuda")
    gb.gma_forward_cross(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps, out=out)
    torch.cuda.synchronize()
    assert not to_np(out).any()


def test_cross_equal_lengths_is_bidir_bitwise():
    """With N_q = N_k the cross forward is the bidirectional forward on the same tensors,
    with the same split plan, hence bit-identical."""
    w = case("bf16", 2900, 2900, 83, B=2, H=3)
    inp = make_inputs(w)
    d = to_device(inp)
    a = run_gpu(w, inp)
    b = gb.gma_forward_bidir(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(a), to_np(b))


def test_cross_deterministic_and_workspace_garbage():
    """Bitwise reproducible, also from a workspace full of random bytes."""
    w = case("bf16", 1500, 4100, 84, B=2, H=2)
    inp = make_inputs(w)
    ref = to_np(run_gpu(w, inp))
    nbytes = gb.gma_cross_workspace_size(w.B, w.H, w.N, w.n_ctx, w.d_r, w.d_v, w.K, gb.GMA_BF16)
    g = torch.Generator(device="cuda").manual_seed(9)
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    for _ in range(3):
        assert np.array_equal(to_np(run_gpu(w, inp, workspace=ws)), ref)


def test_cross_full_size_sampled():
    """The B=8, H=8 cross workload (4096 queries, 16384 context rows) at full size, checked
    on sampled (batch, head) problems."""
    w = WORKLOADS["cross_b8h8_q4096_k16384"]
    inp = make_inputs(w)
    out = run_gpu(w, inp)
    assert torch.isfinite(out.float()).all()
    worst = 0.0
    for b, h in [(0, 0), (w.B - 1, w.H - 1)]:
        ref = run_oracle(w.with_(B=1, H=1), head_slice(inp, b, h))[0, 0]
        worst = max(worst, row_scaled_error(to_np(out[b, h]), ref))
    assert worst <= TOL["bf16"], worst
