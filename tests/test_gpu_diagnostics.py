"""GPU parity of the responsibility diagnostics (Sec. 5.4, Eq. 24-29) through the C ABI
against the oracle's (numpy fp64 over the oracle's responsibilities)."""
import numpy as np
import pytest
import torch

import oracle
from gaussian_mixture_sequence_amd import binding as gb
from gaussian_mixture_sequence_amd.inputs import WORKLOADS, make_inputs
from gma_testutil import to_np

pytestmark = pytest.mark.gpu

# tolerances: fp32 responsibilities are exact to ~1e-7; bf16 ones carry the split-operand MFMA
# score error (~1e-3 in a responsibility at worst, far less on average)
TOL = {"f32": dict(g=2e-6, u=2e-6, s=2e-6), "bf16": dict(g=2e-3, u=5e-4, s=2e-3)}


def run(w):
    inp = make_inputs(w)
    d = {k: inp[k].cuda() for k in ("xq", "mu", "sigma2", "pi")}
    out = gb.gma_responsibility_diagnostics(d["xq"], d["mu"], d["sigma2"], d["pi"], want_argmax=True, want_gbar=True)
    torch.cuda.synchronize()
    ref = oracle.diagnostics.diagnostics(inp["xq"], inp["mu"], inp["sigma2"], inp["pi"])
    return out, ref


def check(w, out, ref):
    t = TOL[w.dtype]
    assert np.abs(to_np(out["gbar"]) - ref["gbar"]).max() <= t["g"]
    assert np.abs(to_np(out["usage"]) - ref["usage"]).max() <= t["u"]
    for k in ("h_usage", "h_token", "r_max"):
        assert abs(float(out[k]) - ref[k]) <= t["s"], k
    # Eq. 29: the argmax is unique where the reference's two largest values are apart by more
    # than twice the responsibility tolerance; elsewhere the GPU's pick must be one of the
    # near-maximal components
    z = to_np(out["argmax"]).astype(np.int64).reshape(-1)
    g = ref["gbar"].reshape(-1, ref["gbar"].shape[-1])
    zr = ref["argmax"].reshape(-1)
    srt = np.sort(g, axis=1)
    gap = srt[:, -1] - (srt[:, -2] if g.shape[1] > 1 else -np.inf)
    clear = gap > 2 * t["g"]
    assert np.array_equal(z[clear], zr[clear])
    picked = g[np.arange(len(z)), z]
    assert (picked >= g.max(axis=1) - 2 * t["g"]).all()


def case(dtype, **kw):
    base = WORKLOADS["bidir_small_f32" if dtype == "f32" else "bidir_b8h8_n4096"]
    return base.with_(**kw)


CASES = [
    case("f32", B=2, H=3, N=333, seed=111),
    case("f32", B=3, H=2, N=100, d_r=7, K=13, seed=112),
    case("bf16", B=2, H=4, N=1000, d_r=64, K=128, seed=113),
    case("bf16", B=1, H=2, N=257, d_r=128, K=256, seed=114),
    case("bf16", B=3, H=3, N=70, d_r=32, K=50, seed=115),
    case("bf16", B=2, H=2, N=65, d_r=16, K=1, seed=116),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: "%s-B%dH%dN%d-dr%d-K%d" % (w.dtype, w.B, w.H, w.N, w.d_r, w.K))
def test_diagnostics_parity(w):
    out, ref = run(w)
    check(w, out, ref)


def test_diagnostics_paper_setting():
    """The paper's diagnostic setting (64 sequences, 8 heads, 1024 positions, K = 128) with the
    routing dim d_model / H = 64, bf16 inputs, at full size."""
    w = WORKLOADS["diag_s64_h8_l1024_k128"]
    out, ref = run(w)
    check(w, out, ref)


def test_diagnostics_deterministic_and_empty():
    w = case("bf16", B=2, H=3, N=500, K=64, seed=117)
    inp = make_inputs(w)
    d = {k: inp[k].cuda() for k in ("xq", "mu", "sigma2", "pi")}
    a = gb.gma_responsibility_diagnostics(d["xq"], d["mu"], d["sigma2"], d["pi"])
    b = gb.gma_responsibility_diagnostics(d["xq"], d["mu"], d["sigma2"], d["pi"])
    torch.cuda.synchronize()
    assert torch.equal(a["usage"], b["usage"]) and torch.equal(a["argmax"], b["argmax"])
    assert all(float(a[k]) == float(b[k]) for k in ("h_usage", "h_token", "r_max"))
    e = gb.gma_responsibility_diagnostics(d["xq"][:, :, :0].contiguous(), d["mu"], d["sigma2"], d["pi"])
    torch.cuda.synchronize()
    assert not e["usage"].any() and float(e["h_usage"]) == 0 and float(e["r_max"]) == 0
