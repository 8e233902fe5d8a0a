"""GPU parity: libgma.so (through the C ABI) against the fp64 oracle, element by element,
on the same seeded inputs.  Tolerances (row-scaled error, see gma_testutil): 1e-5 for
fp32 I/O, 2e-2 for bf16 I/O with fp32 accumulation."""
import numpy as np
import pytest
import torch

import oracle
from gaussian_mixture_sequence_amd import binding as gb
from gaussian_mixture_sequence_amd.inputs import WORKLOADS, Workload, make_inputs
from gma_testutil import TOL, row_scaled_error, to_device, to_np

pytestmark = pytest.mark.gpu


def run_gpu(w: Workload, inp, chunk=None):
    d = to_device(inp)
    if w.causal:
        out = gb.gma_forward_causal(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps,
                                    chunk=chunk or w.chunk)
    else:
        out = gb.gma_forward_bidir(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps)
    torch.cuda.synchronize()
    return out


def run_oracle(w: Workload, inp):
    fn = oracle.forward_causal if w.causal else oracle.forward_bidir
    return fn(inp["xq"], inp["xk"], inp["v"], inp["mu"], inp["sigma2"], inp["pi"], w.eps)


def small(name, **kw):
    return WORKLOADS[name].with_(**kw)


F32_CASES = [
    WORKLOADS["bidir_small_f32"],                                        # the fp32 workload itself
    small("bidir_small_f32", B=2, H=3, N=200, seed=11),                 # ragged tail, several heads
    small("bidir_small_f32", B=1, H=2, N=1000, d_r=7, d_v=5, K=13, seed=12),
    small("bidir_small_f32", N=1, d_r=3, d_v=2, K=1, seed=13),          # single token, K = 1
    small("bidir_small_f32", N=130, d_r=128, d_v=128, K=256, seed=14),  # maximum dims
    small("bidir_small_f32", causal=True, B=2, H=2, N=300, seed=15),
    small("bidir_small_f32", causal=True, N=777, d_r=5, d_v=9, K=6, chunk=16, seed=16),
    small("bidir_small_f32", causal=True, N=1500, K=20, chunk=32, seed=17),  # several segments
    small("bidir_small_f32", causal=True, N=100, d_r=128, d_v=128, K=256, seed=18),
]


@pytest.mark.parametrize("w", F32_CASES, ids=lambda w: "%s-%s-B%dH%dN%d-dr%d-dv%d-K%d" % (
    "causal" if w.causal else "bidir", w.dtype, w.B, w.H, w.N, w.d_r, w.d_v, w.K))
def test_f32_parity(w):
    inp = make_inputs(w)
    out = run_gpu(w, inp)
    assert out.dtype == torch.float32 and out.shape == (w.B, w.H, w.N, w.d_v)
    err = row_scaled_error(to_np(out), run_oracle(w, inp))
    assert err <= TOL["f32"], err


@pytest.mark.parametrize("gamma_dtype", [torch.float32, torch.bfloat16])
def test_f32_responsibilities(gamma_dtype):
    w = small("bidir_small_f32", B=2, H=3, N=333, K=40, seed=21)
    inp = make_inputs(w)
    d = to_device(inp)
    g = gb.gma_responsibilities(d["xq"], d["mu"], d["sigma2"], d["pi"], gamma_dtype=gamma_dtype)
    torch.cuda.synchronize()
    ref = oracle.responsibilities(inp["xq"], inp["mu"], inp["sigma2"], inp["pi"])
    err = np.abs(to_np(g) - ref).max()
    assert err <= (2e-6 if gamma_dtype == torch.float32 else 4e-3), err
    assert np.abs(to_np(g).sum(-1) - 1).max() <= (1e-5 if gamma_dtype == torch.float32 else 2e-2)


def test_f32_deterministic_and_prefix_invariant():
    w = small("bidir_small_f32", causal=True, B=1, H=2, N=700, seed=22)
    inp = make_inputs(w)
    a = to_np(run_gpu(w, inp))
    b = to_np(run_gpu(w, inp))
    assert np.array_equal(a, b)
    i = 345
    pert = {k: v.clone() for k, v in inp.items()}
    g = torch.Generator().manual_seed(5)
    for k in ("xq", "xk", "v"):
        pert[k][:, :, i + 1:] += torch.randn(pert[k][:, :, i + 1:].shape, generator=g).to(pert[k].dtype)
    c = to_np(run_gpu(w, pert))
    assert np.array_equal(c[:, :, :i + 1], a[:, :, :i + 1])


# ----------------------------------------------------------------------------- bf16 MFMA path

def bf16_case(causal=False, **kw):
    base = WORKLOADS["causal_b8h12_n2048" if causal else "bidir_b8h8_n4096"]
    return base.with_(**kw)


BF16_RESP_CASES = [(64, 64), (32, 128), (16, 8), (128, 256), (64, 50), (16, 256), (128, 32)]


@pytest.mark.parametrize("dr,K", BF16_RESP_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("gamma_dtype", [torch.float32, torch.bfloat16])
def test_bf16_responsibilities(dr, K, gamma_dtype):
    w = bf16_case(B=2, H=3, N=333, d_r=dr, K=K, seed=31 + dr + K)
    inp = make_inputs(w)
    d = to_device(inp)
    g = gb.gma_responsibilities(d["xq"], d["mu"], d["sigma2"], d["pi"], gamma_dtype=gamma_dtype)
    torch.cuda.synchronize()
    ref = oracle.responsibilities(inp["xq"], inp["mu"], inp["sigma2"], inp["pi"])
    err = np.abs(to_np(g) - ref).max()
    # score error of the split-operand MFMA (~1e-4 in Gamma) plus the output rounding
    assert err <= (2e-3 if gamma_dtype == torch.float32 else 6e-3), err


BF16_BIDIR_CASES = [
    bf16_case(B=1, H=2, N=1000, seed=41),                                   # the B8H8 shapes, short
    bf16_case(B=2, H=1, N=777, d_r=32, d_v=64, K=128, mu_std=1.5, seed=42),  # long-context dims
    bf16_case(B=1, H=1, N=300, d_r=16, d_v=32, K=8, seed=43),               # K padded to 32
    bf16_case(B=1, H=1, N=200, d_r=128, d_v=128, K=256, seed=44),           # maximum dims
    bf16_case(B=1, H=3, N=1, seed=45),                                      # single token
    bf16_case(B=1, H=1, N=129, d_r=64, d_v=32, K=50, seed=46),              # ragged everything
    bf16_case(B=1, H=2, N=5000, d_r=64, d_v=128, K=256, seed=47),           # several splits
    bf16_case(B=1, H=2, N=900, d_r=32, d_v=64, K=100, seed=140),            # K padded 100 -> 128
    bf16_case(B=1, H=1, N=700, d_r=64, d_v=32, K=150, seed=141),            # K padded 150 -> 256
    bf16_case(B=2, H=1, N=500, d_r=16, d_v=128, K=200, seed=142),           # K padded 200 -> 256
]


def case_id(w):
    return "%s-B%dH%dN%d-dr%d-dv%d-K%d" % ("causal" if w.causal else "bidir", w.B, w.H, w.N, w.d_r, w.d_v, w.K)


@pytest.mark.parametrize("w", BF16_BIDIR_CASES, ids=case_id)
def test_bf16_bidir_parity(w):
    inp = make_inputs(w)
    out = run_gpu(w, inp)
    assert out.dtype == torch.bfloat16 and out.shape == (w.B, w.H, w.N, w.d_v)
    err = row_scaled_error(to_np(out), run_oracle(w, inp))
    assert err <= TOL["bf16"], err


def sampled_heads(w, inp, out, heads):
    """Oracle on a few full (b, h) problems of a full-size run."""
    from gaussian_mixture_sequence_amd.inputs import head_slice
    worst = 0.0
    for b, h in heads:
        sl = head_slice(inp, b, h)
        ref = run_oracle(w.with_(B=1, H=1), sl)[0, 0]
        worst = max(worst, row_scaled_error(to_np(out[b, h]), ref))
    return worst


@pytest.mark.parametrize("name", ["bidir_b8h8_n4096", "bidir_long_n65536"])
def test_bf16_bidir_full_size_sampled(name):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    out = run_gpu(w, inp)
    assert torch.isfinite(out.float()).all()
    err = sampled_heads(w, inp, out, [(0, 0), (w.B - 1, w.H - 1)])
    assert err <= TOL["bf16"], err


def test_bf16_bidir_deterministic():
    w = bf16_case(B=2, H=2, N=3000, seed=48)
    inp = make_inputs(w)
    a = to_np(run_gpu(w, inp))
    b = to_np(run_gpu(w, inp))
    assert np.array_equal(a, b)


BF16_CAUSAL_CASES = [
    bf16_case(causal=True, B=1, H=2, N=700, seed=51),                                   # B8H12 dims, short
    bf16_case(causal=True, B=1, H=1, N=600, d_r=64, d_v=128, K=256, seed=52),           # long-causal dims
    bf16_case(causal=True, B=1, H=2, N=300, d_r=16, d_v=32, K=8, chunk=32, seed=53),    # K padded, chunk 32
    bf16_case(causal=True, B=1, H=1, N=1, seed=54),                                     # single token
    bf16_case(causal=True, B=2, H=1, N=3001, d_r=32, d_v=64, K=128, chunk=64, seed=55),  # several segments
    bf16_case(causal=True, B=1, H=1, N=260, d_r=128, d_v=128, K=256, seed=56),          # maximum dims
    bf16_case(causal=True, B=1, H=1, N=777, d_r=64, d_v=32, K=50, chunk=32, seed=57),   # ragged, chunk 32
    bf16_case(causal=True, B=1, H=2, N=900, d_r=32, d_v=64, K=100, seed=143),           # K padded 100 -> 128
    bf16_case(causal=True, B=1, H=1, N=700, d_r=32, d_v=64, K=150, seed=144),           # K padded 150 -> 256
    bf16_case(causal=True, B=2, H=1, N=500, d_r=16, d_v=128, K=200, seed=145),          # K padded 200 -> 256
]


@pytest.mark.parametrize("w", BF16_CAUSAL_CASES, ids=case_id)
def test_bf16_causal_parity(w):
    inp = make_inputs(w)
    out = run_gpu(w, inp)
    assert out.dtype == torch.bfloat16 and out.shape == (w.B, w.H, w.N, w.d_v)
    err = row_scaled_error(to_np(out), run_oracle(w, inp))
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("name,heads", [("causal_b8h12_n2048", [(0, 0), (7, 11)]),
                                        ("causal_long_n32768", [(1, 15)])])
def test_bf16_causal_full_size_sampled(name, heads):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    out = run_gpu(w, inp)
    assert torch.isfinite(out.float()).all()
    err = sampled_heads(w, inp, out, heads)
    assert err <= TOL["bf16"], err


def test_bf16_causal_prefix_invariance_and_determinism():
    """Output rows <= i are bit-identical when inputs after i change (Sec. 3.5 causality);
    two runs on the same inputs are bit-identical."""
    w = bf16_case(causal=True, B=1, H=2, N=2500, seed=58)
    inp = make_inputs(w)
    a = to_np(run_gpu(w, inp))
    assert np.array_equal(a, to_np(run_gpu(w, inp)))
    for i in (100, 1337):
        pert = {k: v.clone() for k, v in inp.items()}
        g = torch.Generator().manual_seed(i)
        for k in ("xq", "xk", "v"):
            pert[k][:, :, i + 1:] = torch.randn(pert[k][:, :, i + 1:].shape, generator=g).to(pert[k].dtype)
        c = to_np(run_gpu(w, pert))
        assert np.array_equal(c[:, :, :i + 1], a[:, :, :i + 1])
        assert not np.array_equal(c[:, :, i + 1:], a[:, :, i + 1:])


def test_bf16_causal_chunk_invariance():
    """The chunk length only reorders sums: results for chunk 32 and 64 agree to tolerance."""
    w = bf16_case(causal=True, B=1, H=2, N=1000, seed=59)
    inp = make_inputs(w)
    a = to_np(run_gpu(w, inp, chunk=32))
    b = to_np(run_gpu(w, inp, chunk=64))
    assert row_scaled_error(a, b) <= 1e-2


@pytest.mark.parametrize("w", [small("bidir_small_f32", causal=True, B=1, H=2, N=1000, seed=146),
                               bf16_case(causal=True, B=1, H=2, N=1000, seed=147),
                               bf16_case(causal=True, B=1, H=1, N=700, d_r=64, d_v=128, K=256, seed=148)],
                         ids=lambda w: "%s-K%d" % (w.dtype, w.K))
def test_causal_chunk_128(w):
    """Chunk 128, the longest of the chunk set: parity with the oracle, and the same bits as the
    request whose chunk length the scan actually runs (gma_plan_info's chunk_used)."""
    io = gb.GMA_BF16 if w.dtype == "bf16" else gb.GMA_F32
    used = gb.gma_plan_info(gb.GMA_OP_CAUSAL, w.B, w.H, w.N, w.d_r, w.d_v, w.K, io, 128)["chunk_used"]
    inp = make_inputs(w)
    a = to_np(run_gpu(w, inp, chunk=128))
    assert row_scaled_error(a, run_oracle(w, inp)) <= TOL[w.dtype]
    assert np.array_equal(a, to_np(run_gpu(w, inp, chunk=used)))


def test_bf16_causal_last_row_matches_bidir():
    """At the last position the causal prefix memory is the full memory (Eq. 6b vs Eq. 6)."""
    w = bf16_case(causal=True, B=1, H=2, N=1500, seed=60)
    inp = make_inputs(w)
    c = to_np(run_gpu(w, inp))
    b = to_np(run_gpu(w.with_(causal=False), inp))
    assert row_scaled_error(c[:, :, -1:], b[:, :, -1:]) <= 1e-2


@pytest.mark.parametrize("causal", [False, True], ids=["bidir", "causal"])
def test_bf16_workspace_reuse_and_garbage(causal):
    """The fused kernels hand data between workgroups through flag words in the workspace,
    matched against a fresh per-call token: a workspace full of garbage, or one left by
    earlier calls on other inputs, gives bit-identical results to a fresh one."""
    w = bf16_case(causal=causal, B=2, H=3, N=2900, seed=61)
    inp_a, inp_b = make_inputs(w), make_inputs(w.with_(seed=62))
    ref_a, ref_b = to_np(run_gpu(w, inp_a)), to_np(run_gpu(w, inp_b))
    op = gb.GMA_OP_CAUSAL if causal else gb.GMA_OP_BIDIR
    nbytes = gb.gma_workspace_size(op, w.B, w.H, w.N, w.d_r, w.d_v, w.K, gb.GMA_BF16, w.chunk if causal else 0)
    g = torch.Generator(device="cuda").manual_seed(7)
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    for inp, ref in [(inp_a, ref_a), (inp_b, ref_b), (inp_a, ref_a), (inp_a, ref_a), (inp_b, ref_b)]:
        d = to_device(inp)
        if causal:
            out = gb.gma_forward_causal(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps,
                                        chunk=w.chunk, workspace=ws)
        else:
            out = gb.gma_forward_bidir(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(out), ref)


@pytest.mark.parametrize("causal", [False, True], ids=["bidir", "causal"])
def test_bf16_wait_timeout_gives_nan(causal):
    """Failure path of the in-launch hand-off, forced from the host: with a wait bound of 0
    every workgroup's wait fails at once, the launch still ends, every output row is NaN (and
    so is the carried memory of a causal call), and gma_device_status reports the timeout once.
    Restoring the default bound gives the normal result again, with no error reported."""
    w = bf16_case(causal=causal, B=1, H=2, N=1500, seed=63)
    inp = make_inputs(w)
    ref = to_np(run_gpu(w, inp))
    assert gb.gma_device_status() == gb.GMA_OK
    state = None
    try:
        gb.gma_set_wait_limit(0)
        if causal:
            d = to_device(inp)
            state = torch.zeros(w.B, w.H, w.K, w.d_v + 1, dtype=torch.float32, device="cuda")
            out, _ = gb.gma_forward_causal_state(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps,
                                                 chunk=w.chunk, state_out=state)
            torch.cuda.synchronize()
            out = to_np(out)
        else:
            out = to_np(run_gpu(w, inp))
    finally:
        gb.gma_set_wait_limit(gb.WAIT_LIMIT_DEFAULT)
    assert np.isnan(out).all()
    if causal:
        assert torch.isnan(state).all()
    assert gb.gma_device_status() == gb.GMA_ERR_TIMEOUT
    assert gb.gma_device_status() == gb.GMA_OK  # taking the status clears it
    assert np.array_equal(to_np(run_gpu(w, inp)), ref)
    assert gb.gma_device_status() == gb.GMA_OK


BF16_SPLIT_LAUNCH_CASES = [
    bf16_case(B=2, H=3, N=2900, seed=64),
    bf16_case(B=1, H=1, N=70000, d_r=32, d_v=64, K=128, mu_std=1.5, seed=65),
    bf16_case(causal=True, B=2, H=3, N=2900, seed=66),
    bf16_case(causal=True, B=1, H=2, N=3001, d_r=32, d_v=64, K=128, seed=67),
    bf16_case(causal=True, B=1, H=1, N=1100, d_r=64, d_v=128, K=256, seed=68),
]


@pytest.mark.parametrize("w", BF16_SPLIT_LAUNCH_CASES, ids=case_id)
def test_bf16_single_launch_off_is_bitwise_equal(w):
    """gma_set_single_launch(0) runs every phase as its own launch (no workgroup waits for another):
    the same arithmetic in the same order, so the outputs are bit-identical."""
    inp = make_inputs(w)
    a = to_np(run_gpu(w, inp))
    try:
        gb.gma_set_single_launch(False)
        b = to_np(run_gpu(w, inp))
    finally:
        gb.gma_set_single_launch(True)
    assert np.array_equal(a, b)
    assert gb.gma_device_status() == gb.GMA_OK


def test_bf16_bidir_one_head_long_sequence():
    """One problem (B = H = 1) of 262144 positions at the largest per-workgroup LDS (d_r 64, d_v 128,
    K 256): the split count is bounded by the workgroups the device keeps resident, and with more
    than 8 splits the phases run as their own launches; every row against the oracle."""
    w = bf16_case(B=1, H=1, N=262144, d_r=64, d_v=128, K=256, seed=69)
    info = gb.gma_plan_info(gb.GMA_OP_BIDIR, w.B, w.H, w.N, w.d_r, w.d_v, w.K, gb.GMA_BF16)
    assert info["workgroups"] <= info["resident_bound"]
    assert info["waits_on_all_splits"] == (1 if 1 < info["splits"] <= 8 else 0)
    inp = make_inputs(w)
    out = run_gpu(w, inp)
    assert gb.gma_device_status() == gb.GMA_OK
    err = row_scaled_error(to_np(out), run_oracle(w, inp))
    assert err <= TOL["bf16"], err
