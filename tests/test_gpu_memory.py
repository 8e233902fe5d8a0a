"""Memory of the forward grows linearly in N (Sec. 5.1 profiles memory against sequence length; the
method needs O(N K) work and, fused, O(N) memory): the library allocates nothing, so a call's
device memory is its inputs, output and workspace, all allocated by the caller; at the long-context
dims (B=4, H=4, d_r=32, d_v=64, K=128, bf16) the measured peak over N = 4096 .. 65536 is a line in N."""
import numpy as np
import pytest
import torch

from gaussian_mixture_sequence_amd import binding as gb
from gaussian_mixture_sequence_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [False, True], ids=["bidir", "causal"])
def test_peak_memory_linear_in_sequence_length(causal):
    """Per N: the device memory a call needs (inputs, output, workspace, allocated by the caller) and
    the peak while the call runs, which must not rise above it (nothing allocated in the call)."""
    base = WORKLOADS["bidir_long_n65536"].with_(causal=causal)
    ns, need, wsb = [], [], []
    for n in (4096, 8192, 16384, 32768, 65536):
        w = base.with_(N=n)
        torch.cuda.empty_cache()
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        d = {k: v.cuda() for k, v in make_inputs(w).items()}
        op = gb.GMA_OP_CAUSAL if causal else gb.GMA_OP_BIDIR
        nbytes = gb.gma_workspace_size(op, w.B, w.H, w.N, w.d_r, w.d_v, w.K, gb.GMA_BF16, w.chunk if causal else 0)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        out = torch.empty(w.B, w.H, w.N, w.d_v, dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        held = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        if causal:
            gb.gma_forward_causal(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps, chunk=w.chunk,
                                  out=out, workspace=ws)
        else:
            gb.gma_forward_bidir(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.cuda.max_memory_allocated() == held  # the call itself allocates nothing
        assert torch.isfinite(out.float()).all()
        ns.append(n)
        need.append(held - before)
        wsb.append(nbytes)
        del d, ws, out
    # at the full length the materialised responsibilities alone (2 B H N K fp32) exceed what the call holds
    assert need[-1] < 2 * w.B * w.H * ns[-1] * w.K * 4
    ns, need, wsb = np.array(ns, float), np.array(need, float), np.array(wsb, float)
    # inputs and output: exactly proportional to N (up to the allocator's rounding)
    per_pos = (need - wsb) / ns
    assert per_pos.max() <= 1.01 * per_pos.min(), per_pos
    # the workspace grows with the split count and then stays constant: bounded, never superlinear
    assert (np.diff(wsb) >= 0).all() and wsb.max() <= 0.1 * need.max(), wsb
    b, a = np.polyfit(ns, need, 1)
    assert np.abs(need - (a + b * ns)).max() <= 0.05 * need.max(), need
    q = np.polyfit(ns, need, 2)
    assert q[0] * ns.max() ** 2 <= 0.02 * need.max(), q  # no quadratic growth (a concave bend is the capped workspace)
