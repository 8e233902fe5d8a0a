"""gma_forward_bidir_noalloc: the bidirectional forward on the library's static scratch (for
callers that cannot allocate).  Its output must equal gma_forward_bidir's bit for bit (same
kernels, same plan), including when a second call with a smaller input follows and reuses the
scratch the first one left."""
import ctypes

import numpy as np
import pytest
import torch

from gaussian_mixture_sequence_amd import binding as gb
from gaussian_mixture_sequence_amd.inputs import WORKLOADS, make_inputs
from gma_testutil import to_device, to_np


def test_noalloc_rejects_oversize_before_any_hip_call():
    """A shape whose workspace exceeds the static scratch is refused on the host (fake pointers
    never reach a kernel, so this runs without a GPU)."""
    lib = gb.load()
    fake = 0x10000
    big = gb.Shape(64, 16, 1 << 16, 64, 128, 256)  # ~1 GB of split partials
    nbytes = gb.gma_workspace_size(gb.GMA_OP_BIDIR, 64, 16, 1 << 16, 64, 128, 256, gb.GMA_BF16)
    assert nbytes > gb.STATIC_SCRATCH_BYTES
    st = lib.gma_forward_bidir_noalloc(fake, fake, fake, gb.GMA_BF16, fake, fake, fake, 1e-6, fake,
                                       ctypes.byref(big), None)
    assert st == 6  # GMA_ERR_WORKSPACE_TOO_SMALL
    assert lib.gma_forward_bidir_noalloc(fake, fake, fake, gb.GMA_BF16, fake, fake, fake, 1e-6, fake, None,
                                         None) == 1  # GMA_ERR_NULL_POINTER


@pytest.mark.gpu
@pytest.mark.parametrize("first,second", [
    (WORKLOADS["bidir_b8h8_n4096"], WORKLOADS["bidir_b8h8_n4096"].with_(B=2, H=3, N=1000, seed=81)),
    (WORKLOADS["bidir_long_n65536"].with_(B=2, N=40000, seed=82), WORKLOADS["bidir_long_n65536"].with_(B=1, H=1, N=777, seed=83)),
    (WORKLOADS["bidir_small_f32"].with_(B=4, H=4, N=3000, seed=84), WORKLOADS["bidir_small_f32"].with_(N=100, seed=85)),
], ids=["bf16-b8h8", "bf16-long", "f32"])
def test_noalloc_matches_bidir_on_two_calls(first, second):
    outs = []
    for w in (first, second):
        nbytes = gb.gma_workspace_size(gb.GMA_OP_BIDIR, w.B, w.H, w.N, w.d_r, w.d_v, w.K,
                                       gb.GMA_BF16 if w.dtype == "bf16" else gb.GMA_F32)
        assert nbytes <= gb.STATIC_SCRATCH_BYTES, nbytes
        d = to_device(make_inputs(w))
        ref = gb.gma_forward_bidir(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps)
        out = torch.full_like(ref, float("nan"))
        gb.gma_forward_bidir_noalloc(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps, out)
        torch.cuda.synchronize()
        outs.append((to_np(out), to_np(ref)))
    for got, ref in outs:
        assert np.isfinite(got).all()
        assert np.array_equal(got, ref)
    assert gb.gma_device_status() == gb.GMA_OK
