"""Helpers shared by the test modules: error metrics and GPU/oracle runners."""
import numpy as np
import torch

# Tolerances on the row-scaled error below (fp32 I/O and bf16 I/O with fp32 accumulation).
TOL = {"f32": 1e-5, "bf16": 2e-2}


def row_scaled_error(out, ref) -> float:
    """max over (b,h,i,c) of |O - O*| / max_c' |O*_{b,h,i,c'}|.

    Elementwise relative error is ill-posed for GMA outputs (single entries of O can be
    ~1e-7 while the row is O(1)), so each row's error is scaled by the row's largest
    reference magnitude."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    if out.size == 0:
        return 0.0
    scale = np.maximum(np.abs(ref).max(axis=-1, keepdims=True), 1e-30)
    return float((np.abs(out - ref) / scale).max())


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def to_device(inp, device="cuda"):
    return {k: v.to(device) for k, v in inp.items()}
