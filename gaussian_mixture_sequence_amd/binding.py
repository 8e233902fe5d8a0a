"""ctypes binding of ``libgma.so`` (C ABI in ``include/gma.h``).

Argument marshalling only: tensors are passed to the library as raw device pointers
together with their sizes, and every step of the computation runs in the library's
HIP kernels.  The functions carry the ABI's names.  If ``libgma.so`` has not been
built, loading fails with an error; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgma.so")

GMA_OK = 0
STATUS_NAMES = ["GMA_OK", "GMA_ERR_NULL_POINTER", "GMA_ERR_BAD_SHAPE", "GMA_ERR_BAD_VALUE",
                "GMA_ERR_UNSUPPORTED", "GMA_ERR_MISALIGNED", "GMA_ERR_WORKSPACE_TOO_SMALL",
                "GMA_ERR_HIP", "GMA_ERR_TIMEOUT"]
GMA_ERR_TIMEOUT = 8
GMA_F32, GMA_BF16 = 0, 1
GMA_OP_RESPONSIBILITIES, GMA_OP_BIDIR, GMA_OP_CAUSAL, GMA_OP_DIAGNOSTICS = 0, 1, 2, 3
GMA_OP_BACKWARD_BIDIR, GMA_OP_BACKWARD_CAUSAL = 4, 5
EXPORTED = ["gma_status_string", "gma_workspace_size", "gma_responsibilities", "gma_forward_bidir",
            "gma_forward_causal", "gma_forward_causal_state", "gma_cross_workspace_size", "gma_forward_cross", "gma_responsibility_diagnostics", "gma_backward_bidir",
            "gma_backward_causal", "gma_backward_causal_state", "gma_backward_cross_workspace_size", "gma_backward_cross", "gma_profiling",
            "gma_profiling_collect", "gma_set_wait_limit", "gma_device_status", "gma_set_single_launch",
            "gma_plan_info", "gma_forward_bidir_noalloc"]
STATIC_SCRATCH_BYTES = 32 << 20  # GMA_STATIC_SCRATCH_BYTES
WAIT_LIMIT_DEFAULT = 1 << 18  # GMA_WAIT_LIMIT_DEFAULT


class GmaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__("%s returned %s" % (where, name))


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d_r", ctypes.c_int64), ("d_v", ctypes.c_int64), ("K", ctypes.c_int64)]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("splits", "rows_per_split", "workgroups", "threads_per_workgroup",
                                              "lds_bytes", "waits_on_all_splits", "resident_bound", "chunk_used")]


class CrossShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N_q", ctypes.c_int64), ("N_k", ctypes.c_int64),
                ("d_r", ctypes.c_int64), ("d_v", ctypes.c_int64), ("K", ctypes.c_int64)]


_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Load libgma.so from the package directory (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libgma.so not found at %s; build it with "
                                   "`python -m gaussian_mixture_sequence_amd.build`" % LIB_PATH)
            lib = ctypes.CDLL(LIB_PATH)
            vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
            shp = ctypes.POINTER(Shape)
            lib.gma_status_string.argtypes = [i32]
            lib.gma_status_string.restype = ctypes.c_char_p
            lib.gma_workspace_size.argtypes = [i32, shp, i32, i32, ctypes.POINTER(sz)]
            lib.gma_workspace_size.restype = i32
            lib.gma_responsibilities.argtypes = [vp, i32, vp, vp, vp, vp, i32, shp, vp, sz, vp]
            lib.gma_responsibilities.restype = i32
            lib.gma_forward_bidir.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, vp, shp, vp, sz, vp]
            lib.gma_forward_bidir.restype = i32
            lib.gma_forward_causal.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, vp, shp, i32, vp, sz, vp]
            lib.gma_forward_causal.restype = i32
            lib.gma_forward_causal_state.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, vp, shp, i32, vp, vp, vp, sz,
                                                     vp]
            lib.gma_forward_causal_state.restype = i32
            lib.gma_responsibility_diagnostics.argtypes = [vp, i32, vp, vp, vp, shp, vp, vp, vp, vp, vp, sz, vp]
            lib.gma_responsibility_diagnostics.restype = i32
            xshp = ctypes.POINTER(CrossShape)
            lib.gma_cross_workspace_size.argtypes = [xshp, i32, ctypes.POINTER(sz)]
            lib.gma_cross_workspace_size.restype = i32
            lib.gma_forward_cross.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, vp, xshp, vp, sz, vp]
            lib.gma_forward_cross.restype = i32
            lib.gma_backward_bidir.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, shp, vp,
                                               sz, vp]
            lib.gma_backward_bidir.restype = i32
            lib.gma_backward_causal.argtypes = lib.gma_backward_bidir.argtypes
            lib.gma_backward_causal.restype = i32
            lib.gma_backward_causal_state.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp,
                                                      vp, vp, vp, shp, vp, sz, vp]
            lib.gma_backward_causal_state.restype = i32
            lib.gma_backward_cross_workspace_size.argtypes = [xshp, i32, ctypes.POINTER(sz)]
            lib.gma_backward_cross_workspace_size.restype = i32
            lib.gma_backward_cross.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, xshp,
                                               vp, sz, vp]
            lib.gma_backward_cross.restype = i32
            lib.gma_profiling.argtypes = [ctypes.c_int]
            lib.gma_profiling.restype = i32
            lib.gma_profiling_collect.argtypes = [ctypes.POINTER(KernelStat), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
            lib.gma_profiling_collect.restype = i32
            lib.gma_set_wait_limit.argtypes = [ctypes.c_uint32]
            lib.gma_set_wait_limit.restype = i32
            lib.gma_device_status.argtypes = [vp]
            lib.gma_device_status.restype = i32
            lib.gma_set_single_launch.argtypes = [ctypes.c_int]
            lib.gma_set_single_launch.restype = i32
            lib.gma_plan_info.argtypes = [i32, shp, i32, i32, ctypes.POINTER(PlanInfo)]
            lib.gma_plan_info.restype = i32
            lib.gma_forward_bidir_noalloc.argtypes = [vp, vp, vp, i32, vp, vp, vp, f32, vp, shp, vp]
            lib.gma_forward_bidir_noalloc.restype = i32
            _lib = lib
    return _lib


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return GMA_F32
    if t == torch.bfloat16:
        return GMA_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(status: int, where: str) -> None:
    if status != GMA_OK:
        raise GmaError(status, where)


def gma_status_string(status: int) -> str:
    return load().gma_status_string(status).decode()


def gma_workspace_size(op: int, B: int, H: int, N: int, d_r: int, d_v: int, K: int,
                       io_dtype: int, chunk: int = 64) -> int:
    out = ctypes.c_size_t(0)
    _check(load().gma_workspace_size(op, ctypes.byref(Shape(B, H, N, d_r, d_v, K)), io_dtype, chunk,
                                     ctypes.byref(out)), "gma_workspace_size")
    return int(out.value)


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise GmaError(6, "workspace")
    return workspace


def gma_responsibilities(x: torch.Tensor, mu: torch.Tensor, sigma2: torch.Tensor, pi: torch.Tensor,
                         gamma_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Gamma [B,H,N,K] of routing vectors x [B,H,N,d_r] (Eq. 3 / 3b)."""
    B, H, N, dr = x.shape
    K = mu.shape[1]
    io = _dtype_code(x.dtype)
    if out is None:
        out = torch.empty(B, H, N, K, dtype=gamma_dtype, device=x.device)
    ws = _workspace(gma_workspace_size(GMA_OP_RESPONSIBILITIES, B, H, N, dr, 1, K, io), x.device, workspace)
    _check(load().gma_responsibilities(_ptr(x), io, _ptr(mu), _ptr(sigma2), _ptr(pi), _ptr(out),
                                       _dtype_code(out.dtype), ctypes.byref(Shape(B, H, N, dr, 1, K)),
                                       _ptr(ws), ws.numel(), _stream(stream)), "gma_responsibilities")
    return out


def gma_forward_bidir(xq: torch.Tensor, xk: torch.Tensor, v: torch.Tensor, mu: torch.Tensor,
                      sigma2: torch.Tensor, pi: torch.Tensor, eps: float = 1e-6,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Bidirectional GMA O [B,H,N,d_v] (Eq. 5-8)."""
    B, H, N, dr = xq.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    io = _dtype_code(xq.dtype)
    if out is None:
        out = torch.empty(B, H, N, dv, dtype=xq.dtype, device=xq.device)
    ws = _workspace(gma_workspace_size(GMA_OP_BIDIR, B, H, N, dr, dv, K, io), xq.device, workspace)
    _check(load().gma_forward_bidir(_ptr(xq), _ptr(xk), _ptr(v), io, _ptr(mu), _ptr(sigma2), _ptr(pi),
                                    float(eps), _ptr(out), ctypes.byref(Shape(B, H, N, dr, dv, K)),
                                    _ptr(ws), ws.numel(), _stream(stream)), "gma_forward_bidir")
    return out


def gma_forward_causal(xq: torch.Tensor, xk: torch.Tensor, v: torch.Tensor, mu: torch.Tensor,
                       sigma2: torch.Tensor, pi: torch.Tensor, eps: float = 1e-6, chunk: int = 64,
                       out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Causal GMA O [B,H,N,d_v] (Eq. 6b/8b), chunked scan with `chunk` positions per chunk."""
    B, H, N, dr = xq.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    io = _dtype_code(xq.dtype)
    if out is None:
        out = torch.empty(B, H, N, dv, dtype=xq.dtype, device=xq.device)
    ws = _workspace(gma_workspace_size(GMA_OP_CAUSAL, B, H, N, dr, dv, K, io, chunk), xq.device, workspace)
    _check(load().gma_forward_causal(_ptr(xq), _ptr(xk), _ptr(v), io, _ptr(mu), _ptr(sigma2), _ptr(pi),
                                     float(eps), _ptr(out), ctypes.byref(Shape(B, H, N, dr, dv, K)),
                                     int(chunk), _ptr(ws), ws.numel(), _stream(stream)),
           "gma_forward_causal")
    return out


def gma_forward_causal_state(xq: torch.Tensor, xk: torch.Tensor, v: torch.Tensor, mu: torch.Tensor,
                             sigma2: torch.Tensor, pi: torch.Tensor, eps: float = 1e-6, chunk: int = 64,
                             state_in: Optional[torch.Tensor] = None, state_out: Optional[torch.Tensor] = None,
                             out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                             stream=None):
    """Causal GMA continued from a carried memory (Eq. 6b as a recurrence).  state_in, state_out:
    [B,H,K,d_v+1] float32 (row k: Vt_k then Z_k); state_in None is an empty memory, state_out is
    allocated when None.  Returns (O [B,H,N,d_v], state_out)."""
    B, H, N, dr = xq.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    io = _dtype_code(xq.dtype)
    if out is None:
        out = torch.empty(B, H, N, dv, dtype=xq.dtype, device=xq.device)
    if state_out is None:
        state_out = torch.empty(B, H, K, dv + 1, dtype=torch.float32, device=xq.device)
    for s in (state_in, state_out):
        if s is not None and (s.dtype != torch.float32 or tuple(s.shape) != (B, H, K, dv + 1)):
            raise ValueError("states must be float32 [B,H,K,d_v+1]")
    ws = _workspace(gma_workspace_size(GMA_OP_CAUSAL, B, H, N, dr, dv, K, io, chunk), xq.device, workspace)
    _check(load().gma_forward_causal_state(_ptr(xq), _ptr(xk), _ptr(v), io, _ptr(mu), _ptr(sigma2), _ptr(pi),
                                           float(eps), _ptr(out), ctypes.byref(Shape(B, H, N, dr, dv, K)),
                                           int(chunk), _ptr(state_in), _ptr(state_out), _ptr(ws), ws.numel(),
                                           _stream(stream)), "gma_forward_causal_state")
    return out, state_out


def gma_responsibility_diagnostics(x: torch.Tensor, mu: torch.Tensor, sigma2: torch.Tensor, pi: torch.Tensor,
                                   want_argmax: bool = True, want_gbar: bool = False,
                                   workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Sec. 5.4 diagnostics of routing vectors x [B,H,N,d_r]: usage [K], H_usage, H_token, R_max
    (Eq. 25-28, as 0-dim tensors), argmax [B,N] int32 (Eq. 29) and gbar [B,N,K] (Eq. 24) if asked."""
    B, H, N, dr = x.shape
    K = mu.shape[1]
    io = _dtype_code(x.dtype)
    dev = x.device
    usage = torch.empty(K, dtype=torch.float32, device=dev)
    stats = torch.empty(4, dtype=torch.float32, device=dev)  # 3 used; 16 bytes keeps the alignment rule
    z = torch.empty(B, N, dtype=torch.int32, device=dev) if want_argmax else None
    gbar = torch.empty(B, N, K, dtype=torch.float32, device=dev) if want_gbar else None
    ws = _workspace(gma_workspace_size(GMA_OP_DIAGNOSTICS, B, H, N, dr, 0, K, io), dev, workspace)
    _check(load().gma_responsibility_diagnostics(_ptr(x), io, _ptr(mu), _ptr(sigma2), _ptr(pi),
                                                 ctypes.byref(Shape(B, H, N, dr, 0, K)), _ptr(usage), _ptr(stats),
                                                 _ptr(z), _ptr(gbar), _ptr(ws), ws.numel(), _stream(stream)),
           "gma_responsibility_diagnostics")
    return {"usage": usage, "h_usage": stats[0], "h_token": stats[1], "r_max": stats[2], "argmax": z, "gbar": gbar}


def gma_backward_bidir(xq: torch.Tensor, xk: torch.Tensor, v: torch.Tensor, mu: torch.Tensor,
                       sigma2: torch.Tensor, pi: torch.Tensor, d_o: torch.Tensor, eps: float = 1e-6,
                       out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of <d_o, O> for the bidirectional forward O (Sec. 4.1, Eq. 17-20), fp32:
    dXQ, dXK [B,H,N,d_r], dV [B,H,N,d_v], dmu, dsigma2 [H,K,d_r], dpi [H,K] (into `out` when given,
    a dict with those keys)."""
    return _backward(GMA_OP_BACKWARD_BIDIR, "gma_backward_bidir", xq, xk, v, mu, sigma2, pi, d_o, eps, out,
                     workspace, stream)


def gma_backward_causal(xq: torch.Tensor, xk: torch.Tensor, v: torch.Tensor, mu: torch.Tensor,
                        sigma2: torch.Tensor, pi: torch.Tensor, d_o: torch.Tensor, eps: float = 1e-6,
                        out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of <d_o, O> for the causal forward O (Sec. 3.5 Eq. 6b, 8b; Sec. 4.1), fp32; outputs
    as gma_backward_bidir."""
    return _backward(GMA_OP_BACKWARD_CAUSAL, "gma_backward_causal", xq, xk, v, mu, sigma2, pi, d_o, eps, out,
                     workspace, stream)


def gma_backward_causal_state(xq: torch.Tensor, xk: torch.Tensor, v: torch.Tensor, mu: torch.Tensor,
                              sigma2: torch.Tensor, pi: torch.Tensor, d_o: torch.Tensor, eps: float = 1e-6,
                              state_in: Optional[torch.Tensor] = None, dstate_out: Optional[torch.Tensor] = None,
                              out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None,
                              stream=None) -> dict:
    """Gradients of <d_o, O> + <dstate_out, state_out> for a causal call continued from the carried
    memory state_in [B,H,K,d_v+1] (Sec. 3.5 Eq. 6b as a recurrence); outputs as gma_backward_causal
    plus dstate_in [B,H,K,d_v+1], the gradient of state_in."""
    B, H, N, dr = xq.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    io = _dtype_code(xq.dtype)
    if out is None:
        out = {"dXQ": torch.empty_like(xq), "dXK": torch.empty_like(xk), "dV": torch.empty_like(v),
               "dmu": torch.empty_like(mu), "dsigma2": torch.empty_like(sigma2), "dpi": torch.empty_like(pi),
               "dstate_in": torch.empty(B, H, K, dv + 1, dtype=torch.float32, device=xq.device)}
    ws = _workspace(gma_workspace_size(GMA_OP_BACKWARD_CAUSAL, B, H, N, dr, dv, K, io), xq.device, workspace)
    _check(load().gma_backward_causal_state(_ptr(xq), _ptr(xk), _ptr(v), io, _ptr(mu), _ptr(sigma2), _ptr(pi),
                                            float(eps), _ptr(d_o), _ptr(state_in), _ptr(dstate_out),
                                            _ptr(out["dXQ"]), _ptr(out["dXK"]), _ptr(out["dV"]), _ptr(out["dmu"]),
                                            _ptr(out["dsigma2"]), _ptr(out["dpi"]), _ptr(out["dstate_in"]),
                                            ctypes.byref(Shape(B, H, N, dr, dv, K)), _ptr(ws), ws.numel(),
                                            _stream(stream)), "gma_backward_causal_state")
    return out


def gma_backward_cross_workspace_size(B: int, H: int, N_q: int, N_k: int, d_r: int, d_v: int, K: int,
                                      io_dtype: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().gma_backward_cross_workspace_size(ctypes.byref(CrossShape(B, H, N_q, N_k, d_r, d_v, K)), io_dtype,
                                                    ctypes.byref(out)), "gma_backward_cross_workspace_size")
    return int(out.value)


def gma_backward_cross(xq: torch.Tensor, xk: torch.Tensor, v: torch.Tensor, mu: torch.Tensor,
                       sigma2: torch.Tensor, pi: torch.Tensor, d_o: torch.Tensor, eps: float = 1e-6,
                       out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of <d_o, O> for the cross-attention forward O (queries xq [B,H,N_q,d_r], context
    xk [B,H,N_k,d_r], v [B,H,N_k,d_v]; Sec. 3, Sec. 4.1); outputs as gma_backward_bidir."""
    B, H, Nq, dr = xq.shape
    Nk, dv = xk.shape[2], v.shape[-1]
    K = mu.shape[1]
    io = _dtype_code(xq.dtype)
    if out is None:
        out = {"dXQ": torch.empty_like(xq), "dXK": torch.empty_like(xk), "dV": torch.empty_like(v),
               "dmu": torch.empty_like(mu), "dsigma2": torch.empty_like(sigma2), "dpi": torch.empty_like(pi)}
    ws = _workspace(gma_backward_cross_workspace_size(B, H, Nq, Nk, dr, dv, K, io), xq.device, workspace)
    _check(load().gma_backward_cross(_ptr(xq), _ptr(xk), _ptr(v), io, _ptr(mu), _ptr(sigma2), _ptr(pi), float(eps),
                                     _ptr(d_o), _ptr(out["dXQ"]), _ptr(out["dXK"]), _ptr(out["dV"]), _ptr(out["dmu"]),
                                     _ptr(out["dsigma2"]), _ptr(out["dpi"]),
                                     ctypes.byref(CrossShape(B, H, Nq, Nk, dr, dv, K)), _ptr(ws), ws.numel(),
                                     _stream(stream)), "gma_backward_cross")
    return out


def _backward(op, name, xq, xk, v, mu, sigma2, pi, d_o, eps, out, workspace, stream) -> dict:
    B, H, N, dr = xq.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    io = _dtype_code(xq.dtype)
    if out is None:
        out = {"dXQ": torch.empty_like(xq), "dXK": torch.empty_like(xk), "dV": torch.empty_like(v),
               "dmu": torch.empty_like(mu), "dsigma2": torch.empty_like(sigma2), "dpi": torch.empty_like(pi)}
    ws = _workspace(gma_workspace_size(op, B, H, N, dr, dv, K, io), xq.device, workspace)
    _check(getattr(load(), name)(_ptr(xq), _ptr(xk), _ptr(v), io, _ptr(mu), _ptr(sigma2), _ptr(pi),
                                 float(eps), _ptr(d_o), _ptr(out["dXQ"]), _ptr(out["dXK"]), _ptr(out["dV"]),
                                 _ptr(out["dmu"]), _ptr(out["dsigma2"]), _ptr(out["dpi"]),
                                 ctypes.byref(Shape(B, H, N, dr, dv, K)), _ptr(ws), ws.numel(), _stream(stream)),
           name)
    return out


def gma_cross_workspace_size(B: int, H: int, N_q: int, N_k: int, d_r: int, d_v: int, K: int, io_dtype: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().gma_cross_workspace_size(ctypes.byref(CrossShape(B, H, N_q, N_k, d_r, d_v, K)), io_dtype,
                                           ctypes.byref(out)), "gma_cross_workspace_size")
    return int(out.value)


def gma_forward_cross(xq: torch.Tensor, xk: torch.Tensor, v: torch.Tensor, mu: torch.Tensor,
                      sigma2: torch.Tensor, pi: torch.Tensor, eps: float = 1e-6,
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Cross-attention GMA O [B,H,N_q,d_v]: queries xq [B,H,N_q,d_r] read the memory written by
    the context xk [B,H,N_k,d_r], v [B,H,N_k,d_v] (Sec. 3, Eq. 5-8)."""
    B, H, Nq, dr = xq.shape
    Nk, dv = xk.shape[2], v.shape[-1]
    K = mu.shape[1]
    io = _dtype_code(xq.dtype)
    if out is None:
        out = torch.empty(B, H, Nq, dv, dtype=xq.dtype, device=xq.device)
    shape = CrossShape(B, H, Nq, Nk, dr, dv, K)
    ws = _workspace(gma_cross_workspace_size(B, H, Nq, Nk, dr, dv, K, io), xq.device, workspace)
    _check(load().gma_forward_cross(_ptr(xq), _ptr(xk), _ptr(v), io, _ptr(mu), _ptr(sigma2), _ptr(pi),
                                    float(eps), _ptr(out), ctypes.byref(shape), _ptr(ws), ws.numel(),
                                    _stream(stream)), "gma_forward_cross")
    return out


def gma_profiling(enable: bool) -> None:
    """Turn per-kernel hipEvent timing of the library's launches on or off."""
    _check(load().gma_profiling(1 if enable else 0), "gma_profiling")


def gma_profiling_collect(capacity: int = 64):
    """{kernel name: (launches, total milliseconds)} recorded since the last collect."""
    buf = (KernelStat * capacity)()
    n = ctypes.c_int(0)
    _check(load().gma_profiling_collect(buf, capacity, ctypes.byref(n)), "gma_profiling_collect")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n.value, capacity))}


def gma_set_wait_limit(polls: int) -> None:
    """Bound on the hand-off waits of the single-launch bf16 forwards (see gma.h)."""
    _check(load().gma_set_wait_limit(int(polls)), "gma_set_wait_limit")


def gma_device_status(stream=None) -> int:
    """Waits for the stream and returns (and clears) the device's status: GMA_OK, or GMA_ERR_TIMEOUT
    when a single-launch forward's hand-off wait ran out since the last query."""
    st = load().gma_device_status(_stream(stream))
    if st not in (GMA_OK, GMA_ERR_TIMEOUT):
        raise GmaError(st, "gma_device_status")
    return st


def gma_set_single_launch(enable: bool) -> None:
    """Allow (default) or forbid the bf16 forwards' single launches with in-launch hand-offs."""
    _check(load().gma_set_single_launch(1 if enable else 0), "gma_set_single_launch")


def gma_plan_info(op: int, B: int, H: int, N: int, d_r: int, d_v: int, K: int, io_dtype: int, chunk: int = 0) -> dict:
    """The device-independent split of a forward (see gma_plan_info in gma.h) as a dict."""
    info = PlanInfo()
    _check(load().gma_plan_info(op, ctypes.byref(Shape(B, H, N, d_r, d_v, K)), io_dtype, chunk, ctypes.byref(info)),
           "gma_plan_info")
    return {n: getattr(info, n) for n, _ in PlanInfo._fields_}


def gma_forward_bidir_noalloc(xq: torch.Tensor, xk: torch.Tensor, v: torch.Tensor, mu: torch.Tensor,
                              sigma2: torch.Tensor, pi: torch.Tensor, eps: float, out: torch.Tensor,
                              stream=None) -> torch.Tensor:
    """gma_forward_bidir on the library's static scratch: no workspace, and the caller provides `out`
    (so that nothing is allocated)."""
    B, H, N, dr = xq.shape
    dv = v.shape[-1]
    K = mu.shape[1]
    _check(load().gma_forward_bidir_noalloc(_ptr(xq), _ptr(xk), _ptr(v), _dtype_code(xq.dtype), _ptr(mu), _ptr(sigma2),
                                            _ptr(pi), float(eps), _ptr(out), ctypes.byref(Shape(B, H, N, dr, dv, K)),
                                            _stream(stream)), "gma_forward_bidir_noalloc")
    return out
