"""GMA oracle: fp64 CPU reference for the Gaussian Mixture Attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with
the HIP implementation in ``gaussian_mixture_sequence_amd`` and never imports it.

Two independent implementations live here, both written from "Gaussian Mixture
Attention: Linear-Time Sequence Mixing via Probabilistic Latent Routing":

* ``gma_oracle.c`` (loaded through ctypes): the associative form the method uses,
  Sec. 3.3 Eq. 5-8 (bidirectional; with a separate context sequence for keys and
  values, the cross-attention of Sec. 3) and Sec. 3.5 Eq. 6b/8b (causal), with the
  responsibilities of Sec. 3.2 Eq. 3 computed through the log-density scores of
  Sec. 4.1 Eq. 16 and the softmax of Eq. 3b.
* ``brute.py`` (numpy): the explicit N x N affinity forms, Eq. 9-11 and Eq. 9b/10b,
  with responsibilities taken straight from the density ratio of Eq. 2-3.  Only for
  tiny N.

Inputs are converted to float64 exactly (bf16 and fp32 values are representable in
fp64), so a comparison against the GPU measures the GPU's arithmetic, not the
rounding of its inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gma_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ``gma_oracle.c`` with gcc into ``oracle/liboracle.so``."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.oracle_log_scores.argtypes = [dp, i64, i64, i64, i64, dp, dp, dp, i64, dp]
            lib.oracle_responsibilities.argtypes = [dp, i64, i64, i64, i64, dp, dp, dp, i64, dp]
            fwd = [dp, dp, dp, i64, i64, i64, i64, i64, i64, dp, dp, dp, ctypes.c_double, dp]
            lib.oracle_forward_bidir.argtypes = fwd
            lib.oracle_forward_causal.argtypes = fwd
            lib.oracle_forward_causal_state.argtypes = [dp, dp, dp, i64, i64, i64, i64, i64, i64, dp, dp, dp,
                                                        ctypes.c_double, dp, dp, dp]
            lib.oracle_forward_causal_state.restype = ctypes.c_int
            lib.oracle_forward_cross.argtypes = [dp, i64, dp, dp, i64, i64, i64, i64, i64, i64, dp, dp, dp,
                                                 ctypes.c_double, dp]
            for f in (lib.oracle_log_scores, lib.oracle_responsibilities,
                      lib.oracle_forward_bidir, lib.oracle_forward_causal, lib.oracle_forward_cross):
                f.restype = ctypes.c_int
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_num_threads.argtypes = []
            lib.oracle_set_num_threads.restype = None
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    """Exact float64 copy of a numpy array or a CPU torch tensor (bf16 included)."""
    if hasattr(a, "detach"):  # torch tensor: upcast in torch (exact), then hand over
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise RuntimeError("%s failed with code %d" % (name, rc))


def _params(mu, sigma2, pi):
    mu, sigma2, pi = _f64(mu), _f64(sigma2), _f64(pi)
    if mu.ndim != 3 or sigma2.shape != mu.shape or pi.shape != mu.shape[:2]:
        raise ValueError("mu, sigma2 must be [H,K,d_r] and pi [H,K]")
    return mu, sigma2, pi


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's OpenMP loops from now on (n >= 1)."""
    _load().oracle_set_num_threads(int(n))


def log_scores(X, mu, sigma2, pi) -> np.ndarray:
    """Eq. 16 scores s = log pi_k + log N(x | mu_k, Sigma_k) for X [B,H,N,d_r]."""
    X = _f64(X)
    mu, sigma2, pi = _params(mu, sigma2, pi)
    B, H, N, dr = X.shape
    K = mu.shape[1]
    S = np.empty((B, H, N, K), np.float64)
    _check(_load().oracle_log_scores(_ptr(X), B, H, N, dr, _ptr(mu), _ptr(sigma2), _ptr(pi), K, _ptr(S)),
           "oracle_log_scores")
    return S


def responsibilities(X, mu, sigma2, pi) -> np.ndarray:
    """Eq. 3 responsibilities Gamma [B,H,N,K] of routing vectors X [B,H,N,d_r]."""
    X = _f64(X)
    mu, sigma2, pi = _params(mu, sigma2, pi)
    B, H, N, dr = X.shape
    K = mu.shape[1]
    G = np.empty((B, H, N, K), np.float64)
    _check(_load().oracle_responsibilities(_ptr(X), B, H, N, dr, _ptr(mu), _ptr(sigma2), _ptr(pi), K, _ptr(G)),
           "oracle_responsibilities")
    return G


def _forward(fn, XQ, XK, V, mu, sigma2, pi, eps):
    XQ, XK, V = _f64(XQ), _f64(XK), _f64(V)
    mu, sigma2, pi = _params(mu, sigma2, pi)
    B, H, N, dr = XQ.shape
    dv = V.shape[-1]
    K = mu.shape[1]
    if XK.shape != XQ.shape or V.shape[:3] != XQ.shape[:3]:
        raise ValueError("XQ, XK must be [B,H,N,d_r] and V [B,H,N,d_v]")
    O = np.empty((B, H, N, dv), np.float64)
    _check(fn(_ptr(XQ), _ptr(XK), _ptr(V), B, H, N, dr, dv, K, _ptr(mu), _ptr(sigma2), _ptr(pi),
              float(eps), _ptr(O)), fn.__name__)
    return O


def forward_bidir(XQ, XK, V, mu, sigma2, pi, eps) -> np.ndarray:
    """Bidirectional GMA output O [B,H,N,d_v], Sec. 3.3 Eq. 5-8."""
    return _forward(_load().oracle_forward_bidir, XQ, XK, V, mu, sigma2, pi, eps)


def forward_causal(XQ, XK, V, mu, sigma2, pi, eps) -> np.ndarray:
    """Causal GMA output O [B,H,N,d_v], Sec. 3.5 Eq. 6b/8b."""
    return _forward(_load().oracle_forward_causal, XQ, XK, V, mu, sigma2, pi, eps)


def forward_causal_state(XQ, XK, V, mu, sigma2, pi, eps, state_in=None):
    """Causal GMA continued from a carried memory (Sec. 3.5 Eq. 6b as a recurrence).
    state_in [B,H,K,d_v+1] (row k: Vt_k then Z_k) is the memory before position 0, None for
    an empty one.  Returns (O [B,H,N,d_v], state_out [B,H,K,d_v+1]): the outputs and the
    memory after the last position."""
    XQ, XK, V = _f64(XQ), _f64(XK), _f64(V)
    mu, sigma2, pi = _params(mu, sigma2, pi)
    B, H, N, dr = XQ.shape
    dv, K = V.shape[-1], mu.shape[1]
    if XK.shape != XQ.shape or V.shape[:3] != XQ.shape[:3]:
        raise ValueError("XQ, XK must be [B,H,N,d_r] and V [B,H,N,d_v]")
    sin = None
    if state_in is not None:
        sin = _f64(state_in)
        if sin.shape != (B, H, K, dv + 1):
            raise ValueError("state_in must be [B,H,K,d_v+1]")
    O = np.empty((B, H, N, dv), np.float64)
    S = np.empty((B, H, K, dv + 1), np.float64)
    _check(_load().oracle_forward_causal_state(_ptr(XQ), _ptr(XK), _ptr(V), B, H, N, dr, dv, K, _ptr(mu),
                                               _ptr(sigma2), _ptr(pi), float(eps),
                                               _ptr(sin) if sin is not None else None, _ptr(O), _ptr(S)),
           "oracle_forward_causal_state")
    return O, S


def forward_cross(XQ, XK, V, mu, sigma2, pi, eps) -> np.ndarray:
    """Cross-attention GMA output O [B,H,Nq,d_v] (Sec. 3, "Cross-attention"): queries XQ
    [B,H,Nq,d_r] read the latent memory written by a context XK [B,H,Nk,d_r], V [B,H,Nk,d_v]
    through Eq. 5-8."""
    XQ, XK, V = _f64(XQ), _f64(XK), _f64(V)
    mu, sigma2, pi = _params(mu, sigma2, pi)
    B, H, Nq, dr = XQ.shape
    Nk, dv = XK.shape[2], V.shape[-1]
    K = mu.shape[1]
    if XK.shape[:2] != (B, H) or XK.shape[3] != dr or V.shape[:3] != XK.shape[:3]:
        raise ValueError("XQ must be [B,H,Nq,d_r], XK [B,H,Nk,d_r] and V [B,H,Nk,d_v]")
    O = np.empty((B, H, Nq, dv), np.float64)
    _check(_load().oracle_forward_cross(_ptr(XQ), Nq, _ptr(XK), _ptr(V), Nk, B, H, dr, dv, K, _ptr(mu),
                                        _ptr(sigma2), _ptr(pi), float(eps), _ptr(O)), "oracle_forward_cross")
    return O


from . import brute  # noqa: E402  (numpy explicit-affinity forms)
from . import diagnostics  # noqa: E402  (responsibility diagnostics, Sec. 5.4)
from . import backward  # noqa: E402  (backward pass of the bidirectional forward, Sec. 4.1)

__all__ = ["build", "num_threads", "log_scores", "responsibilities", "forward_bidir",
           "forward_causal", "forward_causal_state", "forward_cross", "brute", "diagnostics", "backward"]
