"""Responsibility diagnostics in numpy fp64, from the oracle's responsibilities.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Gaussian Mixture Attention: Linear-Time Sequence Mixing via Probabilistic Latent Routing",
Sec. 5.4, applied to routing vectors X [B,H,N,d_r] of B sequences of N positions:
* Eq. 24: head-averaged responsibilities gbar[t,k] = (1/H) sum_h gamma[b,h,n,k], one token
  occurrence t = (b, n) per sequence position, T = B N;
* Eq. 25: marginal usage p_k = (1/T) sum_t gbar[t,k];
* Eq. 26: normalised usage entropy H_usage = -sum_k p_k log p_k / log K;
* Eq. 27: normalised mean token entropy H_token = (1/T) sum_t (-sum_k gbar log gbar) / log K;
* Eq. 28: mean maximum responsibility R_max = (1/T) sum_t max_k gbar[t,k];
* Eq. 29: hard assignment z_t = argmax_k gbar[t,k] (the lowest k among equal maxima).
0 log 0 is taken as 0 (its limit).  With K = 1 the normalised entropies are 0 / 0; they are
reported as 0 (a single component carries all the mass, so there is no spread to measure).
"""
from __future__ import annotations

import numpy as np


def from_gamma(G: np.ndarray) -> dict:
    """Diagnostics of responsibilities G [B,H,N,K] (fp64)."""
    G = np.asarray(G, np.float64)
    B, H, N, K = G.shape
    gbar = G.mean(axis=1).reshape(B * N, K)                        # Eq. 24
    T = gbar.shape[0]
    usage = gbar.sum(axis=0) / max(T, 1)                            # Eq. 25
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(usage > 0, usage * np.log(usage), 0.0)
        glogg = np.where(gbar > 0, gbar * np.log(gbar), 0.0)
    logk = np.log(K)
    h_usage = float(-plogp.sum() / logk) if K > 1 else 0.0          # Eq. 26
    h_token = float((-glogg.sum(axis=1)).mean() / logk) if K > 1 and T else 0.0   # Eq. 27
    r_max = float(gbar.max(axis=1).mean()) if T else 0.0            # Eq. 28
    z = gbar.argmax(axis=1).astype(np.int32) if T else np.zeros(0, np.int32)  # Eq. 29 (first maximum)
    return {"gbar": gbar.reshape(B, N, K), "usage": usage, "h_usage": h_usage, "h_token": h_token,
            "r_max": r_max, "argmax": z.reshape(B, N)}


def diagnostics(X, mu, sigma2, pi) -> dict:
    """Diagnostics of routing vectors X [B,H,N,d_r] under the per-head mixtures (Eq. 3 via the
    oracle's responsibilities, then Eq. 24-29)."""
    from . import responsibilities
    return from_gamma(responsibilities(X, mu, sigma2, pi))
