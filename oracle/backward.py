"""Backward pass of the bidirectional forward, in numpy fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Gaussian Mixture Attention: Linear-Time Sequence Mixing via Probabilistic Latent Routing",
Sec. 4.1: the loss gradient reaches the responsibilities (g = dL/dgamma), passes the softmax
Jacobian of Eq. 17 as the responsibility-weighted, mean-centred gradient of Eq. 18,
dL/ds_ik = gamma_ik (g_ik - sum_j gamma_ij g_ij), and reaches every parameter that enters the
score through the chain rule of Eq. 19.  For the score of Eq. 16 with Sigma_k = diag(sigma2_k):
  ds/dmu_kd     = (x_d - mu_kd) / sigma2_kd                                   (Eq. 20)
  ds/dsigma2_kd = ((x_d - mu_kd)^2 / sigma2_kd^2 - 1 / sigma2_kd) / 2
  ds/dpi_k      = 1 / pi_k      (pi as given at the boundary; Eq. 15 lies upstream)
  ds/dx_d       = -(x_d - mu_kd) / sigma2_kd
The upstream gradients g come from Eq. 5-8 (O = N / D, N = Gamma_Q Vt, D = Gamma_Q Z + eps,
Vt = Gamma_K^T V, Z = Gamma_K^T 1): with a_i = dO_i . O_i,
  g^Q_ik = (dO_i . Vt_k - a_i Z_k) / D_i,   dVt_k = sum_i gamma^Q_ik dO_i / D_i,
  dZ_k = -sum_i gamma^Q_ik a_i / D_i,       dV_j = sum_k gamma^K_jk dVt_k,
  g^K_jk = dVt_k . V_j + dZ_k.
"""
from __future__ import annotations

import numpy as np


def _score_grads(x, ds, mu, s2, pi):
    """Contributions of one side's score gradients ds [N,K] to dx [N,d], dmu, dsigma2 [K,d], dpi [K]."""
    diff = x[:, None, :] - mu[None]                 # [N,K,d]
    w = ds[:, :, None] * diff / s2[None]            # ds_ik (x_id - mu_kd) / sigma2_kd
    dx = -w.sum(axis=1)
    dmu = w.sum(axis=0)
    ds2 = (ds[:, :, None] * 0.5 * (diff * diff / (s2 * s2)[None] - 1.0 / s2[None])).sum(axis=0)
    dpi = ds.sum(axis=0) / pi
    return dx, dmu, ds2, dpi


def backward_bidir(XQ, XK, V, mu, sigma2, pi, eps, dO) -> dict:
    """Gradients of <dO, O> for the bidirectional forward O (Sec. 3.3): dXQ, dXK [B,H,N,d_r],
    dV [B,H,N,d_v], dmu, dsigma2 [H,K,d_r], dpi [H,K].  The same formulas give the cross-attention
    backward (Sec. 3, "Cross-attention"): XQ, dO and dXQ then have N_q rows, XK, V, dXK, dV N_k."""
    from . import _f64, responsibilities
    XQ, XK, V, dO = (_f64(t) for t in (XQ, XK, V, dO))
    mu, s2, pi = (_f64(t) for t in (mu, sigma2, pi))
    GQ, GK = responsibilities(XQ, mu, s2, pi), responsibilities(XK, mu, s2, pi)
    B, H, N, dr = XQ.shape
    out = {"dXQ": np.zeros_like(XQ), "dXK": np.zeros_like(XK), "dV": np.zeros_like(V),
           "dmu": np.zeros_like(mu), "dsigma2": np.zeros_like(s2), "dpi": np.zeros_like(pi)}
    for b in range(B):
        for h in range(H):
            gq, gk, v, do = GQ[b, h], GK[b, h], V[b, h], dO[b, h]
            vt, z = gk.T @ v, gk.sum(axis=0)                       # Eq. 5-6
            n_, d_ = gq @ vt, gq @ z + eps                         # Eq. 7-8
            o = n_ / d_[:, None]
            a = (do * o).sum(axis=1)
            g_q = (do @ vt.T - a[:, None] * z[None, :]) / d_[:, None]
            dvt = gq.T @ (do / d_[:, None])
            dz = -(gq.T @ (a / d_))
            out["dV"][b, h] = gk @ dvt
            g_k = v @ dvt.T + dz[None, :]
            for x, g, gam, key in ((XQ[b, h], g_q, gq, "dXQ"), (XK[b, h], g_k, gk, "dXK")):
                ds = gam * (g - (gam * g).sum(axis=1, keepdims=True))   # Eq. 18
                dx, dmu, ds2, dpi = _score_grads(x, ds, mu[h], s2[h], pi[h])
                out[key][b, h] = dx
                out["dmu"][h] += dmu
                out["dsigma2"][h] += ds2
                out["dpi"][h] += dpi
    return out


def backward_causal(XQ, XK, V, mu, sigma2, pi, eps, dO, state_in=None, dstate_out=None) -> dict:
    """Gradients of <dO, O> for the causal forward O (Sec. 3.5, Eq. 6b and 8b): position i reads
    the prefix memory Vt^(i) = sum_{j<=i} gamma^K_j V_j^T, Z^(i) = sum_{j<=i} gamma^K_j.  With
    D_i = gamma^Q_i . Z^(i) + eps and a_i = dO_i . O_i,
      g^Q_ik = (dO_i . Vt^(i)_k - a_i Z^(i)_k) / D_i;
    the memory that position i reads receives gamma^Q_i dO_i^T / D_i and -gamma^Q_i a_i / D_i, and
    key position j enters every memory Vt^(i) with i >= j, so its gradients are suffix sums:
      dVt_j = sum_{i>=j} gamma^Q_i dO_i^T / D_i,  dZ_j = -sum_{i>=j} gamma^Q_i a_i / D_i,
      dV_j = sum_k gamma^K_jk dVt_j[k],            g^K_jk = dVt_j[k] . V_j + dZ_j[k].
    The rest (Eq. 18-20) is as for the bidirectional backward.  Shapes as backward_bidir.

    Continued from a carried memory state_in [B,H,K,d_v+1] (row k: Vt_k then Z_k; the forward of
    forward_causal_state), every memory Vt^(i) includes state_in, and the loss may carry a gradient
    dstate_out on the memory after the last position, which every key position enters with weight
    one: dstate_out is added to every dVt_j, dZ_j.  The result then also holds dstate_in, the
    gradient with respect to state_in: dstate_out plus what every query position sends."""
    from . import _f64, responsibilities
    XQ, XK, V, dO = (_f64(t) for t in (XQ, XK, V, dO))
    mu, s2, pi = (_f64(t) for t in (mu, sigma2, pi))
    GQ, GK = responsibilities(XQ, mu, s2, pi), responsibilities(XK, mu, s2, pi)
    B, H, N, dr = XQ.shape
    out = {"dXQ": np.zeros_like(XQ), "dXK": np.zeros_like(XK), "dV": np.zeros_like(V),
           "dmu": np.zeros_like(mu), "dsigma2": np.zeros_like(s2), "dpi": np.zeros_like(pi)}
    K, dv = mu.shape[1], V.shape[-1]
    carried = state_in is not None or dstate_out is not None
    sin = _f64(state_in) if state_in is not None else np.zeros((B, H, K, dv + 1))
    dso = _f64(dstate_out) if dstate_out is not None else np.zeros((B, H, K, dv + 1))
    if carried:
        out["dstate_in"] = dso.copy()
    for b in range(B):
        for h in range(H):
            gq, gk, v, do = GQ[b, h], GK[b, h], V[b, h], dO[b, h]
            if N == 0:
                continue
            vt = sin[b, h, None, :, :dv] + np.cumsum(gk[:, :, None] * v[:, None, :], axis=0)   # Vt^(i) (Eq. 6b)
            z = sin[b, h, None, :, dv] + np.cumsum(gk, axis=0)                                  # Z^(i), [N,K]
            n_ = np.einsum("ik,ikc->ic", gq, vt)                       # Eq. 8b numerator
            d_ = np.einsum("ik,ik->i", gq, z) + eps
            o = n_ / d_[:, None]
            a = (do * o).sum(axis=1)
            g_q = (np.einsum("ic,ikc->ik", do, vt) - a[:, None] * z) / d_[:, None]
            dvt = np.cumsum((gq[:, :, None] * (do / d_[:, None])[:, None, :])[::-1], axis=0)[::-1]
            dz = -np.cumsum((gq * (a / d_)[:, None])[::-1], axis=0)[::-1]
            dvt = dvt + dso[b, h, None, :, :dv]   # the memory after the call depends on every key
            dz = dz + dso[b, h, None, :, dv]
            if carried:  # what every position sends to the memory it read, plus dstate_out
                out["dstate_in"][b, h, :, :dv] = dvt[0]
                out["dstate_in"][b, h, :, dv] = dz[0]
            out["dV"][b, h] = np.einsum("jk,jkc->jc", gk, dvt)
            g_k = np.einsum("jc,jkc->jk", v, dvt) + dz
            for x, g, gam, key in ((XQ[b, h], g_q, gq, "dXQ"), (XK[b, h], g_k, gk, "dXK")):
                ds = gam * (g - (gam * g).sum(axis=1, keepdims=True))   # Eq. 18
                dx, dmu, ds2, dpi = _score_grads(x, ds, mu[h], s2[h], pi[h])
                out[key][b, h] = dx
                out["dmu"][h] += dmu
                out["dsigma2"][h] += ds2
                out["dpi"][h] += dpi
    return out


def backward_magnitudes(XQ, XK, V, mu, sigma2, pi, eps, dO, causal=False, state_in=None, dstate_out=None) -> dict:
    """Per-entry scale of every gradient of backward_bidir (causal=False) or backward_causal
    (causal=True): the formulas above (Sec. 4.1 Eq. 17-20 through Eq. 5-8, or Eq. 6b/8b) evaluated
    on magnitudes, every input and every intermediate replaced by its absolute value and every
    difference by a sum, e.g. for the query side
      |g^Q|_ik = (|dO_i| . |Vt|_k + |a|_i Z_k) / D_i,  |ds|_ik = gamma_ik (|g|_ik + sum_j gamma_ij |g|_ij),
      |dX|_id = sum_k |ds|_ik |x_id - mu_kd| / sigma2_kd.
    Each entry bounds the sum of the absolute values of the terms that form the gradient entry (so
    it is at least the entry's magnitude); an evaluation whose every operation carries a relative
    error u is off by at most a modest multiple of u times it.  Same keys and shapes as the
    gradients (dstate_in only for a carried memory)."""
    from . import _f64, responsibilities
    XQ, XK, V, dO = (_f64(t) for t in (XQ, XK, V, dO))
    mu, s2, pi = (_f64(t) for t in (mu, sigma2, pi))
    GQ, GK = responsibilities(XQ, mu, s2, pi), responsibilities(XK, mu, s2, pi)
    B, H, N, dr = XQ.shape
    K, dv = mu.shape[1], V.shape[-1]
    out = {"dXQ": np.zeros_like(XQ), "dXK": np.zeros_like(XK), "dV": np.zeros_like(V),
           "dmu": np.zeros_like(mu), "dsigma2": np.zeros_like(s2), "dpi": np.zeros_like(pi)}
    carried = state_in is not None or dstate_out is not None
    sin = np.abs(_f64(state_in)) if state_in is not None else np.zeros((B, H, K, dv + 1))
    dso = np.abs(_f64(dstate_out)) if dstate_out is not None else np.zeros((B, H, K, dv + 1))
    if carried:
        out["dstate_in"] = dso.copy()
    for b in range(B):
        for h in range(H):
            gq, gk, v, do = GQ[b, h], GK[b, h], np.abs(V[b, h]), np.abs(dO[b, h])
            if gq.shape[0] == 0 or gk.shape[0] == 0:
                continue
            if causal:
                vt = sin[b, h, None, :, :dv] + np.cumsum(gk[:, :, None] * v[:, None, :], axis=0)   # [N,K,dv]
                z = sin[b, h, None, :, dv] + np.cumsum(gk, axis=0)                                  # [N,K]
                d_ = np.einsum("ik,ik->i", gq, z) + eps
                o = np.einsum("ik,ikc->ic", gq, vt) / d_[:, None]
                a = (do * o).sum(axis=1)
                g_q = (np.einsum("ic,ikc->ik", do, vt) + a[:, None] * z) / d_[:, None]
                dvt = np.cumsum((gq[:, :, None] * (do / d_[:, None])[:, None, :])[::-1], axis=0)[::-1]
                dz = np.cumsum((gq * (a / d_)[:, None])[::-1], axis=0)[::-1]
                dvt = dvt + dso[b, h, None, :, :dv]
                dz = dz + dso[b, h, None, :, dv]
                if carried:
                    out["dstate_in"][b, h, :, :dv] = dvt[0]
                    out["dstate_in"][b, h, :, dv] = dz[0]
                out["dV"][b, h] = np.einsum("jk,jkc->jc", gk, dvt)
                g_k = np.einsum("jc,jkc->jk", v, dvt) + dz
            else:
                vt, z = gk.T @ v, gk.sum(axis=0)
                d_ = gq @ z + eps
                o = (gq @ vt) / d_[:, None]
                a = (do * o).sum(axis=1)
                g_q = (do @ vt.T + a[:, None] * z[None, :]) / d_[:, None]
                dvt = gq.T @ (do / d_[:, None])
                dz = gq.T @ (a / d_)
                out["dV"][b, h] = gk @ dvt
                g_k = v @ dvt.T + dz[None, :]
            for x, g, gam, key in ((XQ[b, h], g_q, gq, "dXQ"), (XK[b, h], g_k, gk, "dXK")):
                ds = gam * (g + (gam * g).sum(axis=1, keepdims=True))
                diff = np.abs(x[:, None, :] - mu[h][None])                  # [N,K,d]
                w = ds[:, :, None] * diff / s2[h][None]
                out[key][b, h] = w.sum(axis=1)
                out["dmu"][h] += w.sum(axis=0)
                out["dsigma2"][h] += (ds[:, :, None] * 0.5 * (diff * diff / (s2[h] * s2[h])[None]
                                                               + 1.0 / s2[h][None])).sum(axis=0)
                out["dpi"][h] += ds.sum(axis=0) / pi[h]
    return out
