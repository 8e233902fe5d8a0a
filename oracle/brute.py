"""Explicit-affinity GMA in numpy fp64, for tiny N only.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is deliberately the *other* parenthesisation of the method, the one the
method avoids: it materialises the N x N affinity.  Sources, all in "Gaussian
Mixture Attention: Linear-Time Sequence Mixing via Probabilistic Latent Routing":

* density: Sec. 3.2 Eq. 2, evaluated as a full multivariate normal with
  Sigma_k = diag(sigma2_k) through ``numpy.linalg`` (no log-space shortcut);
* responsibilities: Sec. 3.2 Eq. 3, the ratio pi_k N_k / sum_l pi_l N_l;
* unnormalised affinity: Sec. 3.3 Eq. 11, A~ = Gamma_Q Gamma_K^T;
* normalised affinity: Eq. 9 in the matrix form of footnote 4,
  A = diag(A~ 1 + eps)^{-1} A~, and the output Eq. 10, O = A V;
* causal: Sec. 3.5 Eq. 9b/10b, the same with A~_ij kept only for j <= i.

Because Eq. 3 is evaluated as a plain ratio of densities, inputs must keep the
densities inside the fp64 range (moderate |x - mu|^2 / sigma2); the tests that use
this module choose such inputs.
"""
from __future__ import annotations

import numpy as np


def density(x: np.ndarray, mu_k: np.ndarray, s2_k: np.ndarray) -> np.ndarray:
    """Eq. 2: N(x | mu_k, diag(s2_k)) for every row of x [N, d_r]."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    cov = np.diag(np.asarray(s2_k, np.float64))
    diff = x - np.asarray(mu_k, np.float64)[None, :]
    sol = np.linalg.solve(cov, diff.T).T          # Sigma_k^{-1} (x - mu_k)
    maha = np.einsum("nd,nd->n", diff, sol)       # (x - mu_k)^T Sigma_k^{-1} (x - mu_k)
    norm = (2.0 * np.pi) ** (d / 2.0) * np.sqrt(np.linalg.det(cov))
    return np.exp(-0.5 * maha) / norm


def responsibilities(x: np.ndarray, mu: np.ndarray, s2: np.ndarray, pi: np.ndarray) -> np.ndarray:
    """Eq. 3 for one head: Gamma [N, K] from x [N, d_r], mu/s2 [K, d_r], pi [K]."""
    K = mu.shape[0]
    weighted = np.stack([pi[k] * density(x, mu[k], s2[k]) for k in range(K)], axis=1)
    return weighted / weighted.sum(axis=1, keepdims=True)


def affinity(gq: np.ndarray, gk: np.ndarray, causal: bool) -> np.ndarray:
    """Eq. 11 (and the j <= i support of Eq. 9b when causal): A~ [N, N]."""
    a = gq @ gk.T
    if causal:
        a = np.tril(a)
    return a


def forward_one_head(xq, xk, v, mu, s2, pi, eps: float, causal: bool) -> np.ndarray:
    """O [Nq, d_v] for one (batch, head) through the explicit affinity, Eq. 9-10 / 9b-10b.
    Without the causal mask the query and key sequences may differ in length (the
    cross-attention of Sec. 3): A~ is then Nq x Nk."""
    gq = responsibilities(xq, mu, s2, pi)
    gk = responsibilities(xk, mu, s2, pi)
    a_tilde = affinity(gq, gk, causal)
    d = a_tilde.sum(axis=1) + eps                 # footnote 4: d = A~ 1 + eps
    a = a_tilde / d[:, None]                      # diag(d)^{-1} A~
    return a @ np.asarray(v, np.float64)


def forward(XQ, XK, V, mu, sigma2, pi, eps: float, causal: bool) -> np.ndarray:
    """Batched explicit form: XQ, XK [B,H,N,d_r], V [B,H,N,d_v], params per head."""
    XQ, XK, V = (np.asarray(t, np.float64) for t in (XQ, XK, V))
    mu, sigma2, pi = (np.asarray(t, np.float64) for t in (mu, sigma2, pi))
    B, H, N, _ = XQ.shape
    out = np.empty(V.shape, np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = forward_one_head(XQ[b, h], XK[b, h], V[b, h], mu[h], sigma2[h], pi[h],
                                         eps, causal)
    return out


def forward_cross(XQ, XK, V, mu, sigma2, pi, eps: float) -> np.ndarray:
    """Batched explicit cross-attention: XQ [B,H,Nq,d_r], XK [B,H,Nk,d_r], V [B,H,Nk,d_v]."""
    XQ, XK, V = (np.asarray(t, np.float64) for t in (XQ, XK, V))
    mu, sigma2, pi = (np.asarray(t, np.float64) for t in (mu, sigma2, pi))
    B, H, Nq, _ = XQ.shape
    out = np.empty((B, H, Nq, V.shape[-1]), np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = forward_one_head(XQ[b, h], XK[b, h], V[b, h], mu[h], sigma2[h], pi[h], eps, False)
    return out


def forward_causal_state(XQ, XK, V, mu, sigma2, pi, eps: float, state_in):
    """Explicit causal form continued from a carried memory (Vt0, Z0) = state_in [B,H,K,d_v+1]:
    O_i = (gammaQ_i Vt0 + sum_{j<=i} A~_ij V_j) / (gammaQ_i Z0 + sum_{j<=i} A~_ij + eps), with
    A~ the masked affinity of Eq. 9b; the memory after the last position is
    (Vt0 + Gamma_K^T V, Z0 + Gamma_K^T 1).  Returns (O, state_out)."""
    XQ, XK, V, S0 = (np.asarray(t, np.float64) for t in (XQ, XK, V, state_in))
    mu, sigma2, pi = (np.asarray(t, np.float64) for t in (mu, sigma2, pi))
    B, H, N, _ = XQ.shape
    dv = V.shape[-1]
    out = np.empty((B, H, N, dv), np.float64)
    s_out = np.empty(S0.shape, np.float64)
    for b in range(B):
        for h in range(H):
            gq = responsibilities(XQ[b, h], mu[h], sigma2[h], pi[h])
            gk = responsibilities(XK[b, h], mu[h], sigma2[h], pi[h])
            a = affinity(gq, gk, True)
            vt0, z0 = S0[b, h, :, :dv], S0[b, h, :, dv]
            num = gq @ vt0 + a @ V[b, h]
            den = gq @ z0 + a.sum(axis=1) + eps
            out[b, h] = num / den[:, None]
            s_out[b, h, :, :dv] = vt0 + gk.T @ V[b, h]
            s_out[b, h, :, dv] = z0 + gk.sum(axis=0)
    return out, s_out


def affinity_matrix(XQ1, XK1, mu1, s21, pi1, causal: bool = False) -> np.ndarray:
    """Unnormalised affinity A~ of one head, for rank checks (Sec. 4.2 Eq. 23)."""
    gq = responsibilities(XQ1, mu1, s21, pi1)
    gk = responsibilities(XK1, mu1, s21, pi1)
    return affinity(gq, gk, causal)
