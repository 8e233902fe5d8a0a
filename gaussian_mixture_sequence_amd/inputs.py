"""Seeded synthetic inputs for GMA, shared by the oracle tests, the GPU tests and the
benchmark.  This module holds none of the method's arithmetic: it draws random
tensors and applies the parameter reparameterisation the workloads are specified
with (Sec. 3.6 Eq. 14: sigma2 = softplus(omega) + eps_sigma; Eq. 15: pi = softmax(alpha)),
so that sigma2 > 0 and pi lies on the simplex.

Draw order for one input set (one ``torch.Generator`` seeded once):
  1. mu     = randn(H, K, d_r) * mu_std
  2. omega  = randn(H, K, d_r);  sigma2 = softplus(omega) + 1e-3
  3. alpha  = randn(H, K);       pi = softmax(alpha) per head
  4. XQ = randn(B, H, N, d_r)
  5. XK = randn(B, H, N, d_r)      (N_k = n_ctx rows instead of N for cross-attention)
  6. V  = randn(B, H, N, d_v)      (likewise)
Parameters stay fp32; XQ, XK, V are rounded to the I/O dtype (round-to-nearest-even
for bf16).  Every tensor is contiguous and on the CPU.
"""
from __future__ import annotations

import dataclasses
from typing import Dict

import torch

EPS_SIGMA = 1e-3


@dataclasses.dataclass(frozen=True)
class Workload:
    """One GMA workload: shapes, variant, dtype and the generator recipe."""
    name: str
    causal: bool
    B: int
    H: int
    N: int
    d_r: int
    d_v: int
    K: int
    dtype: str          # "f32" or "bf16": dtype of XQ, XK, V and O
    eps: float = 1e-6
    mu_std: float = 1.0
    seed: int = 0
    chunk: int = 64     # causal chunk length (ignored by the bidirectional variant)
    n_ctx: int = -1     # cross-attention: context length N_k of XK and V (N is then N_q); -1: self
    decode: bool = False  # causal decoding: one position per call, carrying the memory between calls
    diagnostics: bool = False  # responsibility diagnostics of X_Q (Sec. 5.4); V and X_K unused
    backward: bool = False  # backward pass of the bidirectional forward for a seeded upstream gradient dO
    responsibilities: bool = False  # Gamma of X_Q alone (Eq. 3), written out in the I/O dtype; V, X_K unused

    @property
    def tokens(self) -> int:
        return self.B * self.N

    @property
    def head_rows(self) -> int:
        return self.B * self.H * self.N

    @property
    def cross(self) -> bool:
        return self.n_ctx >= 0

    @property
    def n_keys(self) -> int:
        return self.n_ctx if self.cross else self.N

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the implementation is specified against.  Seeds: the first
# workload states seed 0; the others state none, so 1..4 are used.
WORKLOADS: Dict[str, Workload] = {
    "bidir_small_f32": Workload("bidir_small_f32", False, 1, 1, 256, 16, 32, 8, "f32", seed=0),
    "bidir_b8h8_n4096": Workload("bidir_b8h8_n4096", False, 8, 8, 4096, 64, 64, 64, "bf16", seed=1),
    "causal_b8h12_n2048": Workload("causal_b8h12_n2048", True, 8, 12, 2048, 64, 64, 32, "bf16", seed=2),
    "bidir_long_n65536": Workload("bidir_long_n65536", False, 4, 4, 65536, 32, 64, 128, "bf16",
                                  mu_std=1.5, seed=3),
    "causal_long_n32768": Workload("causal_long_n32768", True, 2, 16, 32768, 64, 128, 256, "bf16",
                                   seed=4),
    # cross-attention (no workload is given for it): the B=8, H=8 bidirectional dims with
    # 4096 queries reading a context four times as long
    # single-token causal decoding with a carried memory: the B=8, H=12 causal dims, one
    # position of each sequence per call (N positions are drawn and cycled through)
    "decode_b8h12_k32": Workload("decode_b8h12_k32", True, 8, 12, 64, 64, 64, 32, "bf16", seed=6, decode=True),
    # responsibility diagnostics in the paper's setting: 64 sequences of 1024 positions, 8 heads,
    # K = 128, routing dim d_model / H = 64 (d_v unused)
    "diag_s64_h8_l1024_k128": Workload("diag_s64_h8_l1024_k128", False, 64, 8, 1024, 64, 32, 128, "bf16", seed=7,
                                       diagnostics=True),
    # backward of the bidirectional forward (Sec. 4.1), fp32: the B=8, H=8, N=4096 bidirectional dims
    "bwd_b8h8_n4096_f32": Workload("bwd_b8h8_n4096_f32", False, 8, 8, 4096, 64, 64, 64, "f32", seed=8,
                                   backward=True),
    # backward of the causal forward, fp32: the B=8, H=12, N=2048 causal dims
    "bwdc_b8h12_n2048_f32": Workload("bwdc_b8h12_n2048_f32", True, 8, 12, 2048, 64, 64, 32, "f32", seed=9,
                                     backward=True),
    # the bidirectional backward at the component counts of the paper's language models (K = 128 and
    # 256; Sec. 5, experimental setup, and Sec. 5.3) beside K = 64: B=8, H=8, N=1024, d_r=d_v=64, fp32
    "bwd_b8h8_n1024_k64_f32": Workload("bwd_b8h8_n1024_k64_f32", False, 8, 8, 1024, 64, 64, 64, "f32", seed=10,
                                       backward=True),
    "bwd_b8h8_n1024_k128_f32": Workload("bwd_b8h8_n1024_k128_f32", False, 8, 8, 1024, 64, 64, 128, "f32", seed=11,
                                        backward=True),
    "bwd_b8h8_n1024_k256_f32": Workload("bwd_b8h8_n1024_k256_f32", False, 8, 8, 1024, 64, 64, 256, "f32", seed=12,
                                        backward=True),
    # the causal backward at the same dims and component counts
    "bwdc_b8h8_n1024_k64_f32": Workload("bwdc_b8h8_n1024_k64_f32", True, 8, 8, 1024, 64, 64, 64, "f32", seed=13,
                                        backward=True),
    "bwdc_b8h8_n1024_k128_f32": Workload("bwdc_b8h8_n1024_k128_f32", True, 8, 8, 1024, 64, 64, 128, "f32",
                                         seed=14, backward=True),
    "bwdc_b8h8_n1024_k256_f32": Workload("bwdc_b8h8_n1024_k256_f32", True, 8, 8, 1024, 64, 64, 256, "f32",
                                         seed=15, backward=True),
    "cross_b8h8_q4096_k16384": Workload("cross_b8h8_q4096_k16384", False, 8, 8, 4096, 64, 64, 64, "bf16",
                                        seed=5, n_ctx=16384),
    # the responsibilities alone (gma_responsibilities) at the B=8, H=8, N=4096, d_r=64, K=64
    # bidirectional dims, bf16 routing vectors in and bf16 Gamma out
    "resp_b8h8_n4096": Workload("resp_b8h8_n4096", False, 8, 8, 4096, 64, 64, 64, "bf16", seed=16,
                                responsibilities=True),
}
WORKLOAD_ORDER = ["bidir_small_f32", "bidir_b8h8_n4096", "causal_b8h12_n2048",
                  "bidir_long_n65536", "causal_long_n32768"]


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def make_params(H: int, K: int, d_r: int, mu_std: float, gen: torch.Generator):
    """mu [H,K,d_r], sigma2 [H,K,d_r], pi [H,K], fp32, drawn in the documented order."""
    mu = torch.randn(H, K, d_r, generator=gen, dtype=torch.float32) * mu_std
    omega = torch.randn(H, K, d_r, generator=gen, dtype=torch.float32)
    sigma2 = torch.nn.functional.softplus(omega) + EPS_SIGMA
    alpha = torch.randn(H, K, generator=gen, dtype=torch.float32)
    pi = torch.softmax(alpha, dim=-1)
    return mu.contiguous(), sigma2.contiguous(), pi.contiguous()


def make_inputs(w: Workload, seed: int | None = None) -> Dict[str, torch.Tensor]:
    """All tensors of one input set for workload ``w`` (seed defaults to ``w.seed``)."""
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    mu, sigma2, pi = make_params(w.H, w.K, w.d_r, w.mu_std, gen)
    dt = torch_dtype(w.dtype)
    xq = torch.randn(w.B, w.H, w.N, w.d_r, generator=gen, dtype=torch.float32).to(dt)
    nk = w.n_keys  # the context length for cross-attention
    xk = torch.randn(w.B, w.H, nk, w.d_r, generator=gen, dtype=torch.float32).to(dt)
    v = torch.randn(w.B, w.H, nk, w.d_v, generator=gen, dtype=torch.float32).to(dt)
    out = {"xq": xq.contiguous(), "xk": xk.contiguous(), "v": v.contiguous(), "mu": mu, "sigma2": sigma2, "pi": pi}
    if w.backward:  # the loss gradient at O, drawn last so the forward inputs match the forward's
        out["d_o"] = torch.randn(w.B, w.H, w.N, w.d_v, generator=gen, dtype=torch.float32).to(dt).contiguous()
    return out


def head_slice(inp: Dict[str, torch.Tensor], b: int, h: int) -> Dict[str, torch.Tensor]:
    """The inputs of one (batch, head) pair as a B=1, H=1 problem."""
    return {"xq": inp["xq"][b:b + 1, h:h + 1].contiguous(),
            "xk": inp["xk"][b:b + 1, h:h + 1].contiguous(),
            "v": inp["v"][b:b + 1, h:h + 1].contiguous(),
            "mu": inp["mu"][h:h + 1].contiguous(),
            "sigma2": inp["sigma2"][h:h + 1].contiguous(),
            "pi": inp["pi"][h:h + 1].contiguous()}
