"""Workload table and seeded synthetic inputs for the GMA forward mixer.

This module holds no arithmetic of the method: it only names the problem
shapes and draws random numbers.  Both the fp64 oracle (test side) and the
HIP path (product side) receive their inputs from here, so the two never share
any code that computes a responsibility, a memory write or a read.

Workloads follow the shapes of the Gaussian Mixture Attention page
("Attention par Mélange Gaussien (GMA)", section "Méthodologie", item 1 for the
routing inputs and item 3 for the two variants; section "Résultats et
Performance" for the K = 256 language-model shape).  The pages evaluate on
Long-Range Arena and WikiText-103; those datasets are not used: i.i.d. normal
inputs of the same shapes stand in for them.

Distributions (one recipe for every workload):
  * routing projections Q_X, K_X and values V ~ N(0, 1), drawn in fp32 and,
    for the bf16 workloads, rounded once to bf16 (round-to-nearest-even);
  * component means mu ~ N(0, 1), shape [H, K, d_r];
  * raw variances rho ~ U(-1, 1), shape [H, K, d_r] (softplus is applied by
    the method, not here);
  * prior logits lambda ~ N(0, 0.5^2), shape [H, K].
Every tensor slice (tensor, b, h) has its own counter-derived seed, so one
head of a long sequence can be drawn without drawing the others.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, Optional

import torch

__all__ = ["Workload", "WORKLOADS", "workload", "make_params", "make_head_inputs", "make_inputs"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    causal: bool
    dtype: str          # "f32" or "bf16": storage type of Q_X, K_X, V and O
    batch: int
    heads: int
    seq_len: int
    d_route: int
    n_comp: int
    d_value: int
    eps: float = 1e-6
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def token_heads(self) -> int:
        return self.batch * self.heads * self.seq_len


# The five workloads, smallest first.  Index i uses seed i.
WORKLOADS = (
    Workload("bidir-f32-B1H1-N256-dr16-K8-dv16", False, "f32", 1, 1, 256, 16, 8, 16, seed=0),
    Workload("causal-f32-B4H8-N4096-dr64-K64-dv64", True, "f32", 4, 8, 4096, 64, 64, 64, seed=1),
    Workload("bidir-bf16-B32H8-N4096-dr64-K32-dv64", False, "bf16", 32, 8, 4096, 64, 32, 64, seed=2),
    Workload("causal-bf16-B1H16-N65536-dr128-K128-dv128", True, "bf16", 1, 16, 65536, 128, 128, 128, seed=3),
    Workload("causal-bf16-B1H8-N1048576-dr64-K256-dv64", True, "bf16", 1, 8, 1048576, 64, 256, 64, seed=4),
)


def workload(i: int, **overrides) -> Workload:
    w = WORKLOADS[i]
    return w.with_(**overrides) if overrides else w


_TENSOR_IDS = {"mu": 1, "raw_var": 2, "prior_logits": 3, "qx": 4, "kx": 5, "v": 6, "dout": 7}


def _generator(seed: int, tensor: str, b: int, h: int) -> torch.Generator:
    # SplitMix64-style mixing of (seed, tensor, b, h) into one 63-bit seed.
    z = (seed * 0x9E3779B97F4A7C15 + _TENSOR_IDS[tensor] * 0xBF58476D1CE4E5B9
         + b * 0x94D049BB133111EB + h * 0x2545F4914F6CDD1D + 0x632BE59BD9B4E019) & (2**64 - 1)
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & (2**64 - 1)
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & (2**64 - 1)
    z ^= z >> 31
    g = torch.Generator(device="cpu")
    g.manual_seed(z & (2**63 - 1))
    return g


def make_params(w: Workload, heads: Optional[Iterable[int]] = None) -> Dict[str, torch.Tensor]:
    """GMM parameters, fp32 on the CPU: mu, raw_var [H', K, d_r] and prior_logits [H', K]."""
    hs = list(range(w.heads)) if heads is None else list(heads)
    mu = torch.stack([torch.randn(w.n_comp, w.d_route, generator=_generator(w.seed, "mu", 0, h))
                      for h in hs])
    rv = torch.stack([torch.rand(w.n_comp, w.d_route, generator=_generator(w.seed, "raw_var", 0, h)) * 2.0 - 1.0
                      for h in hs])
    pl = torch.stack([torch.randn(w.n_comp, generator=_generator(w.seed, "prior_logits", 0, h)) * 0.5
                      for h in hs])
    return {"mu": mu.contiguous(), "raw_var": rv.contiguous(), "prior_logits": pl.contiguous()}


def make_head_inputs(w: Workload, b: int, h: int) -> Dict[str, torch.Tensor]:
    """Q_X [N, d_r], K_X [N, d_r], V [N, d_v] of one (batch, head), in the workload's storage dtype."""
    out = {}
    for name, d in (("qx", w.d_route), ("kx", w.d_route), ("v", w.d_value)):
        x = torch.randn(w.seq_len, d, generator=_generator(w.seed, name, b, h))
        out[name] = x.to(w.torch_dtype)
    return out


def make_inputs(w: Workload, heads: Optional[Iterable[int]] = None) -> Dict[str, torch.Tensor]:
    """All inputs on the CPU: qx, kx [B, H', N, d_r], v [B, H', N, d_v] plus the parameters.

    `heads` selects a subset of heads (default: all); parameters follow the same subset.
    """
    hs = list(range(w.heads)) if heads is None else list(heads)
    out = {
        "qx": torch.empty(w.batch, len(hs), w.seq_len, w.d_route, dtype=w.torch_dtype),
        "kx": torch.empty(w.batch, len(hs), w.seq_len, w.d_route, dtype=w.torch_dtype),
        "v": torch.empty(w.batch, len(hs), w.seq_len, w.d_value, dtype=w.torch_dtype),
    }
    for b in range(w.batch):
        for j, h in enumerate(hs):
            hi = make_head_inputs(w, b, h)
            for k in ("qx", "kx", "v"):
                out[k][b, j].copy_(hi[k])
    out.update(make_params(w, hs))
    return out


def make_dout(w: Workload, heads: Optional[Iterable[int]] = None) -> torch.Tensor:
    """Upstream gradient dL/dO [B, H', N, d_v] for the backward pass: i.i.d. N(0, 1) in the storage dtype."""
    hs = list(range(w.heads)) if heads is None else list(heads)
    out = torch.empty(w.batch, len(hs), w.seq_len, w.d_value, dtype=w.torch_dtype)
    for b in range(w.batch):
        for j, h in enumerate(hs):
            out[b, j].copy_(torch.randn(w.seq_len, w.d_value, generator=_generator(w.seed, "dout", b, h)))
    return out
