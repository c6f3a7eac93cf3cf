"""Seeded synthetic inputs for the gated delta rule core.

This module only draws random tensors: it holds none of the method's arithmetic,
so both the HIP path and the oracle can be fed from it.  Everything is drawn on
the host with ``torch.Generator('cpu')`` so a seed always gives the same bits.

Recipe (the workloads of the gated delta rule pages, made synthetic):
  q, k   ~ N(0, 1) in fp32, then divided by their L2 norm over the key channels
           (real layers feed unit-length queries and keys into the memory step:
           "Attention, Part 4", section 6, "Where alpha and beta come from").
  v      ~ N(0, 1).
  beta   = sigmoid(N(0, 1))  -- a write strength in (0, 1).
  log a  ~ U[-0.2, -0.005]  -- the forget gate stored as its logarithm; per key
           channel for KDA.  alpha = exp(log a) in [0.82, 0.995] brackets the
           ~94 % per-token retention that "Hybrid attention" (section "A test of
           memory") reports for a typical head.
  S0     = std * N(0, 1) in fp32 (zeros when std == 0).
  Then q, k, v, beta, log a are rounded once to the input dtype (round to nearest
  even); the oracle is fed exactly those rounded values.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import torch


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    H: int
    T: int
    Dk: int
    Dv: int
    chunk: int
    dtype: torch.dtype
    s0_std: float
    ckpt_every: int = 0
    kda: bool = False


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    N: int
    H: int
    Dk: int
    Dv: int
    steps: int
    dtype: torch.dtype
    s_std: float
    kda: bool = False


# The five workloads: index = position in the workload list; seed = 1000 + index.
WORKLOADS = {
    0: PrefillConfig("gdn_tiny_fp32", 1, 2, 64, 16, 16, 16, torch.float32, 0.0),
    1: PrefillConfig("gdn_prefill_bf16", 4, 16, 4096, 128, 128, 64, torch.bfloat16, 0.01),
    2: PrefillConfig("gdn_long_prefill_snapshots_bf16", 1, 32, 65536, 128, 128, 64, torch.bfloat16,
                     0.01, ckpt_every=8192),
    3: DecodeConfig("gdn_decode_bf16", 256, 32, 128, 128, 100, torch.bfloat16, 0.02),
    4: PrefillConfig("kda_prefill_bf16", 2, 32, 8192, 128, 128, 64, torch.bfloat16, 0.01, kda=True),
}


def seed_of(index: int) -> int:
    return 1000 + index


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def make_prefill(B: int, H: int, T: int, Dk: int, Dv: int, dtype: torch.dtype = torch.bfloat16,
                 *, kda: bool = False, s0_std: float = 0.01, seed: int = 0,
                 log_alpha_range=(-0.2, -0.005)) -> Dict[str, Optional[torch.Tensor]]:
    """Draw q, k, v, beta, log_alpha, s0 (in that order) on the host."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = _unit(torch.randn(B, H, T, Dk, generator=g))
    k = _unit(torch.randn(B, H, T, Dk, generator=g))
    v = torch.randn(B, H, T, Dv, generator=g)
    beta = torch.sigmoid(torch.randn(B, H, T, generator=g))
    lo, hi = log_alpha_range
    la_shape = (B, H, T, Dk) if kda else (B, H, T)
    log_alpha = torch.rand(*la_shape, generator=g) * (hi - lo) + lo
    s0 = (torch.randn(B, H, Dv, Dk, generator=g) * s0_std) if s0_std > 0 else None
    return {
        "q": q.to(dtype), "k": k.to(dtype), "v": v.to(dtype),
        "beta": beta.to(dtype), "log_alpha": log_alpha.to(dtype), "s0": s0,
    }


def make_decode(N: int, H: int, Dk: int, Dv: int, steps: int, dtype: torch.dtype = torch.bfloat16,
                *, kda: bool = False, s_std: float = 0.02, seed: int = 0,
                log_alpha_range=(-0.2, -0.005)) -> Dict[str, torch.Tensor]:
    """Draw the state first, then every step's q, k, v, beta, log_alpha as [steps, ...] tensors."""
    g = torch.Generator("cpu").manual_seed(seed)
    state = torch.randn(N, H, Dv, Dk, generator=g) * s_std
    q = _unit(torch.randn(steps, N, H, Dk, generator=g))
    k = _unit(torch.randn(steps, N, H, Dk, generator=g))
    v = torch.randn(steps, N, H, Dv, generator=g)
    beta = torch.sigmoid(torch.randn(steps, N, H, generator=g))
    lo, hi = log_alpha_range
    la_shape = (steps, N, H, Dk) if kda else (steps, N, H)
    log_alpha = torch.rand(*la_shape, generator=g) * (hi - lo) + lo
    return {
        "state": state, "q": q.to(dtype), "k": k.to(dtype), "v": v.to(dtype),
        "beta": beta.to(dtype), "log_alpha": log_alpha.to(dtype),
    }


def make_workload(index: int):
    """Inputs of one of the five workloads, with its fixed seed."""
    c = WORKLOADS[index]
    if isinstance(c, DecodeConfig):
        return make_decode(c.N, c.H, c.Dk, c.Dv, c.steps, c.dtype, kda=c.kda, s_std=c.s_std,
                           seed=seed_of(index))
    return make_prefill(c.B, c.H, c.T, c.Dk, c.Dv, c.dtype, kda=c.kda, s0_std=c.s0_std,
                        seed=seed_of(index))


@dataclass(frozen=True)
class ServingConfig:
    """A window of T tokens for N live sequences whose fp32 states sit in a pool of P rows."""
    name: str
    N: int
    H: int
    Hqk: int
    D: int
    T: int
    P: int
    dtype: torch.dtype
    s_std: float
    kda: bool = False
    raw: bool = False


# Serving-side decode workloads (the decode workload's 256 sequences x 32 value heads x
# 128x128 states): speculative verification of 4 draft tokens with 16 query/key heads and
# the raw gate projections; a KDA decode step.
SERVING = {
    "verify": ServingConfig("gdn_decode_verify4_bf16", 256, 32, 16, 128, 4, 512, torch.bfloat16, 0.02, raw=True),
    "kda": ServingConfig("kda_decode_bf16", 256, 32, 32, 128, 1, 256, torch.bfloat16, 0.02, kda=True),
}


def make_serving(N: int, T: int, H: int, Hqk: int, D: int, P: int, dtype: torch.dtype = torch.bfloat16, *,
                 kda: bool = False, raw: bool = False, s_std: float = 0.02, seed: int = 0,
                 skip_every: int = 0) -> Dict[str, Optional[torch.Tensor]]:
    """Draw, in order: the state pool, a slot table (N distinct rows of the pool, every
    skip_every-th sequence marked -1), accepted-token counts in 0..T, then q, k, v and the
    gates of every token.  With ``raw`` the gates are the layer's raw projections b, a
    (N(0, 1)) with per-head A_log ~ U[-1, 1] and dt_bias ~ U[-4, -2], and q, k are left
    unnormalised (3 N(0, 1)); otherwise beta = sigmoid(N(0, 1)), log alpha ~ U[-0.2, -0.005]
    (per key channel for KDA) and q, k have unit length."""
    g = torch.Generator("cpu").manual_seed(seed)
    pool = torch.randn(P, H, D, D, generator=g) * s_std
    slots = torch.randperm(P, generator=g)[:N].to(torch.int32)
    if skip_every > 0:
        slots[::skip_every] = -1
    n_commit = torch.randint(0, T + 1, (N,), generator=g).to(torch.int32)
    if raw:
        q = torch.randn(N, T, Hqk, D, generator=g) * 3
        k = torch.randn(N, T, Hqk, D, generator=g) * 3
    else:
        q = _unit(torch.randn(N, T, Hqk, D, generator=g))
        k = _unit(torch.randn(N, T, Hqk, D, generator=g))
    v = torch.randn(N, T, H, D, generator=g)
    A_log = dt_bias = None
    if raw:
        beta = torch.randn(N, T, H, generator=g)
        log_alpha = torch.randn(N, T, H, generator=g)
        A_log = torch.rand(H, generator=g) * 2 - 1
        dt_bias = torch.rand(H, generator=g) * 2 - 4
    else:
        beta = torch.sigmoid(torch.randn(N, T, H, generator=g))
        log_alpha = torch.rand(*((N, T, H, D) if kda else (N, T, H)), generator=g) * 0.195 - 0.2
    return {"pool": pool, "slots": slots, "n_commit": n_commit, "q": q.to(dtype), "k": k.to(dtype),
            "v": v.to(dtype), "beta": beta.to(dtype), "log_alpha": log_alpha.to(dtype),
            "A_log": A_log, "dt_bias": dt_bias}


def make_prefill_ex(B: int, H: int, Hqk: int, T: int, D: int, dtype: torch.dtype = torch.bfloat16, *,
                    raw: bool = False, unit: bool = True, s0_std: float = 0.01,
                    seed: int = 0) -> Dict[str, Optional[torch.Tensor]]:
    """Prefill inputs with H value heads reading Hqk query/key heads, drawn in the order q, k,
    v, gates, s0 (and A_log, dt_bias for raw gates): q, k [B, Hqk, T, D] ~ N(0, 1), scaled to
    unit length unless ``unit`` is False (the layer's unnormalised projections), v [B, H, T, D];
    the gates as in ``make_serving``."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, Hqk, T, D, generator=g)
    k = torch.randn(B, Hqk, T, D, generator=g)
    if unit:
        q, k = _unit(q), _unit(k)
    v = torch.randn(B, H, T, D, generator=g)
    A_log = dt_bias = None
    if raw:
        beta = torch.randn(B, H, T, generator=g)
        log_alpha = torch.randn(B, H, T, generator=g)
        A_log = torch.rand(H, generator=g) * 2 - 1
        dt_bias = torch.rand(H, generator=g) * 2 - 4
    else:
        beta = torch.sigmoid(torch.randn(B, H, T, generator=g))
        log_alpha = torch.rand(B, H, T, generator=g) * 0.195 - 0.2
    s0 = (torch.randn(B, H, D, D, generator=g) * s0_std) if s0_std > 0 else None
    return {"q": q.to(dtype), "k": k.to(dtype), "v": v.to(dtype), "beta": beta.to(dtype),
            "log_alpha": log_alpha.to(dtype), "s0": s0, "A_log": A_log, "dt_bias": dt_bias}


def ragged_lengths(B: int, lo: int, hi: int, seed: int = 0):
    """Seeded prompt lengths, uniform in [lo, hi] (ragged tails included)."""
    g = torch.Generator("cpu").manual_seed(seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (B,), generator=g)]
