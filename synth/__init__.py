"""Seeded synthetic inputs shaped like the HYPIC workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the GPU path (through the tests and the benchmark)
and the fp64 oracle consume the tensors made here: the oracle reads back the
exact bytes the GPU saw.

Distributions (one z ~ N(0,1) draw per element, independent):
  keys        k = z / ||z||_2 over the key dimension (L2-normalised), then cast
              to the storage dtype (bf16 by round-to-nearest-even, or fp32)
  values      v = z
  write gate  beta = sigmoid(z)                                       (GDN)
  decay       log_alpha = -s * softplus(z), s = 0.1 by default       (GDN)
  scalar      log_gamma_h = log U[g_lo, g_hi], constant per head      (RetNet-style)
  diagonal    log-gates = logsigmoid(z) / div, div = 16 by default   (GLA-style)
  conv        raw x = z (bf16), weights U[-0.5, 0.5] (fp32), no bias

There is no public dataset here: the RAG-shaped mix draws its segment counts,
lengths and cache-hit pattern from seeded uniform / Bernoulli draws.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

SCALAR, DIAGONAL, GDN = 0, 1, 2


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def keys(N: int, H: int, dk: int, dtype, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    z = torch.randn((N, H, dk), generator=g, device=device, dtype=torch.float32)
    z = z / torch.linalg.vector_norm(z, dim=-1, keepdim=True).clamp_min(1e-30)
    return z.to(dtype)


def values(N: int, H: int, dv: int, dtype, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.randn((N, H, dv), generator=g, device=device, dtype=torch.float32).to(dtype)


def write_gate(N: int, H: int, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.sigmoid(torch.randn((N, H), generator=g, device=device, dtype=torch.float32))


def gdn_log_decay(N: int, H: int, seed: int, scale: float = 0.1, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    z = torch.randn((N, H), generator=g, device=device, dtype=torch.float32)
    return -scale * torch.nn.functional.softplus(z)


def scalar_log_gamma(H: int, seed: int, lo: float = 0.9, hi: float = 0.999, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    u = torch.rand((H,), generator=g, device=device, dtype=torch.float64)
    return torch.log(lo + (hi - lo) * u).to(torch.float32)


def diagonal_log_gates(N: int, H: int, dk: int, seed: int, div: float = 16.0, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    z = torch.randn((N, H, dk), generator=g, device=device, dtype=torch.float32)
    return torch.nn.functional.logsigmoid(z) / div


def conv_stream(N: int, C: int, dtype, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.randn((N, C), generator=g, device=device, dtype=torch.float32).to(dtype)


def conv_weights(C: int, K: int, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.rand((C, K), generator=g, device=device, dtype=torch.float32) - 0.5


def even_offsets(num_segments: int, seg_len: int) -> np.ndarray:
    return np.arange(num_segments + 1, dtype=np.int64) * seg_len


def offsets_from_lengths(lengths) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


@dataclass
class GdnStream:
    """A packed GDN token stream: k [N,H,dk], v [N,H,dv], beta [N,H], log_alpha [N,H]."""
    k: torch.Tensor
    v: torch.Tensor
    beta: torch.Tensor
    log_alpha: torch.Tensor
    seg_offsets: np.ndarray


def gdn_stream(seg_lengths, H: int, dk: int, dv: int, kv_dtype, seed: int,
               decay_scale: float = 0.1, device="cpu") -> GdnStream:
    offs = offsets_from_lengths(seg_lengths)
    N = int(offs[-1])
    return GdnStream(
        k=keys(N, H, dk, kv_dtype, seed * 10 + 1, device),
        v=values(N, H, dv, kv_dtype, seed * 10 + 2, device),
        beta=write_gate(N, H, seed * 10 + 3, device),
        log_alpha=gdn_log_decay(N, H, seed * 10 + 4, decay_scale, device),
        seg_offsets=offs,
    )


@dataclass
class RagPlan:
    """Seeded plan of the RAG-shaped mix: per request, its segment positions.

    Each position is either a cache hit (``slot`` in the pre-built pool) or a
    cold segment (``cold_index`` into the cold stream, built in the same launch).
    """
    chain_lengths: List[int]
    is_cached: List[np.ndarray]      # per request, bool per position
    cached_slot: List[np.ndarray]    # per request, pool slot for cached positions (-1 otherwise)
    cold_lengths: np.ndarray         # lengths of the cold segments, in request order
    pool_lengths: np.ndarray         # lengths of the pre-built pool segments


def rag_plan(num_requests: int, pool_slots: int, seed: int, m_lo: int = 24, m_hi: int = 96,
             len_lo: int = 128, len_hi: int = 1024, p_cached: float = 0.7) -> RagPlan:
    rng = np.random.Generator(np.random.PCG64(seed))
    pool_lengths = rng.integers(len_lo, len_hi + 1, size=pool_slots)
    chain_lengths, cached, slots, cold = [], [], [], []
    for _ in range(num_requests):
        m = int(rng.integers(m_lo, m_hi + 1))
        hit = rng.random(m) < p_cached
        sl = np.where(hit, rng.integers(0, pool_slots, size=m), -1).astype(np.int64)
        cold_len = rng.integers(len_lo, len_hi + 1, size=m)
        cold.extend(int(x) for x, h in zip(cold_len, hit) if not h)
        chain_lengths.append(m)
        cached.append(hit)
        slots.append(sl)
    return RagPlan(chain_lengths, cached, slots, np.asarray(cold, dtype=np.int64), pool_lengths)
