"""Conv-coupled exact segment records for conv variants (host orchestration).

Source: besthub article "Cut First-Token Latency by 3.25x ...", paragraph 4 (conv
variants need a convolution state warm-up so that reused segments stay aligned).

In a conv variant the keys and values of a segment's first K-1 tokens depend on
the previous segment's last K-1 raw inputs (the causal short conv reaches back
across the boundary); from token K-1 on they depend on the segment alone.  So:

* first prefill (``cache_segments``): every segment's keys and values with its
  own conv (zero history), and the record of its tokens [K-1, n) -- the suffix,
  exact in any context -- into pool slot s;
* reuse (``reuse``): for every chain position, the segment's first min(n, K-1)
  tokens are recomputed with the conv warmed by the raw inputs that precede them
  in this request; the request's state is the chain  head_1, suffix_1, head_2,
  suffix_2, ...,  which equals the recurrence over the concatenated request.
  Where the fused compose takes the pool (GDN, d_k = d_v = 128), the head tokens
  are applied to the running state inside the compose (hypic_compose_chain_heads:
  a few hundred bytes per entry); elsewhere each head becomes a short record
  (hypic_build_segment) composed before its suffix.

Every step runs in libhypic's kernels (hypic_conv_kv, hypic_build_segment,
hypic_compose_chain, hypic_compose_chain_heads); this module only lays out index tables (which raw rows a
token's conv window reads, which tokens form which record) and launches.  The raw
inputs stay in one stream [rows, C] with per-segment row ranges; a cache that keeps
only each segment's first and last K-1 raw rows would index those instead.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import GDN, SCALAR, Pool, build_segment, compose_chain, compose_chain_heads, conv_kv


@dataclass
class ConvCache:
    """Raw inputs and parameters of the cached segments of one conv variant layer
    (GDN, or the scalar family: both have per-token per-head beta and log alpha)."""
    x: torch.Tensor               # [rows, C] raw inputs (bf16 or fp32); segment s = rows [offsets[s], offsets[s+1])
    offsets: np.ndarray           # int64 [S+1]
    beta: torch.Tensor            # [rows, H] fp32
    log_alpha: torch.Tensor       # [rows, H] fp32
    weight: torch.Tensor          # [C, K] fp32
    bias: Optional[torch.Tensor]
    activation: int
    num_heads: int
    d_k: int
    d_v: int
    kv_dtype: torch.dtype         # dtype of the keys and values the records are built from
    family: int = GDN             # GDN, or SCALAR (Mamba2-style: per-token scalar decay [rows, H])

    @property
    def K(self) -> int:
        return self.weight.shape[1]


def _windows(rows_of_pos: np.ndarray, pos: np.ndarray, K: int) -> np.ndarray:
    """Window rows [len(pos), K] of request positions pos: the raw rows of positions
    pos-K+1 .. pos (-1 before the request's first token)."""
    p = pos[:, None] + np.arange(-K + 1, 1)[None, :]
    return np.where(p >= 0, rows_of_pos[np.clip(p, 0, None)], -1).astype(np.int32)


def cache_segments(c: ConvCache, pool: Pool, slots: np.ndarray, from_token: Optional[int] = None,
                   err_flag: Optional[torch.Tensor] = None) -> None:
    """First prefill: record of every segment's tokens [from_token, n) (default K-1,
    the suffix) built with the segment's own conv (zero history) into pool slot
    slots[s].  from_token = 0 gives the standalone record of the whole segment."""
    K = c.K
    f = K - 1 if from_token is None else from_token
    toks, srcs, lens = [], [], []
    for s in range(len(c.offsets) - 1):
        a, b = int(c.offsets[s]), int(c.offsets[s + 1])
        rows = np.arange(a, b, dtype=np.int64)
        pos = np.arange(min(f, b - a), b - a, dtype=np.int64)
        toks.append(_windows(rows, pos, K))
        srcs.append(rows[pos].astype(np.int32))
        lens.append(len(pos))
    win = np.concatenate(toks) if toks else np.zeros((0, K), np.int32)
    src = np.concatenate(srcs) if srcs else np.zeros(0, np.int32)
    dev = c.weight.device
    k, v, b, la = conv_kv(c.x, torch.as_tensor(win, device=dev), c.weight, c.num_heads, c.d_k, c.d_v,
                          bias=c.bias, activation=c.activation, out_dtype=c.kv_dtype,
                          src_token=torch.as_tensor(src, device=dev), beta=c.beta, log_alpha=c.log_alpha,
                          err_flag=err_flag)
    offs = np.zeros(len(lens) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lens)
    build_segment(c.family, k, v, la, torch.as_tensor(offs, device=dev), pool,
                  torch.as_tensor(np.asarray(slots, dtype=np.int32), device=dev), beta=b, err_flag=err_flag)


@dataclass
class ReusePlan:
    head_window: torch.Tensor     # int32 [T, K]
    head_src: torch.Tensor        # int32 [T]
    head_offsets: torch.Tensor    # int64 [B+1]: head record j = head tokens [o_j, o_{j+1})
    head_slots: torch.Tensor      # int32 [B]
    chain_offsets: torch.Tensor   # int64 [R+1]
    chain_slots: torch.Tensor     # int32: head_1, suffix_1, head_2, suffix_2, ...
    suffix_offsets: torch.Tensor  # int64 [R+1]: the chains of suffix slots alone (fused compose)
    suffix_slots: torch.Tensor    # int32: suffix_1, suffix_2, ... (entry j's head tokens: head_offsets[j..j+1])


def plan_reuse(c: ConvCache, chains: List[np.ndarray], suffix_slot: np.ndarray, head_slot_base: int,
               device="cuda") -> ReusePlan:
    """Index tables of one reuse step: chains[r] lists cached segment ids in prompt order;
    segment s's suffix record sits in pool slot suffix_slot[s]; head records go to
    consecutive slots from head_slot_base (one per chain position)."""
    K = c.K
    wins, srcs, hl, cs, co, ss, so = [], [], [], [], [0], [], [0]
    j = 0
    for ch in chains:
        ch = [int(s) for s in ch]
        rows_of_pos = np.concatenate([np.arange(int(c.offsets[s]), int(c.offsets[s + 1]), dtype=np.int64)
                                      for s in ch]) if ch else np.zeros(0, np.int64)
        p0 = 0
        for s in ch:
            n = int(c.offsets[s + 1] - c.offsets[s])
            h = min(n, K - 1)
            pos = np.arange(p0, p0 + h, dtype=np.int64)
            wins.append(_windows(rows_of_pos, pos, K))
            srcs.append(rows_of_pos[pos].astype(np.int32))
            hl.append(h)
            cs += [head_slot_base + j, int(suffix_slot[s])]
            ss.append(int(suffix_slot[s]))
            j += 1
            p0 += n
        co.append(len(cs))
        so.append(len(ss))
    T = int(sum(hl))
    win = np.concatenate(wins) if wins else np.zeros((0, K), np.int32)
    src = np.concatenate(srcs) if srcs else np.zeros(0, np.int32)
    hoffs = np.zeros(len(hl) + 1, dtype=np.int64)
    hoffs[1:] = np.cumsum(hl)
    assert win.shape == (T, K)
    t = lambda a, dt: torch.as_tensor(np.asarray(a, dtype=dt), device=device)
    return ReusePlan(t(win, np.int32), t(src, np.int32), t(hoffs, np.int64),
                     t(np.arange(head_slot_base, head_slot_base + len(hl)), np.int32),
                     t(co, np.int64), t(cs, np.int32), t(so, np.int64), t(ss, np.int32))


def fused_supported(pool: Pool) -> bool:
    """The compose with head tokens takes GDN pools with d_k = d_v = 128."""
    return pool.family == GDN and pool.d_k == 128 and pool.d_v == 128


def reuse(c: ConvCache, plan: ReusePlan, pool: Pool, out_S: Optional[torch.Tensor] = None,
          err_flag: Optional[torch.Tensor] = None, timer=None, fused: Optional[bool] = None) -> torch.Tensor:
    """One reuse step on the current stream: warmed head keys and values, then every
    request's chain composed (fused: head tokens applied inside the compose; else head
    records first).  Returns out_S [R, H, d_k, d_v]."""
    def run(name, fn):
        return timer.time(name, fn) if timer is not None else fn()

    if c.family not in (GDN, SCALAR):
        raise ValueError("conv-coupled records: GDN or scalar family")
    if fused is None:
        fused = fused_supported(pool)
    if fused:
        k, v, b, la = run("conv_kv", lambda: conv_kv(
            c.x, plan.head_window, c.weight, c.num_heads, c.d_k, c.d_v, bias=c.bias, activation=c.activation,
            out_dtype=torch.float32, src_token=plan.head_src, beta=c.beta, log_alpha=c.log_alpha,
            err_flag=err_flag))
        return run("compose", lambda: compose_chain_heads(pool, plan.suffix_offsets, plan.suffix_slots,
                                                          plan.head_offsets, k, v, b, la, out_S=out_S,
                                                          err_flag=err_flag))
    k, v, b, la = run("conv_kv", lambda: conv_kv(
        c.x, plan.head_window, c.weight, c.num_heads, c.d_k, c.d_v, bias=c.bias, activation=c.activation,
        out_dtype=c.kv_dtype, src_token=plan.head_src, beta=c.beta, log_alpha=c.log_alpha, err_flag=err_flag))
    run("head_build", lambda: build_segment(c.family, k, v, la, plan.head_offsets, pool, plan.head_slots,
                                            beta=b, err_flag=err_flag))
    return run("compose", lambda: compose_chain(pool, plan.chain_offsets, plan.chain_slots, out_S=out_S,
                                                err_flag=err_flag))
