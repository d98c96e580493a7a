"""One prefill step of a RAG-shaped batch with segment-cache hits.

Pages: besthub article "Cut First-Token Latency by 3.25x ...", paragraph 4
(linear layers compose cached (T_C, S(C|0)) records; conv variants get a
convolution state warm-up) and paragraph 6 (longest-processing-time-first
ordering of cold segments).  On one GPU the step is three launches on one
stream, all through the C ABI:

1. build the records of every cold (cache-miss) segment into its fresh pool
   slot, longest segment first (``hypic_build_segment``);
2. the short-conv warm-up at every segment boundary, reading the previous
   segment's last K-1 raw inputs and the segment's first K-1 from per-slot
   tables (``hypic_conv_warmup``);
3. compose every request's chain of slots in prompt order, longest chain first
   (``hypic_compose_chain``).

This module only arranges arguments (device index tables, the longest-first
orders); all arithmetic runs in the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import GDN, Pool, build_segment, compose_chain, conv_warmup


@dataclass
class RagStep:
    """Device-side index tables of one step (built once, reused across steps)."""
    cold_offsets: torch.Tensor     # int64 [n_cold+1], packed cold stream, longest first
    cold_slots: torch.Tensor       # int32 [n_cold], pool slot of each packed cold segment
    chain_offsets: torch.Tensor    # int64 [R+1], requests in longest-chain-first order
    chain_slots: torch.Tensor      # int32, slot ids in prompt order
    request_order: np.ndarray      # request id of each composed row
    tail_index: torch.Tensor       # int32 [B], slot of the segment before each boundary
    head_index: torch.Tensor       # int32 [B], slot of the segment after it
    boundary_request: np.ndarray   # request id of each boundary
    n_cold_tokens: int
    n_compositions: int


def plan_step(chains: List[np.ndarray], cold_slot_lengths: dict, device="cuda") -> RagStep:
    """chains[r]: pool slots of request r in prompt order.  cold_slot_lengths:
    {slot: length} of the segments to build in this step."""
    cold = sorted(cold_slot_lengths.items(), key=lambda kv: -kv[1])           # longest first
    cold_lengths = np.array([n for _, n in cold], dtype=np.int64)
    cold_offsets = np.zeros(len(cold) + 1, dtype=np.int64)
    cold_offsets[1:] = np.cumsum(cold_lengths)
    order = sorted(range(len(chains)), key=lambda r: -len(chains[r]))         # longest chain first
    offs = np.zeros(len(chains) + 1, dtype=np.int64)
    offs[1:] = np.cumsum([len(chains[r]) for r in order])
    flat = np.concatenate([np.asarray(chains[r], dtype=np.int32) for r in order]) if chains else \
        np.zeros(0, np.int32)
    tails, heads, breq = [], [], []
    for r, ch in enumerate(chains):
        for a, b in zip(ch[:-1], ch[1:]):
            tails.append(a)
            heads.append(b)
            breq.append(r)
    t = lambda x, dt: torch.as_tensor(np.asarray(x, dtype=dt)).to(device)
    return RagStep(t(cold_offsets, np.int64), t([s for s, _ in cold], np.int32), t(offs, np.int64),
                   t(flat, np.int32), np.asarray(order), t(tails, np.int32), t(heads, np.int32),
                   np.asarray(breq), int(cold_offsets[-1]), int(offs[-1]))


def prefill_step(step: RagStep, pool: Pool, cold_k: torch.Tensor, cold_v: torch.Tensor,
                 cold_beta: torch.Tensor, cold_log_alpha: torch.Tensor,
                 conv_tails: torch.Tensor, conv_heads: torch.Tensor, conv_weight: torch.Tensor,
                 out_S: torch.Tensor, conv_out: torch.Tensor, conv_bias: Optional[torch.Tensor] = None,
                 conv_activation: int = 0, err_flag: Optional[torch.Tensor] = None, timer=None) -> None:
    """The three launches of one step.  cold_* hold the packed cold stream in
    the order of ``step.cold_offsets``; conv tables are per pool slot
    ([slots, K-1, C]); out_S rows follow ``step.request_order``."""
    run = (lambda name, fn: timer.time(name, fn)) if timer is not None else (lambda name, fn: fn())
    if step.cold_slots.numel():
        run("build", lambda: build_segment(GDN, cold_k, cold_v, cold_log_alpha, step.cold_offsets, pool,
                                           step.cold_slots, beta=cold_beta, err_flag=err_flag))
    if step.tail_index.numel():
        run("conv", lambda: conv_warmup(conv_tails, conv_heads, conv_weight, conv_bias, conv_activation,
                                        tail_index=step.tail_index, head_index=step.head_index,
                                        out=conv_out, err_flag=err_flag))
    run("compose", lambda: compose_chain(pool, step.chain_offsets, step.chain_slots, out_S=out_S,
                                         err_flag=err_flag))
