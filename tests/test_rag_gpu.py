"""GPU parity of one RAG-shaped prefill step (cold builds + conv warm-up + chain
composition, hybrid_prefill_amd.rag) against the fp64 oracle.

The mix follows the RAG workload's structure (seeded segment counts and
lengths uniform on 128-1024 tokens, 70 % cache hits from a pre-built pool,
GDN H=32, d=128, bf16, conv 4096 channels x kernel 4) at a size the oracle
checks in seconds: 5 requests of 24-40 segments, a 40-slot pool.
"""
import numpy as np
import pytest
import torch

import hybrid_prefill_amd as hp
from hybrid_prefill_amd import rag
import oracle
import synth
from oracle import rel_fro
from parity_util import np64, say

pytestmark = pytest.mark.gpu


def test_rag_mix_step():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R, P, H, d, C, K, seed = 5, 40, 32, 128, 4096, 4, 777
    plan = synth.rag_plan(R, P, seed, m_lo=24, m_hi=40)
    say(f"[rag] {R} requests, chains {plan.chain_lengths}, {len(plan.cold_lengths)} cold segments")
    pst = synth.gdn_stream(plan.pool_lengths, H, d, d, torch.bfloat16, seed * 10 + 1, 0.1, "cuda")
    n_cold = len(plan.cold_lengths)
    pool = hp.Pool.allocate(hp.GDN, P + n_cold, H, d, d, device="cuda", fill=0.0)
    hp.build_segment(hp.GDN, pst.k, pst.v, pst.log_alpha, torch.as_tensor(pst.seg_offsets).cuda(), pool,
                     torch.arange(P, dtype=torch.int32, device="cuda"), beta=pst.beta)
    chains, cold_len, j = [], {}, 0
    for r in range(R):
        ch = []
        for pos in range(plan.chain_lengths[r]):
            if plan.is_cached[r][pos]:
                ch.append(int(plan.cached_slot[r][pos]))
            else:
                cold_len[P + j] = int(plan.cold_lengths[j])
                ch.append(P + j)
                j += 1
        chains.append(np.asarray(ch, dtype=np.int32))
    step = rag.plan_step(chains, cold_len)
    cold_order = [s for s, _ in sorted(cold_len.items(), key=lambda kv: -kv[1])]
    cst = synth.gdn_stream([cold_len[s] for s in cold_order], H, d, d, torch.bfloat16, seed * 10 + 2, 0.1,
                           "cuda")
    assert np.array_equal(cst.seg_offsets, step.cold_offsets.cpu().numpy())
    tails = synth.conv_stream((P + n_cold) * (K - 1), C, torch.bfloat16, seed + 3, "cuda").view(-1, K - 1, C)
    heads = synth.conv_stream((P + n_cold) * (K - 1), C, torch.bfloat16, seed + 4, "cuda").view(-1, K - 1, C)
    w = synth.conv_weights(C, K, seed + 5, "cuda")
    out_S = torch.empty((R, H, d, d), device="cuda")
    conv_out = torch.empty((step.tail_index.numel(), K - 1, C), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rag.prefill_step(step, pool, cst.k, cst.v, cst.beta, cst.log_alpha, tails, heads, w, out_S, conv_out,
                     err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    # ---- composed states against the recurrence over each request's concatenated tokens
    src = {}
    for s in range(P):
        src[s] = (pst, int(pst.seg_offsets[s]), int(pst.seg_offsets[s + 1]))
    for i, s in enumerate(cold_order):
        src[s] = (cst, int(cst.seg_offsets[i]), int(cst.seg_offsets[i + 1]))
    heads_chk = [0, 19]
    host = {id(pst): [np64(x) for x in (pst.k, pst.v, pst.beta, pst.log_alpha)],
            id(cst): [np64(x) for x in (cst.k, cst.v, cst.beta, cst.log_alpha)]}
    ks, vs, bs, las, lens = [], [], [], [], []
    for r in range(R):
        parts = [src[int(s)] for s in chains[r]]
        for arr, lst in ((0, ks), (1, vs), (2, bs), (3, las)):
            lst.append(np.concatenate([host[id(stt)][arr][a:b][:, heads_chk] for stt, a, b in parts]))
        lens.append(sum(b - a for _, a, b in parts))
    _, _, S_seq = oracle.build_segments(oracle.GDN, np.concatenate(ks), np.concatenate(vs),
                                        np.concatenate(las), synth.offsets_from_lengths(lens),
                                        beta=np.concatenate(bs), want_P=False)
    row_of = {int(r): i for i, r in enumerate(step.request_order)}
    worst = max(rel_fro(np64(out_S[row_of[r], h]), S_seq[r, j]) for r in range(R) for j, h in enumerate(heads_chk))
    say(f"   composed state vs sequential recurrence over the concatenation: max err {worst:.2e}")
    assert worst <= 2e-2

    # ---- conv warm-up at every boundary against the causal conv over [tail; head]
    th, hh, wn = np64(tails), np64(heads), np64(w)
    ti, hi = step.tail_index.cpu().numpy(), step.head_index.cpu().numpy()
    cw = np64(conv_out)
    worst_c = 0.0
    for b in range(0, len(ti), 7):
        y = oracle.causal_conv(np.concatenate([th[ti[b]], hh[hi[b]]]), wn, None, 0)
        worst_c = max(worst_c, rel_fro(cw[b], y[K - 1:]))
    say(f"   conv warm-up over {len(range(0, len(ti), 7))} boundaries: max err {worst_c:.2e}")
    assert worst_c <= 1e-4
