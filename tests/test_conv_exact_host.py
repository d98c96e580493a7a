"""Host-side index tables of the conv-coupled exact reuse (no GPU):
hybrid_prefill_amd.conv_exact.plan_reuse.

Pages: besthub article "Cut First-Token Latency by 3.25x ...", paragraph 4 (conv
variants need a convolution state warm-up at segment boundaries).  A reused
segment's first K-1 tokens are recomputed with the conv window reaching back into
the raw inputs before them in the request; every later token's window lies inside
the segment (its suffix record is exact in any context)."""
import numpy as np
import torch

from hybrid_prefill_amd import conv_exact


def _cache(offsets, K, C=8, H=1):
    rows = int(offsets[-1])
    return conv_exact.ConvCache(x=torch.zeros(rows, C), offsets=np.asarray(offsets, dtype=np.int64),
                                beta=torch.zeros(rows, H), log_alpha=torch.zeros(rows, H),
                                weight=torch.zeros(C, K), bias=None, activation=0, num_heads=H, d_k=4, d_v=4,
                                kv_dtype=torch.float32)


def test_plan_reuse_worked_example():
    # segments 0, 1, 2 of lengths 5, 2, 3 (raw rows 0-4, 5-6, 7-9); kernel 4; request 2, 0, 1
    c = _cache([0, 5, 7, 10], K=4)
    suffix = np.array([20, 21, 22])
    p = conv_exact.plan_reuse(c, [np.array([2, 0, 1])], suffix, head_slot_base=30, device="cpu")
    assert p.head_window.numpy().tolist() == [
        [-1, -1, -1, 7], [-1, -1, 7, 8], [-1, 7, 8, 9],      # segment 2 opens the request
        [7, 8, 9, 0], [8, 9, 0, 1], [9, 0, 1, 2],           # segment 0 reaches back into segment 2
        [2, 3, 4, 5], [3, 4, 5, 6]]                          # segment 1 (two tokens, both heads)
    assert p.head_src.numpy().tolist() == [7, 8, 9, 0, 1, 2, 5, 6]
    assert p.head_offsets.numpy().tolist() == [0, 3, 6, 8]
    assert p.head_slots.numpy().tolist() == [30, 31, 32]
    assert p.chain_offsets.numpy().tolist() == [0, 6]
    assert p.chain_slots.numpy().tolist() == [30, 22, 31, 20, 32, 21]
    assert p.suffix_offsets.numpy().tolist() == [0, 3]
    assert p.suffix_slots.numpy().tolist() == [22, 20, 21]


def test_plan_reuse_windows_brute_force():
    rng = np.random.default_rng(7)
    lens = rng.integers(0, 9, size=12)
    offs = np.concatenate([[0], np.cumsum(lens)])
    for K in (2, 4, 6):
        c = _cache(offs, K=K)
        chains = [rng.permutation(12)[:m] for m in (1, 4, 7, 12)]
        p = conv_exact.plan_reuse(c, chains, np.arange(12) + 100, head_slot_base=500, device="cpu")
        win, src, ho = p.head_window.numpy(), p.head_src.numpy(), p.head_offsets.numpy()
        j = 0
        for ch in chains:
            stream = [r for s in ch for r in range(offs[s], offs[s + 1])]   # the request's raw rows
            pos = 0
            for s in ch:
                n = int(lens[s])
                h = min(n, K - 1)
                assert ho[j + 1] - ho[j] == h
                for t in range(h):
                    want = [stream[q] if q >= 0 else -1 for q in range(pos + t - K + 1, pos + t + 1)]
                    assert win[ho[j] + t].tolist() == want
                    assert src[ho[j] + t] == stream[pos + t]
                pos += n
                j += 1
        assert j == len(ho) - 1
