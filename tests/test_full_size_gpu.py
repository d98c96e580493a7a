"""GPU parity at the benchmark workloads' full sizes, in the launch configurations
the benchmark times, on sampled outputs the fp64 oracle computes one by one.

  pool compose  4096-slot GDN pool (H=32, d=128, fp32 records built from seeded
                64-token segments), 64 requests x 32 seeded slot ids: one workgroup
                per (request, head) chain.  Sampled (request, head) states against
                the oracle's composition of the same records read back (so build
                error cannot leak in), and sampled pool records against the
                oracle's build of their tokens.
  RAG mix       128 requests of 24-96 segments (128-1024 tokens), 70 % cache hits
                from a 4096-slot pool, cold segments built in the step, conv
                warm-up (4096 channels, kernel 4) at every boundary.  Sampled
                requests' composed states against the recurrence over their
                concatenated tokens, sampled cold records against the oracle's
                build, sampled boundaries against the causal conv.
  KDA build     H=16, d=128, bf16, 8 x 2048 tokens: sampled records' S, and T_C
                over a 256-token build of the same stream.
"""
import numpy as np
import pytest
import torch

import hybrid_prefill_amd as hp
from hybrid_prefill_amd import rag
import oracle
import synth
from oracle import rel_fro
from parity_util import np64, oracle_unit, record_errors, say

pytestmark = pytest.mark.gpu
H, D = 32, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hp.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _records(pool, slots, h):
    """fp64 copies of the pool records of `slots` for head h: (ell [m,1], P [m,1], S [m,1])."""
    idx = torch.as_tensor(np.asarray(slots, dtype=np.int64), device="cuda")
    ell = np64(pool.log_scale[idx, h:h + 1])
    P = np64(pool.P[idx, h:h + 1])
    S = np64(pool.S[idx, h:h + 1])
    return ell, P, S


def test_compose_pool_full_size():
    slots, R, m, seg_len, seed = 4096, 64, 32, 64, 401
    say(f"[full compose] pool {slots} x {H} heads, {R} requests x {m} slots")
    st = synth.gdn_stream([seg_len] * slots, H, D, D, torch.bfloat16, seed, 0.01, "cuda")
    pool = hp.Pool.allocate(hp.GDN, slots, H, D, D, device="cuda")
    hp.build_segment(hp.GDN, st.k, st.v, st.log_alpha, torch.as_tensor(st.seg_offsets).cuda(), pool,
                     torch.arange(slots, dtype=torch.int32, device="cuda"), beta=st.beta)
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = rng.integers(0, slots, size=R * m).astype(np.int32)
    offs = np.arange(0, R * m + 1, m, dtype=np.int64)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out_ell = torch.empty((R, H), device="cuda")
    out = hp.compose_chain(pool, torch.as_tensor(offs).cuda(), torch.as_tensor(ids).cuda(),
                           out_log_scale=out_ell, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    # sampled pool records against the oracle's build of their tokens (bf16 inputs: 2e-2)
    k, v = st.k, st.v
    worst_b = [0.0, 0.0, 0.0]
    for s, h in ((0, 0), (1234, 17), (4095, 31)):
        t0, t1 = int(st.seg_offsets[s]), int(st.seg_offsets[s + 1])
        ref = oracle_unit(oracle.GDN, np64(k[t0:t1]), np64(v[t0:t1]), np64(st.log_alpha[t0:t1]),
                          np64(st.beta[t0:t1]), 0, t1 - t0, h)
        e = record_errors(oracle.GDN, float(pool.log_scale[s, h]), np64(pool.P[s, h]), np64(pool.S[s, h]), *ref)
        worst_b = [max(a, b) for a, b in zip(worst_b, e)]
    say(f"   sampled pool records: S err {worst_b[0]:.2e}, T err {worst_b[1]:.2e}, ell err {worst_b[2]:.2e}")
    assert max(worst_b) <= 2e-2
    del st, k, v

    # sampled chains against the oracle's composition of the same (read-back) records
    worst = [0.0, 0.0]
    for r, h in ((0, 0), (17, 13), (40, 5), (63, 31)):
        chain = ids[offs[r]:offs[r + 1]]
        ell, P, S = _records(pool, chain, h)
        rS, rell, _ = oracle.compose(oracle.GDN, ell, P, S, np.array([0, m], dtype=np.int64),
                                     np.arange(m, dtype=np.int32))
        worst[0] = max(worst[0], rel_fro(np64(out[r, h]), rS[0, 0]))
        worst[1] = max(worst[1], abs(float(out_ell[r, h]) - float(rell[0, 0])))
    say(f"   sampled chains: composed S err {worst[0]:.2e}, ell err {worst[1]:.2e}")
    assert worst[0] <= 1e-4 and worst[1] <= 1e-4
    del pool, out
    torch.cuda.empty_cache()


def test_rag_mix_full_size():
    R, P, C, K, seed = 128, 4096, 4096, 4, 501
    plan = synth.rag_plan(R, P, seed)
    n_cold = len(plan.cold_lengths)
    say(f"[full rag] {R} requests, {sum(plan.chain_lengths)} segments, {n_cold} cold")
    pool = hp.Pool.allocate(hp.GDN, P + n_cold, H, D, D, device="cuda")
    batch = 256
    for b0 in range(0, P, batch):                  # pool fill in seeded batches (regenerated below)
        lens = plan.pool_lengths[b0:b0 + batch]
        st = synth.gdn_stream(lens, H, D, D, torch.bfloat16, seed * 1000 + b0, 0.1, "cuda")
        hp.build_segment(hp.GDN, st.k, st.v, st.log_alpha, torch.as_tensor(st.seg_offsets).cuda(), pool,
                         torch.arange(b0, b0 + len(lens), dtype=torch.int32, device="cuda"), beta=st.beta)
        del st
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
    cst = synth.gdn_stream([cold_len[s] for s in cold_order], H, D, D, torch.bfloat16, seed * 1000 + 999, 0.1,
                           "cuda")
    assert np.array_equal(cst.seg_offsets, step.cold_offsets.cpu().numpy())
    tails = synth.conv_stream((P + n_cold) * (K - 1), C, torch.bfloat16, seed + 7, "cuda").view(-1, K - 1, C)
    heads = synth.conv_stream((P + n_cold) * (K - 1), C, torch.bfloat16, seed + 8, "cuda").view(-1, K - 1, C)
    w = synth.conv_weights(C, K, seed + 9, "cuda")
    out_S = torch.empty((R, H, D, D), device="cuda")
    conv_out = torch.empty((step.tail_index.numel(), K - 1, C), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rag.prefill_step(step, pool, cst.k, cst.v, cst.beta, cst.log_alpha, tails, heads, w, out_S, conv_out,
                     err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    # ---- sampled cold records against the oracle's build (first, middle and last cold slot)
    worst_b = [0.0, 0.0, 0.0]
    for i, h in ((0, 0), (n_cold // 2, 21), (n_cold - 1, 31)):
        s = cold_order[i]
        t0, t1 = int(cst.seg_offsets[i]), int(cst.seg_offsets[i + 1])
        ref = oracle_unit(oracle.GDN, np64(cst.k[t0:t1]), np64(cst.v[t0:t1]), np64(cst.log_alpha[t0:t1]),
                          np64(cst.beta[t0:t1]), 0, t1 - t0, h)
        e = record_errors(oracle.GDN, float(pool.log_scale[s, h]), np64(pool.P[s, h]), np64(pool.S[s, h]), *ref)
        worst_b = [max(a, b) for a, b in zip(worst_b, e)]
    say(f"   sampled cold records: S err {worst_b[0]:.2e}, T err {worst_b[1]:.2e}, ell err {worst_b[2]:.2e}")
    assert max(worst_b) <= 2e-2

    # ---- sampled requests (the two shortest and one more) against the recurrence over their
    #      concatenated tokens; the pool segments' tokens are regenerated from their batch seed
    lens_r = [len(c) for c in chains]
    sample = sorted(range(R), key=lambda r: lens_r[r])[:2] + [R // 2]
    h_chk = [0, 23]
    cache = {}

    def seg_tokens(s):
        if s >= P:
            i = cold_order.index(s)
            a, b = int(cst.seg_offsets[i]), int(cst.seg_offsets[i + 1])
            src = cst
        else:
            b0 = s // batch * batch
            if b0 not in cache:
                cache.clear()
                cache[b0] = synth.gdn_stream(plan.pool_lengths[b0:b0 + batch], H, D, D, torch.bfloat16,
                                             seed * 1000 + b0, 0.1, "cuda")
            src = cache[b0]
            a, b = int(src.seg_offsets[s - b0]), int(src.seg_offsets[s - b0 + 1])
        return [np64(x[a:b][:, h_chk]) for x in (src.k, src.v, src.beta, src.log_alpha)]

    row_of = {int(r): i for i, r in enumerate(step.request_order)}
    worst = 0.0
    for r in sample:
        # regenerate batch by batch in slot order so each batch is drawn once
        parts = {}
        for s in sorted(set(int(x) for x in chains[r])):
            parts[s] = seg_tokens(s)
        seq = [parts[int(s)] for s in chains[r]]
        k, v, b, la = (np.concatenate([p[i] for p in seq]) for i in range(4))
        _, _, S_seq = oracle.build_segments(oracle.GDN, k, v, la, [0, k.shape[0]], beta=b, want_P=False)
        for j, h in enumerate(h_chk):
            worst = max(worst, rel_fro(np64(out_S[row_of[r], h]), S_seq[0, j]))
        say(f"   request {r}: {len(chains[r])} segments, {k.shape[0]} tokens, max err so far {worst:.2e}")
    assert worst <= 2e-2

    # ---- sampled boundaries against the causal conv over [tail; head]
    ti, hi = step.tail_index.cpu().numpy(), step.head_index.cpu().numpy()
    wn = np64(w)
    worst_c = 0.0
    for bnd in list(range(0, len(ti), max(1, len(ti) // 16))) + [len(ti) - 1]:
        y = oracle.causal_conv(np.concatenate([np64(tails[int(ti[bnd])]), np64(heads[int(hi[bnd])])]), wn, None, 0)
        worst_c = max(worst_c, rel_fro(np64(conv_out[bnd]), y[K - 1:]))
    say(f"   sampled conv boundaries: max err {worst_c:.2e}")
    assert worst_c <= 1e-4
    del pool, cst, out_S
    torch.cuda.empty_cache()


def test_kda_build_full_size():
    """KDA family at the benchmark's KDA workload and launch (H=16, d=128, bf16, 8 x 2048
    tokens, diagonal-family gates): sampled (segment, head) records' S against the
    oracle's build of those tokens, and their T_C on the first 256 tokens of the same
    stream (a separate build call: over 2048 tokens T_C falls below the fp32 range)."""
    Hk, nseg, L, seed = 16, 8, 2048, 701
    N = nseg * L
    k = synth.keys(N, Hk, D, torch.bfloat16, seed, "cuda")
    v = synth.values(N, Hk, D, torch.bfloat16, seed + 1, "cuda")
    b = synth.write_gate(N, Hk, seed + 2, "cuda")
    la = synth.diagonal_log_gates(N, Hk, D, seed + 3, 16.0, "cuda")
    offs = synth.even_offsets(nseg, L)
    pool = hp.Pool.allocate(hp.KDA, nseg, Hk, D, D, device="cuda")
    hp.build_segment(hp.KDA, k, v, la, torch.as_tensor(offs).cuda(), pool,
                     torch.arange(nseg, dtype=torch.int32, device="cuda"), beta=b)
    short = np.array([0, 256], dtype=np.int64)
    pool_s = hp.Pool.allocate(hp.KDA, 1, Hk, D, D, device="cuda")
    hp.build_segment(hp.KDA, k, v, la, torch.as_tensor(short).cuda(), pool_s,
                     torch.zeros(1, dtype=torch.int32, device="cuda"), beta=b)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(seed))
    worst = 0.0
    for s, h in zip(rng.integers(0, nseg, 3), rng.integers(0, Hk, 3)):
        s, h = int(s), int(h)
        a, e = int(offs[s]), int(offs[s + 1])
        _, _, S = oracle.build_segments(oracle.KDA, np64(k[a:e, h:h + 1]), np64(v[a:e, h:h + 1]),
                                        np64(la[a:e, h:h + 1]), [0, e - a], beta=np64(b[a:e, h:h + 1]),
                                        want_P=False)
        worst = max(worst, rel_fro(np64(pool.S[s, h]), S[0, 0]))
    h = int(rng.integers(0, Hk))
    _, P, _ = oracle.build_segments(oracle.KDA, np64(k[:256, h:h + 1]), np64(v[:256, h:h + 1]),
                                    np64(la[:256, h:h + 1]), short, beta=np64(b[:256, h:h + 1]))
    eT = rel_fro(np64(pool_s.P[0, h]), P[0, 0])
    say(f"[full kda] sampled S err {worst:.2e}, T_C (256 tokens, head {h}) err {eT:.2e}")
    assert worst <= 2e-2 and eT <= 2e-2
