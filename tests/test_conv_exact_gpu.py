"""GPU parity of conv-coupled exact records (hybrid_prefill_amd.conv_exact):
suffix records built at first prefill, warmed head records built on reuse, the
chain head_1, suffix_1, head_2, ... composed -- against the fp64 recurrence over
each request's concatenated tokens, whose keys and values come from the causal
conv over the request's whole raw stream (oracle.conv_kv).

Negative control: composing the segments' standalone records (every token's conv
with the segment's own zero history) misses the warm-up and must exceed the
tolerance (weak decay, so that earlier tokens still matter).
"""
import numpy as np
import pytest
import torch

import hybrid_prefill_amd as hp
from hybrid_prefill_amd import conv_exact as ce
import oracle
import synth
from oracle import rel_fro
from parity_util import np64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hp.lib()
    yield
    torch.cuda.synchronize()


LENS = [1, 2, 3, 5, 64, 130, 7, 40, 0, 3]
CHAINS = [[0, 1, 2, 3], [4, 5, 6, 7], [5, 0, 5], [2], [7, 6, 5, 4, 3, 2, 1, 0], [8, 9, 8, 4], []]


def _setup(H, dk, dv, x_dtype, kv_dtype, act, bias, seed, decay, family=hp.GDN):
    K = 4
    C = H * (dk + dv)
    offs = synth.offsets_from_lengths(LENS)
    N = int(offs[-1])
    x = synth.conv_stream(N, C, x_dtype, seed, "cuda")
    w = synth.conv_weights(C, K, seed + 1, "cuda")
    b = torch.randn(C, device="cuda") * 0.1 if bias else None
    beta = synth.write_gate(N, H, seed + 2, "cuda")
    la = synth.gdn_log_decay(N, H, seed + 3, decay, "cuda")
    if family == hp.SCALAR:      # Mamba2-style: per-token scalar decay, beta = 1
        beta = torch.ones_like(beta)
        la = synth.gdn_log_decay(N, H, seed + 3, decay * 10, "cuda")
    return ce.ConvCache(x, offs, beta, la, w, b, act, H, dk, dv, kv_dtype, family)


def _sequential(c, chain, H, dk, dv):
    """Oracle: the recurrence over the request's concatenated tokens, keys and values
    from the conv over its whole raw stream."""
    if not chain:
        return np.zeros((H, dk, dv))
    rows = np.concatenate([np.arange(c.offsets[s], c.offsets[s + 1]) for s in chain]).astype(np.int64)
    x = np64(c.x)[rows]
    k, v = oracle.conv_kv(x, np64(c.weight), None if c.bias is None else np64(c.bias), c.activation, H, dk, dv)
    b, la = np64(c.beta)[rows], np64(c.log_alpha)[rows]
    _, _, S = oracle.build_segments(c.family, k, v, la, [0, len(rows)], beta=b, want_P=False)
    return S[0]


@pytest.mark.parametrize("cfg", [(2, 64, 64, torch.float32, torch.float32, 1, True, 1e-4, hp.GDN),
                                 (4, 128, 128, torch.bfloat16, torch.bfloat16, 0, False, 2e-2, hp.GDN),
                                 (2, 64, 64, torch.float32, torch.float32, 1, False, 1e-4, hp.SCALAR),
                                 (4, 128, 128, torch.bfloat16, torch.bfloat16, 1, True, 2e-2, hp.SCALAR)])
def test_conv_exact_reuse_equals_sequential(cfg):
    H, dk, dv, x_dtype, kv_dtype, act, bias, tol, family = cfg
    c = _setup(H, dk, dv, x_dtype, kv_dtype, act, bias, 1300 + dk + 7 * family, 0.001, family)
    S_seg = len(LENS)
    n_heads = sum(len(ch) for ch in CHAINS)
    pool = hp.Pool.allocate(family, S_seg + n_heads, H, dk, dv, device="cuda", fill=0.0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ce.cache_segments(c, pool, np.arange(S_seg), err_flag=err)
    plan = ce.plan_reuse(c, [np.asarray(ch) for ch in CHAINS], np.arange(S_seg), S_seg)
    say(f"[conv exact] family {family} H={H} d={dk} {x_dtype} act={act}: chains {CHAINS}")
    refs = [_sequential(c, ch, H, dk, dv) for ch in CHAINS]
    paths = [False] + ([True] if ce.fused_supported(pool) else [])
    for fused in paths:
        out = ce.reuse(c, plan, pool, err_flag=err, fused=fused)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        worst = max(rel_fro(np64(out[r, h]), refs[r][h]) for r in range(len(CHAINS)) for h in range(H))
        say(f"   {'fused head tokens' if fused else 'head records'} + suffixes vs sequential: max err {worst:.2e}")
        assert worst <= tol
    if not ce.fused_supported(pool):
        with pytest.raises(hp.HypicError):
            ce.reuse(c, plan, pool, fused=True)

    # negative control: standalone records (zero conv history at every segment start)
    pool2 = hp.Pool.allocate(family, S_seg, H, dk, dv, device="cuda", fill=0.0)
    ce.cache_segments(c, pool2, np.arange(S_seg), from_token=0)
    offs = np.concatenate([[0], np.cumsum([len(ch) for ch in CHAINS])]).astype(np.int64)
    flat = np.asarray(sum(CHAINS, []), dtype=np.int32)
    naive = hp.compose_chain(pool2, torch.as_tensor(offs).cuda(), torch.as_tensor(flat).cuda())
    torch.cuda.synchronize()
    worst_n = max(rel_fro(np64(naive[r, h]), refs[r][h]) for r in (0, 1, 2, 4, 5) for h in range(H))
    say(f"   negative control, standalone segment records: max err {worst_n:.2e}")
    assert worst_n > 10 * tol


def test_conv_kv_bad_window_flags_and_nans():
    H, dk, dv, K = 2, 8, 8, 4
    C = H * (dk + dv)
    x = synth.conv_stream(6, C, torch.float32, 1400, "cuda")
    w = synth.conv_weights(C, K, 1401, "cuda")
    win = torch.tensor([[-1, -1, 0, 1], [0, 1, 2, 9], [2, 3, 4, 5]], dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    k, v = hp.conv_kv(x, win, w, H, dk, dv, out_dtype=torch.float32, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == hp.EFLAG_SLOT_OUT_OF_RANGE
    assert torch.all(torch.isnan(k[1])) and torch.all(torch.isnan(v[1]))
    assert not torch.any(torch.isnan(k[[0, 2]])) and not torch.any(torch.isnan(v[[0, 2]]))
    # rows 0 and 2 against the oracle's conv of their windows
    xs = np64(x)
    for t, rows in ((0, [0, 1]), (2, [2, 3, 4, 5])):
        kr, vr = oracle.conv_kv(xs[rows], np64(w), None, 1, H, dk, dv)
        assert rel_fro(np64(k[t]), kr[-1]) < 1e-5 and rel_fro(np64(v[t]), vr[-1]) < 1e-5


@pytest.mark.parametrize("R", [3, 20])
def test_compose_chain_heads_against_oracle(R):
    """hypic_compose_chain_heads on synthetic records and head tokens (0 to 8 per entry):
    each entry's head tokens built into a record by the oracle, composed before the
    entry's record; 3 requests (a 1100-entry chain crosses the LDS slot ring's refill)
    and 20 requests; malformed head offsets (9 tokens) flag and NaN-fill that request."""
    H, d, nslots = 2, 128, 16
    rng = np.random.default_rng(1500 + R)
    q, _ = np.linalg.qr(rng.standard_normal((nslots, H, d, d)))
    pool = hp.Pool.allocate(hp.GDN, nslots, H, d, d, device="cuda", fill=0.0)
    pool.P.copy_(torch.from_numpy(q * rng.uniform(0.9, 1.0, size=(nslots, H, 1, d))).float())
    pool.S.copy_(torch.from_numpy(rng.standard_normal((nslots, H, d, d))).float())
    pool.log_scale.copy_(torch.from_numpy(rng.uniform(-0.05, 0.0, size=(nslots, H))).float())
    lens = [1100, 0, 7] if R == 3 else [int(x) for x in rng.integers(0, 12, size=R)]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    flat = rng.integers(0, nslots, size=int(offs[-1])).astype(np.int32)
    nh = rng.integers(0, 9, size=len(flat))
    hoffs = np.concatenate([[0], np.cumsum(nh)]).astype(np.int64)
    T = int(hoffs[-1])
    hk = synth.keys(T, H, d, torch.float32, 1510 + R, "cuda")
    hv = synth.values(T, H, d, torch.float32, 1511 + R, "cuda")
    hb = synth.write_gate(T, H, 1512 + R, "cuda")
    hla = synth.gdn_log_decay(T, H, 1513 + R, 0.1, "cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out_ell = torch.empty((R, H), device="cuda")
    out = hp.compose_chain_heads(pool, torch.as_tensor(offs).cuda(), torch.as_tensor(flat).cuda(),
                                 torch.as_tensor(hoffs).cuda(), hk, hv, hb, hla, out_log_scale=out_ell,
                                 err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # oracle: a record per entry's head tokens, composed before the entry's record
    k_, v_, b_, la_ = np64(hk), np64(hv), np64(hb), np64(hla)
    hell, hP, hS = oracle.build_segments(oracle.GDN, k_, v_, la_, hoffs, beta=b_)
    E = len(flat)
    mp_ell = np.concatenate([hell, np64(pool.log_scale)[flat]])           # [2E + ..., H]
    mp_P = np.concatenate([hP, np64(pool.P)[flat]])
    mp_S = np.concatenate([hS, np64(pool.S)[flat]])
    chain = np.empty(2 * E, dtype=np.int32)
    chain[0::2] = np.arange(E)
    chain[1::2] = E + np.arange(E)
    rS, rell, _ = oracle.compose(oracle.GDN, mp_ell, mp_P, mp_S, 2 * offs, chain)
    worst = max(rel_fro(np64(out[r, h]), rS[r, h]) for r in range(R) for h in range(H))
    dl = float(np.max(np.abs(np64(out_ell) - rell)))
    say(f"[compose heads] R={R} lens={lens[:6]} head tokens {T}: S err {worst:.2e}, ell err {dl:.2e}")
    assert worst <= 1e-4 and dl <= 1e-4
    # 9 head tokens at one entry of request 1: that request only is NaN, the flag says bad offsets
    nh2 = nh.copy()
    e1 = int(offs[1]) if lens[1] > 0 else int(offs[2]) if R > 2 and lens[2] > 0 else None
    if e1 is not None:
        nh2[e1] = 9
        hoffs2 = np.concatenate([[0], np.cumsum(nh2)]).astype(np.int64)
        T2 = int(hoffs2[-1])
        err.zero_()
        out2 = hp.compose_chain_heads(pool, torch.as_tensor(offs).cuda(), torch.as_tensor(flat).cuda(),
                                      torch.as_tensor(hoffs2).cuda(),
                                      *[torch.cat([x, x[:max(0, T2 - T)]]) for x in (hk, hv, hb, hla)],
                                      err_flag=err)
        torch.cuda.synchronize()
        bad_r = 1 if lens[1] > 0 else 2
        assert int(err.item()) & hp.EFLAG_BAD_OFFSETS
        assert torch.all(torch.isnan(out2[bad_r])) and not torch.any(torch.isnan(out2[0]))


@pytest.mark.parametrize("dims,dtype", [((1, 3, 2), torch.float32), ((3, 5, 3), torch.bfloat16),
                                        ((2, 64, 64), torch.bfloat16)])
def test_conv_kv_against_oracle(dims, dtype):
    """conv_kv on a stream with per-token windows (the stream's own history) against the
    oracle, on channel counts off and on the 16-byte vector width (both kernel forms)."""
    H, dk, dv = dims
    K, n = 4, 37
    C = H * (dk + dv)
    x = synth.conv_stream(n, C, dtype, 1600 + C, "cuda")
    w = synth.conv_weights(C, K, 1601 + C, "cuda")
    bias = torch.randn(C, device="cuda") * 0.1
    pos = np.arange(n)[:, None] + np.arange(-K + 1, 1)[None, :]
    win = torch.as_tensor(np.where(pos >= 0, pos, -1).astype(np.int32), device="cuda")
    k, v = hp.conv_kv(x, win, w, H, dk, dv, bias=bias, activation=1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    kr, vr = oracle.conv_kv(np64(x), np64(w), np64(bias), 1, H, dk, dv)
    ek, ev = rel_fro(np64(k), kr), rel_fro(np64(v), vr)
    say(f"[conv_kv] H={H} dk={dk} dv={dv} C={C} {dtype}: k err {ek:.2e}, v err {ev:.2e}")
    assert ek <= 1e-5 and ev <= 1e-5


def test_compose_chain_heads_strong_gates():
    """hypic_compose_chain_heads with some head tokens gated by e^-50 and e^-80 (decays
    far below the others, so an entry's head tokens all but reset the state), against
    the oracle as above."""
    H, d, nslots, R = 2, 128, 16, 12
    rng = np.random.default_rng(1580)
    q, _ = np.linalg.qr(rng.standard_normal((nslots, H, d, d)))
    pool = hp.Pool.allocate(hp.GDN, nslots, H, d, d, device="cuda", fill=0.0)
    pool.P.copy_(torch.from_numpy(q * rng.uniform(0.9, 1.0, size=(nslots, H, 1, d))).float())
    pool.S.copy_(torch.from_numpy(rng.standard_normal((nslots, H, d, d))).float())
    pool.log_scale.copy_(torch.from_numpy(rng.uniform(-0.05, 0.0, size=(nslots, H))).float())
    lens = [int(x) for x in rng.integers(1, 12, size=R)]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    flat = rng.integers(0, nslots, size=int(offs[-1])).astype(np.int32)
    nh = rng.integers(0, 9, size=len(flat))
    hoffs = np.concatenate([[0], np.cumsum(nh)]).astype(np.int64)
    T = int(hoffs[-1])
    hk = synth.keys(T, H, d, torch.float32, 1581, "cuda")
    hv = synth.values(T, H, d, torch.float32, 1582, "cuda")
    hb = synth.write_gate(T, H, 1583, "cuda")
    hla = synth.gdn_log_decay(T, H, 1584, 0.1, "cuda")
    hla[::7] = -50.0
    hla[3::11] = -80.0
    out = hp.compose_chain_heads(pool, torch.as_tensor(offs).cuda(), torch.as_tensor(flat).cuda(),
                                 torch.as_tensor(hoffs).cuda(), hk, hv, hb, hla)
    torch.cuda.synchronize()
    k_, v_, b_, la_ = np64(hk), np64(hv), np64(hb), np64(hla)
    hell, hP, hS = oracle.build_segments(oracle.GDN, k_, v_, la_, hoffs, beta=b_)
    E = len(flat)
    mp_ell = np.concatenate([hell, np64(pool.log_scale)[flat]])
    mp_P = np.concatenate([hP, np64(pool.P)[flat]])
    mp_S = np.concatenate([hS, np64(pool.S)[flat]])
    chain = np.empty(2 * E, dtype=np.int32)
    chain[0::2] = np.arange(E)
    chain[1::2] = E + np.arange(E)
    rS, _, _ = oracle.compose(oracle.GDN, mp_ell, mp_P, mp_S, 2 * offs, chain)
    worst = max(rel_fro(np64(out[r, h]), rS[r, h]) for r in range(R) for h in range(H))
    say(f"[compose heads strong gates] head tokens {T}: S err {worst:.2e}")
    assert worst <= 1e-4
