"""Edge cases, error paths and bit-exact pool indexing through the kernels the
benchmark times: the GDN build on the matrix cores (bf16 k/v, d_k = d_v = 128) and
both d = 128 compose launch paths (four workgroups per chain while there are at most
512 (request, head) units, one workgroup per chain above that).

What is fixed independently of any implementation:
  * beta = 0 writes nothing: S = 0 and P = I exactly, ell = sum of log alpha;
  * a repeated key with beta = 1 and no decay overwrites (against the fp64 oracle);
  * an out-of-range destination slot flags and writes nothing; every other slot
    keeps its bytes;
  * bad offsets flag and NaN-fill that segment's record only;
  * a NaN or Inf input reaches the record of its (segment, head) and no other; log
    alpha enters ell and S only, v enters S only, so P stays finite and correct;
  * a chain of one record from a zero start returns that record's S (and P) bit for
    bit; a record with ell = -inf forgets the state before it, so the output is that
    record's S (pool indexing is bit-exact).
"""
import math

import numpy as np
import pytest
import torch

import hybrid_prefill_amd as hp
import oracle
import synth
from oracle import rel_fro
from parity_util import TOL, dev_i32, dev_i64, np64, record_errors, say

pytestmark = pytest.mark.gpu
CANARY = 12345.0
D = 128
BF = torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hp.lib()
    yield
    torch.cuda.synchronize()


def _stream(lens, H, seed, scale=0.1):
    st = synth.gdn_stream(lens, H, D, D, BF, seed, scale, "cuda")
    return st.k, st.v, st.beta, st.log_alpha, np.asarray(st.seg_offsets, dtype=np.int64)


def _build(k, v, beta, la, offs, slots, num_slots, err):
    pool = hp.Pool.allocate(hp.GDN, num_slots, k.shape[1], D, D, device="cuda", fill=CANARY)
    hp.build_segment(hp.GDN, k, v, la, dev_i64(offs), pool, dev_i32(slots), beta=beta, err_flag=err)
    torch.cuda.synchronize()
    return pool


def _oracle(k, v, beta, la, offs):
    return oracle.build_segments(oracle.GDN, np64(k), np64(v), np64(la), offs, beta=np64(beta))


def _check_record(pool, slot, ref, s, h, tol=TOL[BF]):
    ell_r, P_r, S_r = ref
    e = record_errors(oracle.GDN, float(pool.log_scale[slot, h]), np64(pool.P[slot, h]), np64(pool.S[slot, h]),
                      ell_r[s, h], P_r[s, h], S_r[s, h])
    assert max(e) <= tol, (slot, h, e)
    return e


def _err():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def test_mfma_build_beta_zero():
    """beta = 0 on every token: nothing is written, over full chunks and a ragged tail."""
    H, lens = 4, [130, 64, 1, 0, 200]
    k, v, beta, la, offs = _stream(lens, H, 1101)
    beta = torch.zeros_like(beta)
    err = _err()
    pool = _build(k, v, beta, la, offs, list(range(len(lens))), len(lens), err)
    say(f"[mfma beta=0] H={H} lens={lens}")
    assert int(err.item()) == 0
    assert torch.all(pool.S == 0)
    assert torch.equal(pool.P, torch.eye(D, device="cuda").expand_as(pool.P))
    la64 = np64(la)
    for s in range(len(lens)):
        ref = la64[offs[s]:offs[s + 1]].sum(axis=0)
        assert np.max(np.abs(np64(pool.log_scale[s]) - ref)) <= 1e-5 * max(1.0, float(np.max(np.abs(ref))))


def test_mfma_build_repeated_key_overwrites():
    """beta = 1, no decay, one key repeated: each token's write replaces the last
    (the delta rule's overwrite), against the oracle on the same bytes."""
    H, n = 4, 150
    k, v, beta, la, offs = _stream([n], H, 1102, scale=0.0)
    k[:] = k[0:1].clone()
    beta = torch.ones_like(beta)
    err = _err()
    pool = _build(k, v, beta, la, offs, [0], 1, err)
    ref = _oracle(k, v, beta, la, offs)
    assert int(err.item()) == 0
    worst = max(max(_check_record(pool, 0, ref, 0, h)) for h in range(H))
    # the oracle itself is the overwrite up to the key's bf16 norm error
    for h in range(H):
        kv = np.outer(np64(k[0, h]), np64(v[n - 1, h]))
        assert rel_fro(ref[2][0, h], kv) <= 2e-2
    say(f"[mfma repeated key] H={H} n={n}: max err {worst:.2e}")


def test_mfma_build_out_of_range_slot_keeps_other_slots():
    """A destination slot outside the pool flags and writes nothing; the in-range
    segment's record is correct; the untouched slots keep their canary bytes."""
    H, lens = 32, [200, 300]
    k, v, beta, la, offs = _stream(lens, H, 1103)
    err = _err()
    pool = _build(k, v, beta, la, offs, [1, 7], 3, err)
    say(f"[mfma bad slot] H={H} lens={lens} slots [1, 7] of 3")
    assert int(err.item()) == hp.EFLAG_SLOT_OUT_OF_RANGE
    for t in (pool.S, pool.P, pool.log_scale):
        assert torch.all(t[[0, 2]] == CANARY)
    ref = _oracle(k, v, beta, la, offs)
    for h in range(H):
        _check_record(pool, 1, ref, 0, h)


@pytest.mark.parametrize("bad_offs", ["past_end", "decreasing"])
def test_mfma_build_bad_offsets_nan_record(bad_offs):
    """Offsets past the stream (or decreasing) flag and NaN-fill that segment's record;
    the segment beside it is built normally."""
    H, lens = 32, [200, 300]
    k, v, beta, la, offs = _stream(lens, H, 1104)
    N = int(offs[-1])
    offs_bad = np.array([0, 200, N + 5] if bad_offs == "past_end" else [0, 200, 150], dtype=np.int64)
    err = _err()
    pool = _build(k, v, beta, la, offs_bad, [0, 2], 3, err)
    say(f"[mfma bad offsets] {bad_offs}: {offs_bad.tolist()}")
    assert int(err.item()) == hp.EFLAG_BAD_OFFSETS
    for t in (pool.S, pool.P, pool.log_scale):
        assert torch.all(torch.isnan(t[2]))
        assert torch.all(t[1] == CANARY)
    ref = _oracle(k, v, beta, la, offs)
    for h in range(H):
        _check_record(pool, 0, ref, 0, h)


def test_mfma_build_nan_inf_inputs_stay_in_their_record():
    """NaN in a key, NaN in a log decay and +Inf in a value, each in one (segment, head):
    each reaches that record and no other."""
    H, lens = 8, [130, 200, 64]
    k, v, beta, la, offs = _stream(lens, H, 1105)
    k[10, 1, 5] = float("nan")                      # segment 0, head 1: everything
    la[130 + 77, 2] = float("nan")                  # segment 1, head 2: ell and S, not P
    v[130 + 150, 3, 7] = float("inf")               # segment 1, head 3: S, not P or ell
    err = _err()
    pool = _build(k, v, beta, la, offs, [0, 1, 2], 3, err)
    say(f"[mfma nan/inf] H={H} lens={lens}")
    assert int(err.item()) == 0
    ref = _oracle(k, v, beta, la, offs)
    assert torch.any(torch.isnan(pool.S[0, 1])) and torch.any(torch.isnan(pool.P[0, 1]))
    assert torch.isnan(pool.S[1, 2]).any() and math.isnan(float(pool.log_scale[1, 2]))
    assert not torch.isfinite(pool.S[1, 3]).all()
    hit = {(0, 1), (1, 2), (1, 3)}
    for s in range(len(lens)):
        for h in range(H):
            if (s, h) in hit:
                continue
            assert torch.isfinite(pool.S[s, h]).all() and torch.isfinite(pool.P[s, h]).all()
            _check_record(pool, s, ref, s, h)
    # P does not depend on the decay or the values: those two records keep a correct P
    for s, h in ((1, 2), (1, 3)):
        assert torch.isfinite(pool.P[s, h]).all()
        assert rel_fro(np64(pool.P[s, h]), ref[1][s, h]) <= TOL[BF]
    assert math.isfinite(float(pool.log_scale[1, 3]))


def _expect_special(pool, slot, kind):
    """Record of an empty segment (identity) or of bad offsets (NaN), every head."""
    if kind == "nan":
        for t in (pool.S, pool.P, pool.log_scale):
            assert torch.all(torch.isnan(t[slot]))
    else:
        P = pool.P[slot]
        assert torch.all(pool.S[slot] == 0) and torch.all(pool.log_scale[slot] == 0)
        assert torch.equal(P, torch.eye(D, device="cuda").expand_as(P))


def test_mfma_build_unit_stream_mixed():
    """More (segment, head) units than workgroups (40 x 32 = 1280 units, five per
    workgroup, each running its units' chunks back to back): lengths around the chunk
    edges, empty segments, a decreasing offset pair and an end past the stream (NaN
    records, flag), an out-of-range slot (flag, nothing written).  Every record against
    the oracle on its own tokens; the slots nobody writes keep their canary bytes."""
    H = 32
    base = [0, 1, 63, 64, 65, 127, 128, 129, 200, 300]
    lens = [base[(7 * i) % len(base)] for i in range(40)]
    k, v, beta, la, offs = _stream(lens, H, 1107)
    N = int(offs[-1])
    offs = offs.copy()
    offs[21] = offs[20] - 10                  # segment 20: decreasing; segment 21 longer by 10
    offs[40] = N + 5                          # segment 39: past the stream
    nseg = 40
    num_slots = nseg + 4
    slots = np.random.default_rng(1107).permutation(num_slots)[:nseg].astype(np.int32)
    slots[13] = num_slots + 3                 # out of range
    err = _err()
    pool = _build(k, v, beta, la, offs, slots, num_slots, err)
    assert int(err.item()) == hp.EFLAG_BAD_OFFSETS | hp.EFLAG_SLOT_OUT_OF_RANGE
    unused = sorted(set(range(num_slots)) - set(int(x) for x in slots))
    for t in (pool.S, pool.P, pool.log_scale):
        assert torch.all(t[unused] == CANARY)
    kn, vn, bn, lan = np64(k), np64(v), np64(beta), np64(la)
    worst, counts = 0.0, {"stream": 0, "empty": 0, "nan": 0}
    for s in range(nseg):
        o0, o1 = int(offs[s]), int(offs[s + 1])
        if s == 13:
            continue
        if o1 < o0 or o1 > N:
            _expect_special(pool, slots[s], "nan")
            counts["nan"] += 1
        elif o1 == o0:
            _expect_special(pool, slots[s], "empty")
            counts["empty"] += 1
        else:
            ref = oracle.build_segments(oracle.GDN, kn[o0:o1], vn[o0:o1], lan[o0:o1], [0, o1 - o0], beta=bn[o0:o1])
            for h in range(H):
                worst = max(worst, max(_check_record(pool, slots[s], ref, 0, h)))
            counts["stream"] += 1
    say(f"[mfma unit stream] {nseg * H} units: {counts}, max err {worst:.2e}")
    assert counts["nan"] == 2 and counts["empty"] >= 3


def test_mfma_build_unit_stream_full_table():
    """4096 segments x 32 heads = 131072 units: 256 workgroups of exactly 512 units each
    (one per set-up thread).  Lengths 0-3 and 64-65 tokens; the empty segments' records
    checked in full, a sample of the others (among them every unit of set-up thread 511)
    against the oracle."""
    H, nseg = 32, 4096
    rng = np.random.default_rng(1108)
    lens = rng.choice([0, 1, 2, 3, 64, 65], size=nseg).tolist()
    k, v, beta, la, offs = _stream(lens, H, 1108)
    err = _err()
    pool = _build(k, v, beta, la, offs, np.arange(nseg, dtype=np.int32), nseg, err)
    assert int(err.item()) == 0
    empty = [s for s in range(nseg) if lens[s] == 0]
    _expect_special(pool, empty, "empty")
    units = list(range(511 * 256, 512 * 256, 7)) + rng.choice(nseg * H, size=120, replace=False).tolist()
    worst, n_checked = 0.0, 0
    for u in units:
        s, h = divmod(int(u), H)
        o0, o1 = int(offs[s]), int(offs[s + 1])
        if o1 == o0:
            continue
        ref = oracle.build_segments(oracle.GDN, np64(k[o0:o1, h:h + 1]), np64(v[o0:o1, h:h + 1]),
                                    np64(la[o0:o1, h:h + 1]), [0, o1 - o0], beta=np64(beta[o0:o1, h:h + 1]))
        e = record_errors(oracle.GDN, float(pool.log_scale[s, h]), np64(pool.P[s, h]), np64(pool.S[s, h]),
                          ref[0][0, 0], ref[1][0, 0], ref[2][0, 0])
        assert max(e) <= TOL[BF], (s, h, e)
        worst, n_checked = max(worst, max(e)), n_checked + 1
    say(f"[mfma unit table] {nseg * H} units, {len(empty)} empty segments, {n_checked} sampled: max err {worst:.2e}")


# ----------------------------------------------------------------------------- compose, d = 128

def _random_pool(nslots, H, seed):
    rng = np.random.default_rng(seed)
    q, _ = np.linalg.qr(rng.standard_normal((nslots, H, D, D)))
    pool = hp.Pool.allocate(hp.GDN, nslots, H, D, D, device="cuda", fill=0.0)
    pool.P.copy_(torch.from_numpy(q * rng.uniform(0.9, 1.0, size=(nslots, H, 1, D))).float())
    pool.S.copy_(torch.from_numpy(rng.standard_normal((nslots, H, D, D))).float())
    pool.log_scale.copy_(torch.from_numpy(rng.uniform(-0.5, 0.0, size=(nslots, H))).float())
    return pool


@pytest.mark.parametrize("num_req", [1, 17])
def test_compose_d128_bit_exact_indexing(num_req):
    """Chains of one record return its S and P bit for bit; a record with ell = -inf
    makes the output that record's S exactly.  num_req = 1 runs four workgroups per
    chain (32 units), 17 requests x 32 heads one workgroup per chain."""
    H, nslots = 32, 8
    pool = _random_pool(nslots, H, 1200 + num_req)
    pool.log_scale[6] = -math.inf
    rng = np.random.default_rng(1210 + num_req)
    for flip in (0, 1):
        chains = []
        for r in range(num_req):
            if (r + flip) % 2 == 0:
                chains.append([int(rng.integers(0, 6))])                    # one record
            else:
                chains.append([int(x) for x in rng.integers(0, 6, size=int(rng.integers(1, 5)))] + [6])
        offs = np.concatenate([[0], np.cumsum([len(c) for c in chains])]).astype(np.int64)
        flat = dev_i32(sum(chains, []))
        out_P = torch.empty((num_req, H, D, D), device="cuda")
        out_ell = torch.empty((num_req, H), device="cuda")
        err = _err()
        out = hp.compose_chain(pool, dev_i64(offs), flat, out_log_scale=out_ell, out_P=out_P, err_flag=err)
        torch.cuda.synchronize()
        say(f"[compose d128 bit-exact] requests={num_req} chains={chains[:4]}")
        assert int(err.item()) == 0
        for r, c in enumerate(chains):
            assert torch.equal(out[r], pool.S[c[-1]]), r
            if len(c) == 1:
                assert torch.equal(out_P[r], pool.P[c[0]]) and torch.equal(out_ell[r], pool.log_scale[c[0]])
            else:
                assert torch.all(out_ell[r] == -math.inf)
        # with an initial state the -inf record still forgets everything before it
        init = torch.randn((num_req, H, D, D), device="cuda")
        out = hp.compose_chain(pool, dev_i64(offs), flat, init_S=init)
        torch.cuda.synchronize()
        for r, c in enumerate(chains):
            if len(c) > 1:
                assert torch.equal(out[r], pool.S[6]), r


@pytest.mark.parametrize("num_req", [3, 17])
def test_compose_d128_out_of_range_slot_and_bad_offsets(num_req):
    """An out-of-range slot in one chain flags and NaN-fills that request only; the other
    requests equal a clean run bit for bit.  Decreasing chain offsets do the same."""
    H, nslots = 32, 6
    pool = _random_pool(nslots, H, 1300 + num_req)
    rng = np.random.default_rng(1310 + num_req)
    chains = [[int(x) for x in rng.integers(0, nslots, size=int(rng.integers(1, 6)))] for _ in range(num_req)]
    bad = list(chains)
    bad[1] = chains[1][:1] + [nslots + 3] + chains[1][1:]
    offs_b = np.concatenate([[0], np.cumsum([len(c) for c in bad])]).astype(np.int64)
    offs_c = np.concatenate([[0], np.cumsum([len(c) for c in chains])]).astype(np.int64)
    err = _err()
    ell = torch.empty((num_req, H), device="cuda")
    out = hp.compose_chain(pool, dev_i64(offs_b), dev_i32(sum(bad, [])), out_log_scale=ell, err_flag=err)
    clean = hp.compose_chain(pool, dev_i64(offs_c), dev_i32(sum(chains, [])))
    torch.cuda.synchronize()
    say(f"[compose d128 bad slot] requests={num_req}")
    assert int(err.item()) == hp.EFLAG_SLOT_OUT_OF_RANGE
    assert torch.all(torch.isnan(out[1])) and torch.all(torch.isnan(ell[1]))
    others = [r for r in range(num_req) if r != 1]
    assert torch.equal(out[others], clean[others])
    # decreasing offsets for request 1
    offs_d = offs_c.copy()
    offs_d[2] = offs_d[1] - 1                       # offs_c[1] >= 1: request 1 runs backwards
    err.zero_()
    out = hp.compose_chain(pool, dev_i64(offs_d), dev_i32(sum(chains, [])), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) & hp.EFLAG_BAD_OFFSETS
    assert torch.all(torch.isnan(out[1]))
    assert not torch.any(torch.isnan(out[0]))


@pytest.mark.parametrize("d", [128, 64])
def test_compose_operator_renormalised_below_fp32_range(d):
    """A chain of 40 records whose operators each shrink by about 1/50: the product
    (about 1e-68) lies far below the fp32 range, so the compose moves exact powers of
    two from P into ell; (out_ell, out_P) must still be the chain's operator
    T = e^ell P.  d = 128 runs the matrix-core compose, d = 64 the fp32 one."""
    from parity_util import composed_P_errors
    H, nslots, m = 4, 6, 40
    rng = np.random.default_rng(1400 + d)
    q, _ = np.linalg.qr(rng.standard_normal((nslots, H, d, d)))
    pool = hp.Pool.allocate(hp.GDN, nslots, H, d, d, device="cuda", fill=0.0)
    pool.P.copy_(torch.from_numpy(q * rng.uniform(0.01, 0.03, size=(nslots, H, 1, d))).float())
    pool.S.copy_(torch.from_numpy(rng.standard_normal((nslots, H, d, d))).float())
    pool.log_scale.copy_(torch.from_numpy(rng.uniform(-0.5, 0.0, size=(nslots, H))).float())
    flat = rng.integers(0, nslots, size=m).astype(np.int32)
    offs = np.array([0, m], dtype=np.int64)
    out_ell = torch.empty((1, H), device="cuda")
    out_P = torch.empty((1, H, d, d), device="cuda")
    out_S = hp.compose_chain(pool, dev_i64(offs), dev_i32(flat), out_log_scale=out_ell, out_P=out_P)
    torch.cuda.synchronize()
    rS, rell, rP = oracle.compose(hp.GDN, np64(pool.log_scale), np64(pool.P), np64(pool.S), offs, flat,
                                  want_P=True)
    worst = [0.0, 0.0, 0.0]
    for h in range(H):
        assert torch.isfinite(out_P[0, h]).all() and float(out_P[0, h].abs().max()) >= 2.0 ** -33
        eP, dl = composed_P_errors(out_ell[0, h], np64(out_P[0, h]), rell[0, h], rP[0, h])
        worst = [max(worst[0], eP), max(worst[1], dl), max(worst[2], rel_fro(np64(out_S[0, h]), rS[0, h]))]
    say(f"[compose renormalised d={d}] |P| product {np.abs(rP).max():.1e}: P err {worst[0]:.2e}, "
        f"ell err {worst[1]:.2e}, S err {worst[2]:.2e}")
    assert worst[0] <= 1e-4 and worst[1] <= 1e-4 and worst[2] <= 1e-4
