"""GPU parity of the KDA family (A_t = (I - beta k k^T) diag(alpha_t); record
ell = 0, P = T_C) against the fp64 oracle: every record's T_C and S, and the
chain of the segments' records composed against the recurrence over the
concatenated tokens (dense MFMA compose at d = 128, the fp32 compose at d = 64).

Gates log alpha = logsigmoid(z) / div per token and key channel: div = 16 as for
the diagonal family (T_C of a 2048-token segment falls below the fp32 range, so
T_C is compared on shorter segments and with div = 1600), and S, which stays in
range, at full length."""
import numpy as np
import pytest
import torch

import hybrid_prefill_amd as hp
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


def _inputs(lens, H, dk, dv, dtype, seed, div):
    offs = synth.offsets_from_lengths(lens)
    N = int(offs[-1])
    k = synth.keys(N, H, dk, dtype, seed, "cuda")
    v = synth.values(N, H, dv, dtype, seed + 1, "cuda")
    b = synth.write_gate(N, H, seed + 2, "cuda")
    la = synth.diagonal_log_gates(N, H, dk, seed + 3, div, "cuda")
    return offs, k, v, b, la


@pytest.mark.parametrize("cfg", [(2, 64, 64, torch.float32, 1e-4), (3, 128, 128, torch.bfloat16, 2e-2),
                                 (2, 128, 64, torch.float32, 1e-4)])
def test_kda_records_and_chain(cfg):
    H, dk, dv, dtype, tol = cfg
    lens = [130, 0, 1, 64, 65, 300]
    offs, k, v, b, la = _inputs(lens, H, dk, dv, dtype, 1700 + dk + dv, 1600.0)
    nseg = len(lens)
    slots = np.arange(nseg)[::-1].copy()
    pool = hp.Pool.allocate(hp.KDA, nseg, H, dk, dv, device="cuda", fill=12345.0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp.build_segment(hp.KDA, k, v, la, torch.as_tensor(offs).cuda(), pool,
                     torch.as_tensor(slots.astype(np.int32)).cuda(), beta=b, err_flag=err)
    out = hp.compose_chain(pool, torch.as_tensor(np.array([0, nseg], np.int64)).cuda(),
                           torch.as_tensor(slots.astype(np.int32)).cuda(), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    kn, vn, bn, lan = np64(k), np64(v), np64(b), np64(la)
    ell, P, S = oracle.build_segments(oracle.KDA, kn, vn, lan, offs, beta=bn)
    worst = [0.0, 0.0]
    for s in range(nseg):
        assert torch.all(pool.log_scale[slots[s]] == 0)
        for h in range(H):
            worst[0] = max(worst[0], rel_fro(np64(pool.P[slots[s], h]), P[s, h]))
            worst[1] = max(worst[1], rel_fro(np64(pool.S[slots[s], h]), S[s, h]))
    _, _, S_seq = oracle.build_segments(oracle.KDA, kn, vn, lan, [0, int(offs[-1])], beta=bn, want_P=False)
    wc = max(rel_fro(np64(out[0, h]), S_seq[0, h]) for h in range(H))
    say(f"[kda] H={H} dk={dk} dv={dv} {dtype}: T_C err {worst[0]:.2e}, S err {worst[1]:.2e}, "
        f"composed vs sequential {wc:.2e}")
    assert max(worst) <= tol and wc <= tol


def test_kda_long_segments_as_given_gates():
    """div = 16 (the diagonal family's gates), 2 x 2048 tokens, H=4, d=128, bf16: S of
    every record and the composed state (T_C underflows here, as it does in fp64 below
    the fp32 range; its product with the state is what the chain needs)."""
    H, d = 4, 128
    lens = [2048, 2048]
    offs, k, v, b, la = _inputs(lens, H, d, d, torch.bfloat16, 1750, 16.0)
    pool = hp.Pool.allocate(hp.KDA, 2, H, d, d, device="cuda")
    hp.build_segment(hp.KDA, k, v, la, torch.as_tensor(offs).cuda(), pool,
                     torch.arange(2, dtype=torch.int32, device="cuda"), beta=b)
    out = hp.compose_chain(pool, torch.as_tensor(np.array([0, 2], np.int64)).cuda(),
                           torch.arange(2, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    kn, vn, bn, lan = np64(k), np64(v), np64(b), np64(la)
    _, _, S = oracle.build_segments(oracle.KDA, kn, vn, lan, offs, beta=bn, want_P=False)
    _, _, S_seq = oracle.build_segments(oracle.KDA, kn, vn, lan, [0, 4096], beta=bn, want_P=False)
    eS = max(rel_fro(np64(pool.S[s, h]), S[s, h]) for s in range(2) for h in range(H))
    eC = max(rel_fro(np64(out[0, h]), S_seq[0, h]) for h in range(H))
    say(f"[kda long] S err {eS:.2e}, composed vs sequential {eC:.2e}")
    assert eS <= 2e-2 and eC <= 2e-2


@pytest.mark.parametrize("dtype,tol", [(torch.float32, 1e-4), (torch.bfloat16, 2e-2)])
def test_kda_strong_gates(dtype, tol):
    """Stretches where a few key channels decay by e^-20 per token (and one token that
    closes a channel by e^-200): at d = 128 the chunks that hold them are applied token
    by token inside the chunked kernel (a scaled key there would leave the fp32 range),
    the rest of each segment in chunk form; T_C, S and the composed chain against the
    oracle."""
    H, d = 2, 128
    lens = [300, 97, 32, 33]
    offs, k, v, b, la = _inputs(lens, H, d, d, dtype, 1790, 1600.0)
    la[40:120, :, :8] = -20.0
    la[250, 1, 100] = -200.0
    la[330:345, 0, 5] = -12.0
    nseg = len(lens)
    slots = np.arange(nseg, dtype=np.int32)
    pool = hp.Pool.allocate(hp.KDA, nseg, H, d, d, device="cuda", fill=777.0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp.build_segment(hp.KDA, k, v, la, torch.as_tensor(offs).cuda(), pool, torch.as_tensor(slots).cuda(),
                     beta=b, err_flag=err)
    out = hp.compose_chain(pool, torch.as_tensor(np.array([0, nseg], np.int64)).cuda(),
                           torch.as_tensor(slots).cuda(), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    kn, vn, bn, lan = np64(k), np64(v), np64(b), np64(la)
    _, P, S = oracle.build_segments(oracle.KDA, kn, vn, lan, offs, beta=bn)
    eT = max(rel_fro(np64(pool.P[s, h]), P[s, h]) for s in range(nseg) for h in range(H))
    eS = max(rel_fro(np64(pool.S[s, h]), S[s, h]) for s in range(nseg) for h in range(H))
    _, _, S_seq = oracle.build_segments(oracle.KDA, kn, vn, lan, [0, int(offs[-1])], beta=bn, want_P=False)
    eC = max(rel_fro(np64(out[0, h]), S_seq[0, h]) for h in range(H))
    say(f"[kda strong gates] {dtype}: T_C err {eT:.2e}, S err {eS:.2e}, composed vs sequential {eC:.2e}")
    assert eT <= tol and eS <= tol and eC <= tol


@pytest.mark.parametrize("d", [64, 128])
def test_kda_without_gates_or_beta(d):
    """log alpha and beta left out (NULL: no decay, beta = 1), bf16, one head, segments
    of 1, 40 and 33 tokens: the ungated delta rule, against the oracle with zero gates
    and unit beta."""
    H = 1
    lens = [1, 40, 33]
    offs = synth.offsets_from_lengths(lens)
    N = int(offs[-1])
    k = synth.keys(N, H, d, torch.bfloat16, 1830 + d, "cuda")
    v = synth.values(N, H, d, torch.bfloat16, 1831 + d, "cuda")
    nseg = len(lens)
    pool = hp.Pool.allocate(hp.KDA, nseg, H, d, d, device="cuda", fill=55.0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp.build_segment(hp.KDA, k, v, None, torch.as_tensor(offs).cuda(), pool,
                     torch.arange(nseg, dtype=torch.int32, device="cuda"), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    kn, vn = np64(k), np64(v)
    _, P, S = oracle.build_segments(oracle.KDA, kn, vn, np.zeros((N, H, d)), offs)
    eT = max(rel_fro(np64(pool.P[s, 0]), P[s, 0]) for s in range(nseg))
    eS = max(rel_fro(np64(pool.S[s, 0]), S[s, 0]) for s in range(nseg))
    say(f"[kda no gates] d={d}: T_C err {eT:.2e}, S err {eS:.2e}")
    assert eT <= 2e-2 and eS <= 2e-2


def test_kda_error_paths():
    """d = 128 (chunk kernel): a slot out of range raises its flag and leaves the pool
    untouched, decreasing offsets raise theirs and fill that record with NaN, and the
    valid segments of the same call still match the oracle."""
    H, d = 2, 128
    lens = [70, 40, 33]
    offs, k, v, b, la = _inputs(lens, H, d, d, torch.bfloat16, 1860, 16.0)
    bad_offs = offs.copy()
    bad_offs[2] = bad_offs[1] - 5                 # segment 1 ends before it starts
    pool = hp.Pool.allocate(hp.KDA, 4, H, d, d, device="cuda", fill=9.0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    slots = torch.tensor([0, 1, 7], dtype=torch.int32, device="cuda")   # 7: out of range
    hp.build_segment(hp.KDA, k, v, la, torch.as_tensor(bad_offs).cuda(), pool, slots, beta=b, err_flag=err)
    torch.cuda.synchronize()
    flags = int(err.item())
    assert flags & hp.EFLAG_SLOT_OUT_OF_RANGE and flags & hp.EFLAG_BAD_OFFSETS
    assert torch.isnan(pool.S[1]).all() and torch.isnan(pool.P[1]).all()
    assert torch.all(pool.S[2:] == 9.0) and torch.all(pool.P[2:] == 9.0)
    kn, vn, bn, lan = np64(k), np64(v), np64(b), np64(la)
    _, P, S = oracle.build_segments(oracle.KDA, kn, vn, lan, offs[:2], beta=bn)
    e = max(max(rel_fro(np64(pool.P[0, h]), P[0, h]), rel_fro(np64(pool.S[0, h]), S[0, h])) for h in range(H))
    say(f"[kda errors] flags {flags:#x}, valid segment err {e:.2e}")
    assert e <= 2e-2
