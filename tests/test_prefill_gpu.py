"""GPU parity of the chunked prefill forward (in-segment outputs o_t = S_t^T q_t)
and its record side-outputs, through hypic_prefill_segment, against the fp64 oracle.

Bars: outputs and records within relative Frobenius error 2e-2 per (segment, head)
(bf16 inputs); the same outputs whether or not the records are built (bit for bit:
the record columns run on waves of their own); records equal to what
hypic_build_segment writes within the same bound; pool indexing bit-exact
(canaries, error flags).
"""
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
OCANARY = 12288.0          # exact in bf16 and fp32
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
    q = synth.keys(int(st.seg_offsets[-1]), H, D, BF, seed * 10 + 7, "cuda")    # unit-norm queries
    return st, q, np.asarray(st.seg_offsets, dtype=np.int64)


def _oracle(st, q, offs):
    return oracle.forward(oracle.GDN, np64(st.k), np64(st.v), np64(q), np64(st.log_alpha), offs,
                          beta=np64(st.beta))


def _output_errors(o_gpu, o_ref, offs):
    """max over (segment, head) of the relative Frobenius error of that segment's outputs."""
    worst = 0.0
    og, orf = np64(o_gpu), o_ref
    for s in range(len(offs) - 1):
        if offs[s + 1] == offs[s]:
            continue
        sl = slice(int(offs[s]), int(offs[s + 1]))
        for h in range(og.shape[1]):
            worst = max(worst, rel_fro(og[sl, h], orf[sl, h]))
    return worst


def _record_errors(pool, slots, ref, H):
    _, ell_r, P_r, S_r = ref
    worst = [0.0, 0.0, 0.0]
    for s, sl in enumerate(slots):
        for h in range(H):
            e = record_errors(oracle.GDN, float(pool.log_scale[sl, h]), np64(pool.P[sl, h]), np64(pool.S[sl, h]),
                              ell_r[s, h], P_r[s, h], S_r[s, h])
            worst = [max(a, b) for a, b in zip(worst, e)]
    return worst


@pytest.mark.parametrize("variant", ["as_given", "none"])
def test_prefill_32_heads_16x2048(variant):
    """H=32, d=128, bf16, one 32768-token request in 16 x 2048 segments: every output
    and every record against one batched oracle run; outputs identical with and
    without the records; records against hypic_build_segment's."""
    H, lens = 32, [2048] * 16
    st, q, offs = _stream(lens, H, 331, 0.1 if variant == "as_given" else 0.0)
    nseg = len(lens)
    slots = np.random.default_rng(5).permutation(nseg + 2)[:nseg].astype(np.int32)
    pool = hp.Pool.allocate(hp.GDN, nseg + 2, H, D, D, device="cuda", fill=CANARY)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o_rec = hp.prefill_segment(hp.GDN, st.k, st.v, q, st.log_alpha, dev_i64(offs), beta=st.beta, pool=pool,
                               dst_slots=dev_i32(slots), err_flag=err)
    o_fwd = hp.prefill_segment(hp.GDN, st.k, st.v, q, st.log_alpha, dev_i64(offs), beta=st.beta, err_flag=err)
    pool_b = hp.Pool.allocate(hp.GDN, nseg + 2, H, D, D, device="cuda", fill=CANARY)
    hp.build_segment(hp.GDN, st.k, st.v, st.log_alpha, dev_i64(offs), pool_b, dev_i32(slots), beta=st.beta,
                     err_flag=err)
    # no outputs: the records alone, exactly as hypic_build_segment writes them
    pool_r = hp.Pool.allocate(hp.GDN, nseg + 2, H, D, D, device="cuda", fill=CANARY)
    assert hp.prefill_segment(hp.GDN, st.k, st.v, None, st.log_alpha, dev_i64(offs), beta=st.beta, pool=pool_r,
                              dst_slots=dev_i32(slots), outputs=False, err_flag=err) is None
    torch.cuda.synchronize()
    for t_r, t_b in ((pool_r.S, pool_b.S), (pool_r.P, pool_b.P), (pool_r.log_scale, pool_b.log_scale)):
        assert torch.equal(t_r, t_b)
    assert int(err.item()) == 0
    say(f"[prefill 32x128 {variant}] 16 x 2048 tokens")
    assert torch.equal(o_rec, o_fwd)
    unused = sorted(set(range(nseg + 2)) - set(slots.tolist()))
    for t in (pool.S, pool.P, pool.log_scale):
        assert torch.all(t[unused] == CANARY)
    ref = _oracle(st, q, offs)
    eo = _output_errors(o_fwd, ref[0], offs)
    er = _record_errors(pool, slots, ref, H)
    eb = max(rel_fro(np64(pool.S), np64(pool_b.S)), rel_fro(np64(pool.P), np64(pool_b.P)))
    say(f"   outputs: max err {eo:.2e};  records: S {er[0]:.2e} T {er[1]:.2e} ell {er[2]:.2e};  "
        f"vs build_segment's records {eb:.2e}")
    assert eo <= TOL[BF] and max(er) <= TOL[BF]
    assert torch.equal(pool.log_scale, pool_b.log_scale)
    assert eb <= 1e-2


@pytest.mark.parametrize("scale", [0.1, 0.0])
def test_prefill_segments_past_2048(scale):
    """Segments of up to 100 chunks (the decay scale carried beside the state and folded
    into it, over many cycles): every output and record against the oracle."""
    H, lens = 4, [4200, 64, 6100, 1]
    st, q, offs = _stream(lens, H, 371 + int(scale * 10), scale)
    nseg = len(lens)
    slots = np.arange(nseg, dtype=np.int32)
    pool = hp.Pool.allocate(hp.GDN, nseg, H, D, D, device="cuda", fill=CANARY)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = hp.prefill_segment(hp.GDN, st.k, st.v, q, st.log_alpha, dev_i64(offs), beta=st.beta, pool=pool,
                             dst_slots=dev_i32(slots), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = _oracle(st, q, offs)
    eo = _output_errors(out, ref[0], offs)
    er = _record_errors(pool, slots, ref, H)
    say(f"[prefill long] decay {scale} lens {lens}: outputs {eo:.2e}, records {max(er):.2e}")
    assert eo <= TOL[BF] and max(er) <= TOL[BF]


EDGE_LENS = [0, 1, 63, 64, 65, 127, 129, 200]


@pytest.mark.parametrize("scale", [0.1, 0.0])
@pytest.mark.parametrize("out_dtype", [torch.float32, BF])
def test_prefill_edge_lengths(scale, out_dtype):
    """Empty, one-token, partial-chunk and multi-chunk segments in one stream; outputs
    in fp32 and bf16; the outputs of tokens outside every segment are never written."""
    H = 4
    st, q, offs = _stream(EDGE_LENS, H, 341 + int(scale * 10), scale)
    N = int(offs[-1])
    pad = 5                                         # tokens after the last segment
    k = torch.cat([st.k, st.k[:pad]]); v = torch.cat([st.v, st.v[:pad]]); qq = torch.cat([q, q[:pad]])
    la = torch.cat([st.log_alpha, st.log_alpha[:pad]]); b = torch.cat([st.beta, st.beta[:pad]])
    out = torch.full((N + pad, H, D), OCANARY, dtype=out_dtype, device="cuda")
    pool = hp.Pool.allocate(hp.GDN, len(EDGE_LENS), H, D, D, device="cuda", fill=CANARY)
    slots = np.arange(len(EDGE_LENS), dtype=np.int32)[::-1].copy()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp.prefill_segment(hp.GDN, k, v, qq, la, dev_i64(offs), beta=b, out=out, pool=pool, dst_slots=dev_i32(slots),
                       err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.all(out[N:] == OCANARY)
    ref = _oracle(st, q, offs)
    eo = _output_errors(out[:N], ref[0], offs)
    er = _record_errors(pool, slots, ref, H)
    say(f"[prefill edges] decay {scale} out {out_dtype}: outputs {eo:.2e}, records {max(er):.2e}")
    assert eo <= TOL[BF] and max(er) <= TOL[BF]
    # the empty segment's record is the identity record
    e = EDGE_LENS.index(0)
    assert torch.all(pool.S[slots[e]] == 0) and torch.all(pool.log_scale[slots[e]] == 0)
    assert torch.equal(pool.P[slots[e]], torch.eye(D, device="cuda").expand(H, D, D))


def test_prefill_strided_views():
    """q, k, v as head-interleaved views of one [N, H, 3, d] projection, and the output
    written into a wider buffer: the strides go through unchanged."""
    H, lens = 4, [300, 77]
    offs = synth.offsets_from_lengths(lens)
    N = int(offs[-1])
    qkv = torch.randn((N, H, 3, D), device="cuda").to(BF)
    qkv[:, :, 1] = synth.keys(N, H, D, BF, 351, "cuda")
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    b = synth.write_gate(N, H, 352, "cuda")
    la = synth.gdn_log_decay(N, H, 353, 0.1, "cuda")
    wide = torch.zeros((N, H, 2 * D), device="cuda")
    out = wide[:, :, :D]
    hp.prefill_segment(hp.GDN, k, v, q, la, dev_i64(offs), beta=b, out=out)
    torch.cuda.synchronize()
    ref = oracle.forward(oracle.GDN, np64(k), np64(v), np64(q), np64(la), offs, beta=np64(b))
    eo = _output_errors(out, ref[0], offs)
    say(f"[prefill strided] outputs {eo:.2e}")
    assert eo <= TOL[BF] and torch.all(wide[:, :, D:] == 0)


def test_prefill_error_paths():
    """An out-of-range slot flags, and nothing of that segment is written (neither its
    record nor its outputs); bad offsets flag, NaN-fill that record and write none of
    its outputs.  The other segment is computed normally in both cases."""
    H, lens = 4, [200, 300]
    st, q, offs = _stream(lens, H, 361)
    N = int(offs[-1])
    pool = hp.Pool.allocate(hp.GDN, 3, H, D, D, device="cuda", fill=CANARY)
    out = torch.full((N, H, D), OCANARY, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp.prefill_segment(hp.GDN, st.k, st.v, q, st.log_alpha, dev_i64(offs), beta=st.beta, out=out, pool=pool,
                       dst_slots=dev_i32([1, 9]), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == hp.EFLAG_SLOT_OUT_OF_RANGE
    for t in (pool.S, pool.P, pool.log_scale):
        assert torch.all(t[[0, 2]] == CANARY)
    ref = _oracle(st, q, offs)
    assert _output_errors(out[:200], ref[0][:200], [0, 200]) <= TOL[BF]
    assert torch.all(out[200:] == OCANARY)
    assert max(_record_errors(pool, [1], ref, H)) <= TOL[BF]
    err.zero_()
    out.fill_(OCANARY)
    pool = hp.Pool.allocate(hp.GDN, 3, H, D, D, device="cuda", fill=CANARY)
    hp.prefill_segment(hp.GDN, st.k, st.v, q, st.log_alpha, dev_i64([0, 200, N + 3]), beta=st.beta, out=out,
                       pool=pool, dst_slots=dev_i32([0, 2]), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == hp.EFLAG_BAD_OFFSETS
    for t in (pool.S, pool.P, pool.log_scale):
        assert torch.all(torch.isnan(t[2])) and torch.all(t[1] == CANARY)
    assert torch.all(out[200:] == OCANARY)
    assert _output_errors(out[:200], ref[0][:200], [0, 200]) <= TOL[BF]
    assert max(_record_errors(pool, [0], ref, H)) <= TOL[BF]
