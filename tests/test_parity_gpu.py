"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: relative Frobenius error <= 1e-4 for fp32 inputs and <= 2e-2 for
bf16 inputs, per (segment or request, head); pool indexing bit-exact.
Every input is seeded and synthetic (module ``synth``).
"""
import math

import numpy as np
import pytest
import torch

import hybrid_prefill_amd as hp
import oracle
import synth
from oracle import rel_fro
from parity_util import (TOL, composed_P_errors, dev_i32, dev_i64, full_log_alpha, np64, oracle_unit,
                         record_errors, say)

pytestmark = pytest.mark.gpu
CANARY = 12345.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hp.lib()
    yield
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------- inputs

def make_inputs(family, lens, H, dk, dv, dtype, seed, variant="as_given"):
    """Seeded stream for one family; variant 'weak' weakens the decay so the prefix matters."""
    offs = synth.offsets_from_lengths(lens)
    N = int(offs[-1])
    k = synth.keys(N, H, dk, dtype, seed * 10 + 1, "cuda")
    v = synth.values(N, H, dv, dtype, seed * 10 + 2, "cuda")
    beta = None
    if family == hp.GDN:
        beta = synth.write_gate(N, H, seed * 10 + 3, "cuda")
        scale = {"as_given": 0.1, "weak": 0.001, "none": 0.0}[variant]
        la = synth.gdn_log_decay(N, H, seed * 10 + 4, scale, "cuda")
    elif family == hp.SCALAR:
        lo, hi = (0.9, 0.999) if variant == "as_given" else (0.9995, 0.99995)
        la = synth.scalar_log_gamma(H, seed * 10 + 4, lo, hi, "cuda")
    else:
        div = 16.0 if variant == "as_given" else 1600.0
        la = synth.diagonal_log_gates(N, H, dk, seed * 10 + 4, div, "cuda")
    return dict(k=k, v=v, beta=beta, la=la, offs=offs, N=N)


def host_inputs(family, inp, H):
    return (np64(inp["k"]), np64(inp["v"]), full_log_alpha(family, inp["la"], inp["N"], H),
            None if inp["beta"] is None else np64(inp["beta"]))


def gpu_build(family, inp, H, dk, dv, slots, num_slots, err=None):
    pool = hp.Pool.allocate(family, num_slots, H, dk, dv, device="cuda", fill=CANARY)
    err = torch.zeros(1, dtype=torch.int32, device="cuda") if err is None else err
    hp.build_segment(family, inp["k"], inp["v"], inp["la"], dev_i64(inp["offs"]), pool, dev_i32(slots),
                     beta=inp["beta"], err_flag=err)
    return pool, err


# ----------------------------------------------------------------------------- core check

def check_build_compose(family, lens, H, dk, dv, dtype, seed, variant="as_given", label=""):
    """Build every segment into permuted slots, compose the whole chain, compare with the oracle.

    Every (segment, head) record is checked against one batched oracle build of the
    same bytes, and every head's composed state against the sequential recurrence over
    the concatenation.  For GDN the composed operator is checked twice: against the
    fp64 product of the GPU's own records (the compose arithmetic, 1e-4), and against
    the operator of the whole token stream, whose error is the records' own error
    compounded over the chain: at most sqrt(m) times the per-record tolerance for m
    records with independent rounding.
    """
    tol = TOL[dtype]
    nseg = len(lens)
    num_slots = nseg + 3
    slots = np.random.default_rng(seed).permutation(num_slots)[:nseg].astype(np.int32)
    inp = make_inputs(family, lens, H, dk, dv, dtype, seed, variant)
    say(f"[{label}] family={family} H={H} dk={dk} dv={dv} {dtype} lens={lens[:6]}{'...' if nseg > 6 else ''}")
    pool, err = gpu_build(family, inp, H, dk, dv, slots, num_slots)
    out_ell = torch.empty((1, H, dk) if family == hp.DIAGONAL else (1, H), device="cuda")
    out_P = torch.empty((1, H, dk, dk), device="cuda") if family == hp.GDN else None
    out_S = hp.compose_chain(pool, dev_i64([0, nseg]), dev_i32(slots), out_log_scale=out_ell,
                             out_P=out_P, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    k, v, la, b = host_inputs(family, inp, H)
    offs = inp["offs"]
    # canary slots untouched, bit for bit
    unused = sorted(set(range(num_slots)) - set(slots.tolist()))
    assert torch.all(pool.S[unused] == CANARY)
    assert torch.all(pool.log_scale[unused] == CANARY)
    if pool.P is not None:
        assert torch.all(pool.P[unused] == CANARY)
    # every record, one batched oracle call
    ell_r, P_r, S_r = oracle.build_segments(family, k, v, la, offs, beta=b)
    g_ell = np64(pool.log_scale[slots])
    g_P = None if pool.P is None else np64(pool.P[slots])
    g_S = np64(pool.S[slots])
    worst = [0.0, 0.0, 0.0]
    for s in range(nseg):
        for h in range(H):
            e = record_errors(family, g_ell[s, h], None if g_P is None else g_P[s, h], g_S[s, h],
                              ell_r[s, h], None if P_r is None else P_r[s, h], S_r[s, h])
            worst = [max(a, c) for a, c in zip(worst, e)]
    say(f"   {nseg * H} records: max err S {worst[0]:.2e}  T {worst[1]:.2e}  ell {worst[2]:.2e}  (tol {tol:g})")
    assert worst[0] <= tol and worst[1] <= tol and worst[2] <= tol
    # every head's composed state against the recurrence over the whole request
    ell_q, P_q, S_q = oracle.build_segments(family, k, v, la, [0, inp["N"]], beta=b)
    worst_seq = worst_ell = worst_Pc = worst_Pseq = naive = 0.0
    if family == hp.GDN:
        _, ell_c, Pc = oracle.compose(family, np64(pool.log_scale), np64(pool.P), np64(pool.S), [0, nseg], slots,
                                      want_P=True)
    for h in range(H):
        worst_seq = max(worst_seq, rel_fro(np64(out_S[0, h]), S_q[0, h]))
        naive = max(naive, rel_fro(g_S[:, h].sum(axis=0), S_q[0, h]))
        if family == hp.GDN:
            # (ell, P) of the composed operator, up to the power of two the compose may
            # have moved between them
            eP, _ = composed_P_errors(out_ell[0, h], np64(out_P[0, h]), ell_c[0, h], Pc[0, h])
            worst_Pc = max(worst_Pc, eP)
            eP, dl = composed_P_errors(out_ell[0, h], np64(out_P[0, h]), ell_q[0, h], P_q[0, h])
            worst_Pseq = max(worst_Pseq, eP)
            worst_ell = max(worst_ell, dl)
        else:
            worst_ell = max(worst_ell, float(np.max(np.abs(np64(out_ell[0, h]) - ell_q[0, h]))))
    tol_chain = tol * math.sqrt(nseg)
    say(f"   composed vs sequential ({H} heads): S err {worst_seq:.2e}, ell err {worst_ell:.2e}; naive end-state "
        f"sum err {naive:.2e}" + (f"; composed P vs product of records {worst_Pc:.2e}, vs whole stream "
                                  f"{worst_Pseq:.2e} (tol {tol_chain:.2g})" if family == hp.GDN else ""))
    assert worst_seq <= tol and worst_ell <= tol
    assert worst_Pc <= 1e-4
    assert worst_Pseq <= tol_chain
    return naive


# ----------------------------------------------------------------------------- configs

def test_gdn_fp32_two_segments_of_256():
    """GDN, 1 head, d_k=d_v=64, fp32, 2 x 256 tokens: build both, compose, vs sequential."""
    check_build_compose(hp.GDN, [256, 256], 1, 64, 64, torch.float32, 101, label="gdn-1x64-fp32")


@pytest.mark.parametrize("variant", ["weak", "none"])
def test_gdn_fp32_two_segments_sensitivity(variant):
    """Same shapes with weak (or no) decay: the prefix matters, naive addition must fail."""
    naive = check_build_compose(hp.GDN, [256, 256], 1, 64, 64, torch.float32, 101, variant,
                                label=f"gdn-1x64-fp32-{variant}")
    assert naive > 1e-4


@pytest.mark.parametrize("family", [hp.SCALAR, hp.DIAGONAL])
@pytest.mark.parametrize("variant", ["as_given", "weak"])
def test_scalar_diagonal_16_heads_8x2048(family, variant):
    """Scalar and diagonal families, H=16, d=128, bf16, 8 segments x 2048 tokens, chain of 8."""
    naive = check_build_compose(family, [2048] * 8, 16, 128, 128, torch.bfloat16, 201, variant,
                                label=f"sd-{family}-{variant}")
    if variant == "weak":
        assert naive > 2e-2


def test_scalar_mixed_lengths_128_units():
    """Scalar family, H=16, d=128, bf16, 8 segments of mixed length (empty, one
    token, partial chunks, odd and even chunk counts): 128 units take the value
    split whose compute waves read each chunk's operands one chunk ahead."""
    check_build_compose(hp.SCALAR, [2048, 1, 65, 0, 129, 700, 64, 1000], 16, 128, 128, torch.bfloat16, 211,
                        "weak", label="scalar-mixed-128-units")


@pytest.mark.parametrize("H,lens", [(4, [4200, 2049, 64, 4160]),                          # 16 units: 4 splits
                                    (16, [4200, 2048, 2049, 1, 0, 4160, 130, 6200]),      # 128 units: 2 splits
                                    (32, [4200, 2100, 64, 2049, 1, 0, 130, 2500])])       # 256 units: 1 split
def test_scalar_segments_past_one_weight_table(H, lens):
    """Scalar family on the matrix cores with segments longer than one 2048-token weight
    table (the tables after the first and the state carried between them), for each
    value split of the grid (4, 2 and 1 workgroups per (segment, head)); weak gates, so
    the first table's tokens still count at the end of the segment."""
    check_build_compose(hp.SCALAR, lens, H, 128, 128, torch.bfloat16, 221 + H, "weak",
                        label=f"scalar-long-{H}x{len(lens)}")


@pytest.mark.parametrize("family,variant", [(hp.GDN, "as_given"), (hp.GDN, "none"), (hp.DIAGONAL, "weak")])
def test_gdn_diagonal_segments_past_2048(family, variant):
    """GDN and diagonal builds on the matrix cores over segments of up to 100 chunks
    (the chunk-parity buffers, and for GDN the decay scale carried beside the state and
    folded into it, over many cycles), composed into one chain."""
    check_build_compose(family, [4200, 64, 6100, 1, 2049], 4, 128, 128, torch.bfloat16, 231 + family, variant,
                        label=f"long-{family}-{variant}")


@pytest.mark.parametrize("variant", ["as_given", "none"])
def test_gdn_32_heads_16x2048(variant):
    """GDN H=32, d=128, bf16, one 32768-token request in 16 x 2048 segments: all 512
    records and all 32 composed heads against one batched oracle run."""
    check_build_compose(hp.GDN, [2048] * 16, 32, 128, 128, torch.bfloat16, 301, variant,
                        label=f"gdn-32x128-{variant}")


# ----------------------------------------------------------------------------- edge cases

EDGE_LENS = [0, 1, 63, 64, 65, 127, 129, 200]


@pytest.mark.parametrize("family", [hp.GDN, hp.SCALAR, hp.DIAGONAL])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_edge_lengths(family, dtype, dims):
    dk, dv = dims
    variant = "none" if family == hp.GDN else "weak"
    check_build_compose(family, EDGE_LENS, 2, dk, dv, dtype, 401 + family, variant,
                        label=f"edge-{family}-{dk}x{dv}")


def test_special_gdn_inputs():
    """beta = 0 (nothing written), log alpha = 0 (DeltaNet), a repeated key with beta = 1."""
    H, d, n = 2, 64, 130
    inp = make_inputs(hp.GDN, [n], H, d, d, torch.float32, 501)
    inp["beta"] = torch.zeros_like(inp["beta"])
    pool, err = gpu_build(hp.GDN, inp, H, d, d, [0], 1)
    torch.cuda.synchronize()
    assert torch.all(pool.S == 0) and int(err.item()) == 0
    eye = torch.eye(d, device="cuda").expand(1, H, d, d)
    assert torch.equal(pool.P, eye)
    ref = np64(inp["la"]).sum(axis=0)
    assert np.max(np.abs(np64(pool.log_scale[0]) - ref)) < 1e-4
    # repeated key, beta = 1, no decay: the last value overwrites
    inp = make_inputs(hp.GDN, [n], H, d, d, torch.float32, 502, "none")
    inp["k"][:] = inp["k"][0:1]
    inp["beta"] = torch.ones_like(inp["beta"])
    pool, err = gpu_build(hp.GDN, inp, H, d, d, [0], 1)
    torch.cuda.synchronize()
    for h in range(H):
        ref = np.outer(np64(inp["k"][0, h]), np64(inp["v"][n - 1, h]))
        assert rel_fro(np64(pool.S[0, h]), ref) < 1e-4


@pytest.mark.parametrize("family", [hp.GDN, hp.SCALAR, hp.DIAGONAL, hp.KDA])
@pytest.mark.parametrize("layout", ["fused", "kv_offset", "gate_offset"])
def test_build_strided_views(family, layout):
    """k and v as head-interleaved views of one [N, H, 3, d + 8] projection buffer, beta and
    the decay as views of wider buffers (d = 128, bf16).  'fused': every row 16-byte
    aligned with strides in whole 16-byte units, the layout the matrix-core builds take;
    'kv_offset': k and v rows start one element in, so none is 16-byte aligned and the
    GDN, scalar and diagonal builds go to the generic kernel; 'gate_offset': only the
    gate views start one element in (for the diagonal family that alone sends the build
    to the generic kernel).  Every record is compared with the oracle on the same values."""
    H, d = 3, 128
    lens = [200, 0, 77, 64, 129]
    offs = synth.offsets_from_lengths(lens)
    N, nseg = int(offs[-1]), len(lens)
    seed = 2300 + 10 * [hp.GDN, hp.SCALAR, hp.DIAGONAL, hp.KDA].index(family)
    kv_sh = 1 if layout == "kv_offset" else 0
    g_sh = 1 if layout == "gate_offset" else 0
    proj = torch.zeros((N, H, 3, d + 8), dtype=torch.bfloat16, device="cuda")
    k = proj[:, :, 1, kv_sh:kv_sh + d]
    v = proj[:, :, 2, kv_sh:kv_sh + d]
    k.copy_(synth.keys(N, H, d, torch.bfloat16, seed + 1, "cuda"))
    v.copy_(synth.values(N, H, d, torch.bfloat16, seed + 2, "cuda"))
    beta = None
    if family in (hp.GDN, hp.KDA):
        beta = torch.zeros((N, H, 3), device="cuda")[:, :, 1 + g_sh]
        beta.copy_(synth.write_gate(N, H, seed + 3, "cuda"))
    if family == hp.GDN:
        la = torch.zeros((N, H, 3), device="cuda")[:, :, g_sh]
        la.copy_(synth.gdn_log_decay(N, H, seed + 4, 0.1, "cuda"))
    elif family == hp.SCALAR:
        la = torch.zeros((H, 3), device="cuda")[:, 1 + g_sh]
        la.copy_(synth.scalar_log_gamma(H, seed + 4, 0.9, 0.999, "cuda"))
    else:
        la = torch.zeros((N, H, d + 8), device="cuda")[:, :, g_sh:g_sh + d]
        la.copy_(synth.diagonal_log_gates(N, H, d, seed + 4, 1600.0 if family == hp.KDA else 16.0, "cuda"))
    assert not k.is_contiguous() and not la.is_contiguous()
    assert beta is None or not beta.is_contiguous()
    slots = np.arange(nseg)[::-1].copy()
    pool = hp.Pool.allocate(family, nseg, H, d, d, device="cuda", fill=CANARY)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp.build_segment(family, k, v, la, dev_i64(offs), pool, dev_i32(slots), beta=beta, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    kn, vn = np64(k), np64(v)
    ell_r, P_r, S_r = oracle.build_segments(family, kn, vn, full_log_alpha(family, la, N, H), offs,
                                            beta=None if beta is None else np64(beta))
    g_ell, g_S = np64(pool.log_scale[slots]), np64(pool.S[slots])
    g_P = None if pool.P is None else np64(pool.P[slots])
    worst = [0.0, 0.0, 0.0]
    for s in range(nseg):
        for h in range(H):
            if family == hp.KDA:
                # ell = 0 and P = T_C for this family
                e = (rel_fro(g_S[s, h], S_r[s, h]), rel_fro(g_P[s, h], P_r[s, h]), float(np.max(np.abs(g_ell[s, h]))))
            else:
                e = record_errors(family, g_ell[s, h], None if g_P is None else g_P[s, h], g_S[s, h],
                                  ell_r[s, h], None if P_r is None else P_r[s, h], S_r[s, h])
            worst = [max(a, c) for a, c in zip(worst, e)]
    say(f"[strided {layout}] family={family}: max err S {worst[0]:.2e}  T {worst[1]:.2e}  ell {worst[2]:.2e}")
    assert max(worst) <= TOL[torch.bfloat16]


# ----------------------------------------------------------------------------- pool indexing / errors

def _gdn_pool(num_slots=6, H=2, d=64, seed=601):
    lens = [70] * num_slots
    inp = make_inputs(hp.GDN, lens, H, d, d, torch.float32, seed, "weak")
    pool, err = gpu_build(hp.GDN, inp, H, d, d, list(range(num_slots)), num_slots)
    torch.cuda.synchronize()
    return pool


def test_compose_indexing_bit_exact():
    pool = _gdn_pool()
    # chains of length 1 from a zero start return the slot's S bit for bit; repeats are fine
    chains = [[3], [0], [5], [3]]
    offs = np.concatenate([[0], np.cumsum([len(c) for c in chains])])
    out = hp.compose_chain(pool, dev_i64(offs), dev_i32(sum(chains, [])))
    torch.cuda.synchronize()
    for r, c in enumerate(chains):
        assert torch.equal(out[r], pool.S[c[0]])
    # a record with ell = -inf forgets everything before it: output == its S exactly
    pool.log_scale[4] = -math.inf
    out = hp.compose_chain(pool, dev_i64([0, 3]), dev_i32([1, 2, 4]))
    torch.cuda.synchronize()
    assert torch.equal(out[0], pool.S[4])
    # empty chain: the init state comes back unchanged
    init = torch.randn((2, 2, 64, 64), device="cuda")
    out = hp.compose_chain(pool, dev_i64([0, 0, 1]), dev_i32([2]), init_S=init)
    torch.cuda.synchronize()
    assert torch.equal(out[0], init[0])


@pytest.mark.parametrize("num_req", [1, 16, 17])
def test_compose_d128_chain_paths(num_req):
    """d=128 compose on synthetic records, against the oracle: up to 16 x 32 chains run four
    workgroups per chain (one per 32-column slice of the state), more run one per chain.
    Chains of length 16, 0 and 1 and random ones, with and without an initial state, and
    the composed operator."""
    H, d, nslots = 32, 128, 12
    rng = np.random.default_rng(900 + num_req)
    q, _ = np.linalg.qr(rng.standard_normal((nslots, H, d, d)))
    P = q * rng.uniform(0.9, 1.0, size=(nslots, H, 1, d))     # contractions: chains stay bounded
    S = rng.standard_normal((nslots, H, d, d))
    ell = rng.uniform(-0.5, 0.0, size=(nslots, H))
    pool = hp.Pool.allocate(hp.GDN, nslots, H, d, d, device="cuda", fill=0.0)
    pool.P.copy_(torch.from_numpy(P).float())
    pool.S.copy_(torch.from_numpy(S).float())
    pool.log_scale.copy_(torch.from_numpy(ell).float())
    lens = [int(x) for x in rng.integers(0, 17, size=num_req)]
    lens[0] = 16
    if num_req > 2:
        lens[1], lens[2] = 0, 1
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    flat = rng.integers(0, nslots, size=int(offs[-1])).astype(np.int32)
    heads = [0, 13, 31]
    for with_init in (False, True):
        init = torch.randn((num_req, H, d, d), device="cuda") if with_init else None
        out_ell = torch.empty((num_req, H), device="cuda")
        out_P = torch.empty((num_req, H, d, d), device="cuda")
        out_S = hp.compose_chain(pool, dev_i64(offs), dev_i32(flat), init_S=init, out_log_scale=out_ell,
                                 out_P=out_P)
        torch.cuda.synchronize()
        say(f"[compose d128] requests={num_req} init={with_init} lens={lens[:8]}")
        worst = [0.0, 0.0, 0.0]
        for h in heads:
            rS, rell, rP = oracle.compose(hp.GDN, np64(pool.log_scale[:, h:h + 1]), np64(pool.P[:, h:h + 1]),
                                          np64(pool.S[:, h:h + 1]), offs, flat,
                                          init_S=None if init is None else np64(init[:, h:h + 1]), want_P=True)
            for r in range(num_req):
                worst[0] = max(worst[0], rel_fro(np64(out_S[r, h]), rS[r, 0]))
                eP, dl = composed_P_errors(out_ell[r, h], np64(out_P[r, h]), rell[r, 0], rP[r, 0])
                worst[1] = max(worst[1], eP)
                worst[2] = max(worst[2], dl)
        say(f"   S err {worst[0]:.2e}  P err {worst[1]:.2e}  ell err {worst[2]:.2e}")
        assert worst[0] <= 1e-4 and worst[1] <= 1e-4 and worst[2] <= 1e-5


@pytest.mark.parametrize("num_req", [1, 17])
def test_compose_d128_long_chains(num_req):
    """d=128 chains longer than the 1024 slot entries the compose kernels keep in LDS
    (the ring is refilled every 512 steps), on both launch paths (1 request: four
    workgroups per chain; 17 requests x 32 heads: one per chain)."""
    H, d, nslots = 32, 128, 40
    rng = np.random.default_rng(950 + num_req)
    q, _ = np.linalg.qr(rng.standard_normal((nslots, H, d, d)))
    P = q * rng.uniform(0.9, 1.0, size=(nslots, H, 1, d))
    S = rng.standard_normal((nslots, H, d, d))
    ell = rng.uniform(-0.05, 0.0, size=(nslots, H))
    pool = hp.Pool.allocate(hp.GDN, nslots, H, d, d, device="cuda", fill=0.0)
    pool.P.copy_(torch.from_numpy(P).float())
    pool.S.copy_(torch.from_numpy(S).float())
    pool.log_scale.copy_(torch.from_numpy(ell).float())
    lens = [1537] + ([1025] + [int(x) for x in rng.integers(0, 9, size=num_req - 2)] if num_req > 1 else [])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    flat = rng.integers(0, nslots, size=int(offs[-1])).astype(np.int32)
    out_ell = torch.empty((num_req, H), device="cuda")
    say(f"[compose d128 long] requests={num_req} lens={lens[:4]}")
    out_S = hp.compose_chain(pool, dev_i64(offs), dev_i32(flat), out_log_scale=out_ell)
    torch.cuda.synchronize()
    worst = [0.0, 0.0]
    for h in (0, 31):
        rS, rell, _ = oracle.compose(hp.GDN, np64(pool.log_scale[:, h:h + 1]), np64(pool.P[:, h:h + 1]),
                                     np64(pool.S[:, h:h + 1]), offs, flat)
        for r in range(num_req):
            worst[0] = max(worst[0], rel_fro(np64(out_S[r, h]), rS[r, 0]))
            worst[1] = max(worst[1], abs(float(out_ell[r, h]) - float(rell[r, 0])) / max(1.0, abs(float(rell[r, 0]))))
    say(f"   S err {worst[0]:.2e}  ell rel err {worst[1]:.2e}")
    assert worst[0] <= 1e-4 and worst[1] <= 1e-5


def test_compose_out_of_range_slot_flags_and_isolates():
    pool = _gdn_pool()
    chains = [[0, 1, 2], [1, 9, 2], [3, 4]]          # slot 9 is outside the 6-slot pool
    offs = dev_i64(np.concatenate([[0], np.cumsum([len(c) for c in chains])]))
    flat = dev_i32(sum(chains, []))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ell = torch.empty((3, 2), device="cuda")
    out = hp.compose_chain(pool, offs, flat, out_log_scale=ell, err_flag=err)
    clean = hp.compose_chain(pool, dev_i64([0, 3, 5]), dev_i32([0, 1, 2, 3, 4]))
    torch.cuda.synchronize()
    assert int(err.item()) == hp.EFLAG_SLOT_OUT_OF_RANGE
    assert torch.all(torch.isnan(out[1])) and torch.all(torch.isnan(ell[1]))
    assert torch.equal(out[0], clean[0]) and torch.equal(out[2], clean[1])
    # decreasing offsets: flag 2, NaN for that request only
    err.zero_()
    out = hp.compose_chain(pool, dev_i64([0, 2, 1, 3]), dev_i32([0, 1, 2]), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) & hp.EFLAG_BAD_OFFSETS
    assert torch.all(torch.isnan(out[1])) and not torch.any(torch.isnan(out[0]))


@pytest.mark.parametrize("family", [hp.SCALAR, hp.DIAGONAL])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_compose_scalar_diagonal_chains(family, dims):
    """Scalar / diagonal compose on synthetic records against the oracle: chain lengths
    around the kernel's 8-step load batches (0, 1, 7, 8, 9, 17, 20), with and without an
    initial state; a chain of one returns the slot's S bit for bit; an out-of-range slot
    flags and NaN-fills only its request."""
    dk, dv = dims
    H, nslots = 3, 10
    rng = np.random.default_rng(970 + 7 * family + dk + dv // 2)
    pool = hp.Pool.allocate(family, nslots, H, dk, dv, device="cuda", fill=0.0)
    pool.S.copy_(torch.from_numpy(rng.standard_normal((nslots, H, dk, dv))).float())
    ell_shape = (nslots, H, dk) if family == hp.DIAGONAL else (nslots, H)
    pool.log_scale.copy_(torch.from_numpy(rng.uniform(-0.3, 0.0, size=ell_shape)).float())
    lens = [0, 1, 7, 8, 9, 17, 20]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    flat = rng.integers(0, nslots, size=int(offs[-1])).astype(np.int32)
    R = len(lens)
    for with_init in (False, True):
        init = torch.randn((R, H, dk, dv), device="cuda") if with_init else None
        out_ell = torch.empty((R, H, dk) if family == hp.DIAGONAL else (R, H), device="cuda")
        out = hp.compose_chain(pool, dev_i64(offs), dev_i32(flat), init_S=init, out_log_scale=out_ell)
        torch.cuda.synchronize()
        rS, rell, _ = oracle.compose(family, np64(pool.log_scale), None, np64(pool.S), offs, flat,
                                     init_S=None if init is None else np64(init))
        for r in range(R):
            for h in range(H):
                assert rel_fro(np64(out[r, h]), rS[r, h]) <= 1e-5, (r, h)
        assert np.max(np.abs(np64(out_ell) - rell)) <= 1e-5
        if not with_init:
            assert torch.equal(out[1], pool.S[int(flat[offs[1]])])
            assert torch.all(out[0] == 0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = hp.compose_chain(pool, dev_i64([0, 2, 4]), dev_i32([1, 2, 3, nslots + 4]), err_flag=err)
    clean = hp.compose_chain(pool, dev_i64([0, 2]), dev_i32([1, 2]))
    torch.cuda.synchronize()
    assert int(err.item()) == hp.EFLAG_SLOT_OUT_OF_RANGE
    assert torch.all(torch.isnan(out[1])) and torch.equal(out[0], clean[0])


def test_build_error_flags():
    H, d = 2, 64
    inp = make_inputs(hp.GDN, [40, 50], H, d, d, torch.float32, 701)
    pool = hp.Pool.allocate(hp.GDN, 3, H, d, d, device="cuda", fill=CANARY)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp.build_segment(hp.GDN, inp["k"], inp["v"], inp["la"], dev_i64(inp["offs"]), pool, dev_i32([1, 7]),
                     beta=inp["beta"], err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == hp.EFLAG_SLOT_OUT_OF_RANGE
    assert torch.all(pool.S[[0, 2]] == CANARY) and not torch.any(pool.S[1] == CANARY)
    # offsets beyond the stream: flag 2, NaN record in the (valid) slot
    err.zero_()
    hp.build_segment(hp.GDN, inp["k"], inp["v"], inp["la"], dev_i64([0, 40, 95]), pool, dev_i32([0, 2]),
                     beta=inp["beta"], err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == hp.EFLAG_BAD_OFFSETS
    assert torch.all(torch.isnan(pool.S[2])) and torch.all(torch.isnan(pool.P[2]))
    assert not torch.any(torch.isnan(pool.S[0]))


def test_scalar_mfma_build_error_flags():
    """Scalar family, bf16 d=128 (the MFMA build with its weight table, value
    split 4): an out-of-range slot leaves every other slot's canary alone;
    bad offsets give a NaN record beside a finite one."""
    H, d = 2, 128
    inp = make_inputs(hp.SCALAR, [100, 300], H, d, d, torch.bfloat16, 711)
    pool = hp.Pool.allocate(hp.SCALAR, 3, H, d, d, device="cuda", fill=CANARY)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp.build_segment(hp.SCALAR, inp["k"], inp["v"], inp["la"], dev_i64(inp["offs"]), pool, dev_i32([1, 7]),
                     err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == hp.EFLAG_SLOT_OUT_OF_RANGE
    assert torch.all(pool.S[[0, 2]] == CANARY) and torch.all(pool.log_scale[[0, 2]] == CANARY)
    k, v, la, _ = host_inputs(hp.SCALAR, inp, H)
    for h in range(H):
        ell_r, P_r, S_r = oracle_unit(hp.SCALAR, k, v, la, None, 0, 100, h)
        e = record_errors(hp.SCALAR, np64(pool.log_scale[1, h]), None, np64(pool.S[1, h]), ell_r, P_r, S_r)
        assert max(e) <= TOL[torch.bfloat16], e
    err.zero_()
    hp.build_segment(hp.SCALAR, inp["k"], inp["v"], inp["la"], dev_i64([0, 100, 500]), pool, dev_i32([0, 2]),
                     err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == hp.EFLAG_BAD_OFFSETS
    assert torch.all(torch.isnan(pool.S[2])) and torch.all(torch.isnan(pool.log_scale[2]))
    assert not torch.any(torch.isnan(pool.S[0])) and not torch.any(pool.S[0] == CANARY)


# ----------------------------------------------------------------------------- conv warm-up

@pytest.mark.parametrize("K,C,dtype,act,bias", [(4, 4096, torch.bfloat16, 0, False),
                                                (4, 4096, torch.bfloat16, 1, True),
                                                (2, 96, torch.float32, 1, True),
                                                (8, 200, torch.float32, 0, True),
                                                (3, 100, torch.bfloat16, 0, True),
                                                # channel counts that are not a multiple of 4:
                                                # the one-channel-per-thread kernel
                                                (3, 98, torch.bfloat16, 0, True),
                                                (4, 30, torch.float32, 1, False)])
def test_conv_warmup_equals_sequential_conv(K, C, dtype, act, bias):
    rng = np.random.default_rng(800 + K)
    lens = rng.integers(K, 40, size=12)
    offs = synth.offsets_from_lengths(lens)
    N = int(offs[-1])
    x = synth.conv_stream(N, C, dtype, 801, "cuda")
    w = synth.conv_weights(C, K, 802, "cuda")
    bvec = torch.randn(C, device="cuda") if bias else None
    # per segment: its first and last K-1 raw tokens, as a cache would keep them
    heads = torch.stack([x[offs[s]:offs[s] + K - 1] for s in range(len(lens))]).contiguous()
    tails = torch.stack([x[offs[s + 1] - (K - 1):offs[s + 1]] for s in range(len(lens))]).contiguous()
    B = len(lens) - 1
    out = hp.conv_warmup(tails, heads, w, bvec, act, tail_index=dev_i32(np.arange(B)),
                         head_index=dev_i32(np.arange(1, B + 1)))
    torch.cuda.synchronize()
    y = oracle.causal_conv(np64(x), np64(w), None if bvec is None else np64(bvec), act)
    worst = max(rel_fro(np64(out[b]), y[offs[b + 1]:offs[b + 1] + K - 1]) for b in range(B))
    say(f"   conv warm-up K={K} C={C} {dtype} act={act}: max err {worst:.2e}")
    assert worst <= 1e-4


@pytest.mark.parametrize("C", [64, 62])
def test_conv_warmup_bad_index(C):
    """A bad index beside good ones in the same pass of the vector kernel (C = 64) and
    in the one-channel-per-thread kernel (C = 62): NaN rows and the flag, neighbours exact."""
    K = 4
    x = synth.conv_stream(12, C, torch.bfloat16, 810, "cuda").reshape(4, 3, C)
    w = synth.conv_weights(C, K, 811, "cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = hp.conv_warmup(x, x, w, tail_index=dev_i32([0, 5, 1]), head_index=dev_i32([1, 2, 3]),
                         err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == hp.EFLAG_SLOT_OUT_OF_RANGE
    assert torch.all(torch.isnan(out[1])) and not torch.any(torch.isnan(out[[0, 2]]))
