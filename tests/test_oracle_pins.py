"""Pins for the fp64 oracle: it is checked here against things other than itself.

* hand-worked golden examples (tests/golden/, each with its derivation),
* closed forms of the scalar and diagonal families and of GDN with orthonormal keys,
* textbook delta-rule special cases (single token, overwrite with a repeated key, beta = 0),
* a dense brute-force product of the per-token transitions A_t on tiny inputs,
* invariants the pages fix: composition equals the sequential recurrence over the
  concatenation (besthub article, paragraph 4; podcast page, "The transition
  operator: compose, don't add"), partition invariance, associativity,
  contractivity of P, and the negative controls (naive end-state addition fails,
  podcast page "RetNet: naive add vs. operator compose"),
* numpy's convolution for the causal short conv.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import DIAGONAL, GDN, KDA, SCALAR, rel_fro

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------- helpers

def rand_inputs(family, n, H, dk, dv, seed, decay=0.1, beta=True):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n, H, dk))
    k = z / np.linalg.norm(z, axis=-1, keepdims=True)
    v = rng.standard_normal((n, H, dv))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((n, H)))) if beta else None
    if family in (DIAGONAL, KDA):
        la = -decay * np.log1p(np.exp(rng.standard_normal((n, H, dk))))
    else:
        la = -decay * np.log1p(np.exp(rng.standard_normal((n, H))))
    return k, v, b, la


def dense_transition(family, k, b, la):
    """A_t as an explicit matrix (the definition, formed densely)."""
    dk = k.shape[0]
    if family == SCALAR:
        return math.exp(la) * np.eye(dk)
    if family == DIAGONAL:
        return np.diag(np.exp(la))
    if family == KDA:
        return (np.eye(dk) - b * np.outer(k, k)) @ np.diag(np.exp(la))
    return math.exp(la) * (np.eye(dk) - b * np.outer(k, k))


def brute_force(family, k, v, b, la, S0=None):
    """T = A_n ... A_1 and S_n by dense matrix products, one head (k [n,dk])."""
    n, dk = k.shape
    dv = v.shape[1]
    T = np.eye(dk)
    S = np.zeros((dk, dv)) if S0 is None else S0.copy()
    for t in range(n):
        bt = 1.0 if b is None else b[t]
        A = dense_transition(family, k[t], bt, la[t])
        T = A @ T
        S = A @ S + bt * np.outer(k[t], v[t])
    return T, S


def record_T(family, ell, P, dk):
    if family in (GDN, KDA):       # KDA: ell = 0, P = T_C
        return math.exp(ell) * P
    if family == SCALAR:
        return math.exp(ell) * np.eye(dk)
    return np.diag(np.exp(ell))


def one_head(x, h):
    return None if x is None else x[:, h]


# ----------------------------------------------------------------------------- golden

def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_golden_gdn_two_tokens():
    g = _load("gdn_two_tokens.json")
    toks = g["tokens"]
    k = np.array([t["k"] for t in toks])[:, None, :]
    v = np.array([t["v"] for t in toks])[:, None, :]
    b = np.array([[t["beta"]] for t in toks])
    la = np.log(np.array([[t["alpha"]] for t in toks]))
    ell, P, S = oracle.build_segments(GDN, k, v, la, [0, 2], beta=b)
    e = g["expected"]
    assert abs(ell[0, 0] - e["ell"]) < 1e-12
    np.testing.assert_allclose(P[0, 0], e["P"], atol=1e-12)
    np.testing.assert_allclose(S[0, 0], e["S"], atol=1e-12)
    np.testing.assert_allclose(math.exp(ell[0, 0]) * P[0, 0], e["T"], atol=1e-12)
    # the two one-token records, composed in prompt order, give the same state
    ell1, P1, S1 = oracle.build_segments(GDN, k, v, la, [0, 1, 2], beta=b)
    Sc, _, _ = oracle.compose(GDN, ell1, P1, S1, [0, 2], [0, 1])
    np.testing.assert_allclose(Sc[0, 0], e["S"], atol=1e-12)
    np.testing.assert_allclose(S1[0, 0] + S1[1, 0], e["naive_sum"], atol=1e-12)


def test_golden_scalar_three_tokens():
    g = _load("scalar_three_tokens.json")
    toks = g["tokens"]
    k = np.array([t["k"] for t in toks])[:, None, :]
    v = np.array([t["v"] for t in toks])[:, None, :]
    la = np.full((3, 1), math.log(g["gamma"]))
    ell, P, S = oracle.build_segments(SCALAR, k, v, la, [0, 3])
    e = g["expected"]
    assert P is None
    assert abs(ell[0, 0] - e["ell"]) < 1e-12
    np.testing.assert_allclose(S[0, 0], e["S"], atol=1e-12)
    np.testing.assert_allclose(record_T(SCALAR, ell[0, 0], None, 2), e["T"], atol=1e-12)


def test_golden_diagonal_two_tokens():
    g = _load("diagonal_two_tokens.json")
    toks = g["tokens"]
    k = np.array([t["k"] for t in toks])[:, None, :]
    v = np.array([t["v"] for t in toks])[:, None, :]
    la = np.log(np.array([t["alpha"] for t in toks]))[:, None, :]
    ell, _, S = oracle.build_segments(DIAGONAL, k, v, la, [0, 2])
    e = g["expected"]
    np.testing.assert_allclose(ell[0, 0], e["ell"], atol=1e-12)
    np.testing.assert_allclose(S[0, 0], e["S"], atol=1e-12)
    np.testing.assert_allclose(record_T(DIAGONAL, ell[0, 0], None, 2), e["T"], atol=1e-12)


def test_golden_conv_impulse():
    g = _load("conv_impulse.json")
    x = np.array(g["x"])[:, None]
    w = np.array(g["kernel"])[None, :]
    np.testing.assert_allclose(oracle.causal_conv(x, w, None, 0)[:, 0], g["expected_identity"], atol=1e-12)
    np.testing.assert_allclose(oracle.causal_conv(x, w, None, 1)[:, 0], g["expected_silu"], atol=1e-12)


# ----------------------------------------------------------------------------- closed forms

def test_scalar_closed_form():
    n, dk, dv, H = 50, 5, 3, 2
    k, v, b, _ = rand_inputs(SCALAR, n, H, dk, dv, 1)
    log_g = np.log(np.array([0.93, 0.998]))
    la = np.broadcast_to(log_g, (n, H)).copy()
    ell, P, S = oracle.build_segments(SCALAR, k, v, la, [0, n], beta=b)
    for h in range(H):
        assert abs(ell[0, h] - n * log_g[h]) < 1e-12
        w = np.exp((n - 1 - np.arange(n)) * log_g[h]) * b[:, h]
        S_cf = np.einsum("t,ti,tj->ij", w, k[:, h], v[:, h])
        assert rel_fro(S[0, h], S_cf) < 1e-13


def test_diagonal_closed_form():
    n, dk, dv, H = 40, 6, 4, 2
    k, v, _, la = rand_inputs(DIAGONAL, n, H, dk, dv, 2)
    ell, _, S = oracle.build_segments(DIAGONAL, k, v, la, [0, n])
    for h in range(H):
        np.testing.assert_allclose(ell[0, h], la[:, h].sum(axis=0), atol=1e-12)
        # the gate product of the tokens after t, per key channel
        after = np.cumsum(la[::-1, h], axis=0)[::-1] - la[:, h]
        S_cf = np.einsum("ti,ti,tj->ij", np.exp(after), k[:, h], v[:, h])
        assert rel_fro(S[0, h], S_cf) < 1e-13


def test_gdn_orthonormal_keys_closed_form():
    # with mutually orthogonal keys the projections commute
    n, dk, dv = 6, 8, 3
    rng = np.random.default_rng(3)
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Q[:, :n].T.copy()[:, None, :]
    v = rng.standard_normal((n, 1, dv))
    b = rng.uniform(0.1, 1.0, (n, 1))
    la = -0.3 * rng.uniform(0.0, 1.0, (n, 1))
    ell, P, S = oracle.build_segments(GDN, k, v, la, [0, n], beta=b)
    P_cf = np.eye(dk) - np.einsum("t,ti,tj->ij", b[:, 0], k[:, 0], k[:, 0])
    L = np.cumsum(la[:, 0])
    S_cf = np.einsum("t,ti,tj->ij", np.exp(L[-1] - L) * b[:, 0], k[:, 0], v[:, 0])
    assert abs(ell[0, 0] - L[-1]) < 1e-12
    assert rel_fro(P[0, 0], P_cf) < 1e-13
    assert rel_fro(S[0, 0], S_cf) < 1e-13


def test_gdn_single_token_and_delta_rule_cases():
    rng = np.random.default_rng(4)
    dk, dv = 5, 4
    kk = rng.standard_normal(dk)
    kk /= np.linalg.norm(kk)
    v1, v2 = rng.standard_normal(dv), rng.standard_normal(dv)
    a, bb = 0.7, 0.35
    # single token: T = alpha (I - beta k k^T), S = beta k v^T
    ell, P, S = oracle.build_segments(GDN, kk[None, None], v1[None, None], [[math.log(a)]], [0, 1], beta=[[bb]])
    assert rel_fro(math.exp(ell[0, 0]) * P[0, 0], a * (np.eye(dk) - bb * np.outer(kk, kk))) < 1e-14
    assert rel_fro(S[0, 0], bb * np.outer(kk, v1)) < 1e-14
    # beta = 1 with a repeated key overwrites the value stored under that key
    k2 = np.stack([kk, kk])[:, None]
    v12 = np.stack([v1, v2])[:, None]
    _, _, S = oracle.build_segments(GDN, k2, v12, np.zeros((2, 1)), [0, 2], beta=np.ones((2, 1)))
    assert rel_fro(S[0, 0], np.outer(kk, v2)) < 1e-14
    # beta = 1/2 twice: S = (I - k k^T/2)(k v1^T/2) + k v2^T/2 = k (v1/4 + v2/2)^T
    _, _, S = oracle.build_segments(GDN, k2, v12, np.zeros((2, 1)), [0, 2], beta=np.full((2, 1), 0.5))
    assert rel_fro(S[0, 0], np.outer(kk, v1 / 4 + v2 / 2)) < 1e-14
    # beta = 0: nothing is written and P = I, T = e^ell I
    ell, P, S = oracle.build_segments(GDN, k2, v12, [[-0.2], [-0.5]], [0, 2], beta=np.zeros((2, 1)))
    assert abs(ell[0, 0] + 0.7) < 1e-15
    np.testing.assert_array_equal(P[0, 0], np.eye(dk))
    np.testing.assert_array_equal(S[0, 0], np.zeros((dk, dv)))


def test_plain_linear_attention_naive_add_exact():
    # alpha = 1, beta = 1, scalar family: T = I and the naive end-state sum is exact
    n, H, dk, dv = 30, 1, 4, 3
    k, v, _, _ = rand_inputs(SCALAR, n, H, dk, dv, 5)
    la = np.zeros((n, H))
    offs = [0, 10, 21, 30]
    ell, _, S = oracle.build_segments(SCALAR, k, v, la, offs)
    _, _, S_seq = oracle.build_segments(SCALAR, k, v, la, [0, n])
    assert np.all(ell == 0.0)
    assert rel_fro(S.sum(axis=0), S_seq[0]) < 1e-14


# ----------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("family", [SCALAR, DIAGONAL, GDN, KDA])
def test_brute_force_dense_products(family):
    n, H, dk, dv = 37, 2, 6, 5
    k, v, b, la = rand_inputs(family, n, H, dk, dv, 10 + family, decay=0.3)
    offs = [0, 1, 13, 13, 37]          # includes an empty segment
    ell, P, S = oracle.build_segments(family, k, v, la, offs, beta=b)
    for s in range(len(offs) - 1):
        lo, hi = offs[s], offs[s + 1]
        for h in range(H):
            T_bf, S_bf = brute_force(family, k[lo:hi, h], v[lo:hi, h], b[lo:hi, h], la[lo:hi, h])
            T = record_T(family, ell[s, h], None if P is None else P[s, h], dk)
            assert np.max(np.abs(T - T_bf)) < 1e-13
            assert np.max(np.abs(S[s, h] - S_bf)) < 1e-12


def test_empty_segment_is_identity_record():
    k, v, b, la = rand_inputs(GDN, 4, 2, 3, 2, 11)
    ell, P, S = oracle.build_segments(GDN, k, v, la, [0, 0, 4], beta=b)
    assert np.all(ell[0] == 0.0)
    np.testing.assert_array_equal(P[0], np.broadcast_to(np.eye(3), (2, 3, 3)))
    np.testing.assert_array_equal(S[0], np.zeros((2, 3, 2)))


# ----------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("family", [SCALAR, DIAGONAL, GDN, KDA])
def test_composition_equals_sequential(family):
    # the identity the pages fix: composed records = recurrence over the concatenation
    H, dk, dv = 2, 8, 6
    lens = [17, 1, 40, 0, 25]
    offs = np.concatenate([[0], np.cumsum(lens)])
    n = int(offs[-1])
    k, v, b, la = rand_inputs(family, n, H, dk, dv, 20 + family, decay=0.02)
    ell, P, S = oracle.build_segments(family, k, v, la, offs, beta=b)
    Sc, ellc, Pc = oracle.compose(family, ell, P, S, [0, len(lens)], np.arange(len(lens)), want_P=True)
    ell_seq, P_seq, S_seq = oracle.build_segments(family, k, v, la, [0, n], beta=b)
    assert rel_fro(Sc[0], S_seq[0]) < 1e-12
    np.testing.assert_allclose(ellc[0], ell_seq[0], atol=1e-12)
    if family in (GDN, KDA):
        assert rel_fro(Pc[0], P_seq[0]) < 1e-12


@pytest.mark.parametrize("family", [SCALAR, DIAGONAL, GDN, KDA])
def test_record_maps_any_start_state(family):
    # S_n(S_0) = T_C S_0 + S(C|0) for an arbitrary start state
    n, H, dk, dv = 23, 2, 5, 4
    k, v, b, la = rand_inputs(family, n, H, dk, dv, 30 + family, decay=0.05)
    S0 = np.random.default_rng(31).standard_normal((1, H, dk, dv))
    ell, P, S = oracle.build_segments(family, k, v, la, [0, n], beta=b)
    _, _, S_from = oracle.build_segments(family, k, v, la, [0, n], beta=b, init_S=S0)
    for h in range(H):
        T = record_T(family, ell[0, h], None if P is None else P[0, h], dk)
        assert rel_fro(S_from[0, h], T @ S0[0, h] + S[0, h]) < 1e-13
    # compose with an initial state agrees as well
    Sc, _, _ = oracle.compose(family, ell, P, S, [0, 1], [0], init_S=S0)
    assert rel_fro(Sc, S_from) < 1e-13


@pytest.mark.parametrize("family", [SCALAR, DIAGONAL, GDN, KDA])
def test_partition_invariance(family):
    H, dk, dv, n = 1, 6, 4, 60
    k, v, b, la = rand_inputs(family, n, H, dk, dv, 40 + family, decay=0.02)
    outs = []
    for offs in ([0, 60], [0, 30, 60], [0, 7, 8, 33, 59, 60], [0, 1, 2, 3, 60]):
        ell, P, S = oracle.build_segments(family, k, v, la, offs, beta=b)
        m = len(offs) - 1
        Sc, _, _ = oracle.compose(family, ell, P, S, [0, m], np.arange(m))
        outs.append(Sc[0, 0])
    for o in outs[1:]:
        assert rel_fro(o, outs[0]) < 1e-12


def test_associativity_tree_vs_chain():
    H, dk, dv = 2, 6, 5
    lens = [9, 14, 3, 20]
    offs = np.concatenate([[0], np.cumsum(lens)])
    k, v, b, la = rand_inputs(GDN, int(offs[-1]), H, dk, dv, 50, decay=0.02)
    ell, P, S = oracle.build_segments(GDN, k, v, la, offs, beta=b)
    # pair records (0,1) and (2,3), then compose the two pair records
    S01, e01, P01 = oracle.compose(GDN, ell, P, S, [0, 2], [0, 1], want_P=True)
    S23, e23, P23 = oracle.compose(GDN, ell, P, S, [0, 2], [2, 3], want_P=True)
    pe = np.concatenate([e01, e23])
    pP = np.concatenate([P01, P23])
    pS = np.concatenate([S01, S23])
    S_tree, e_tree, P_tree = oracle.compose(GDN, pe, pP, pS, [0, 2], [0, 1], want_P=True)
    S_chain, e_chain, P_chain = oracle.compose(GDN, ell, P, S, [0, 4], [0, 1, 2, 3], want_P=True)
    assert rel_fro(S_tree, S_chain) < 1e-13
    assert rel_fro(P_tree, P_chain) < 1e-13
    np.testing.assert_allclose(e_tree, e_chain, atol=1e-13)


def test_contractivity():
    # beta in [0,1] and ||k|| = 1: every factor I - beta k k^T has 2-norm <= 1, and ell <= 0
    k, v, b, la = rand_inputs(GDN, 300, 2, 16, 8, 60)
    ell, P, _ = oracle.build_segments(GDN, k, v, la, [0, 100, 300], beta=b)
    assert np.all(ell <= 0.0)
    for s in range(2):
        for h in range(2):
            assert np.linalg.norm(P[s, h], 2) <= 1.0 + 1e-12


# ----------------------------------------------------------------------------- negative controls

def test_negative_controls_fail_on_weak_gates():
    """Naive end-state addition and the wrong composition order are wrong.

    Podcast page, "The transition operator: compose, don't add" and "RetNet:
    naive add vs. operator compose": naive addition fails already for RetNet
    and its error grows as more segments are chained.  Weak gates make the
    prefix matter (with strong gates every family forgets it).
    """
    H, dk, dv, L = 1, 16, 8, 64
    # RetNet-style scalar decay close to 1
    errs = []
    for m in (2, 4, 8):
        n = m * L
        k, v, _, _ = rand_inputs(SCALAR, n, H, dk, dv, 70)
        la = np.full((n, H), math.log(0.999))
        offs = np.arange(m + 1) * L
        ell, _, S = oracle.build_segments(SCALAR, k, v, la, offs)
        _, _, S_seq = oracle.build_segments(SCALAR, k, v, la, [0, n])
        Sc, _, _ = oracle.compose(SCALAR, ell, None, S, [0, m], np.arange(m))
        assert rel_fro(Sc[0], S_seq[0]) < 1e-12
        errs.append(rel_fro(S.sum(axis=0), S_seq[0]))
    assert errs[0] > 2e-2 and errs[0] < errs[1] < errs[2]
    # GDN with alpha = 1 (DeltaNet): naive add and the swapped order both fail
    n = 2 * L
    k, v, b, _ = rand_inputs(GDN, n, H, dk, dv, 71)
    la = np.zeros((n, H))
    ell, P, S = oracle.build_segments(GDN, k, v, la, [0, L, n], beta=b)
    _, _, S_seq = oracle.build_segments(GDN, k, v, la, [0, n], beta=b)
    Sc, _, _ = oracle.compose(GDN, ell, P, S, [0, 2], [0, 1])
    S_wrong, _, _ = oracle.compose(GDN, ell, P, S, [0, 2], [1, 0])
    assert rel_fro(Sc[0], S_seq[0]) < 1e-12
    assert rel_fro(S[0] + S[1], S_seq[0]) > 2e-2
    assert rel_fro(S_wrong[0], S_seq[0]) > 2e-2


# ----------------------------------------------------------------------------- compose indexing

def test_compose_single_and_dead_record_are_exact():
    k, v, b, la = rand_inputs(GDN, 30, 2, 4, 3, 80)
    ell, P, S = oracle.build_segments(GDN, k, v, la, [0, 10, 30], beta=b)
    # one record from a zero start returns that record's S exactly
    Sc, _, _ = oracle.compose(GDN, ell, P, S, [0, 1, 2], [1, 0])
    np.testing.assert_array_equal(Sc[0], S[1])
    np.testing.assert_array_equal(Sc[1], S[0])
    # a record with ell = -inf forgets everything before it
    ell2 = ell.copy()
    ell2[1] = -np.inf
    Sc, _, _ = oracle.compose(GDN, ell2, P, S, [0, 2], [0, 1])
    np.testing.assert_array_equal(Sc[0], S[1])
    # the empty chain returns the start state
    S0 = np.random.default_rng(81).standard_normal((1, 2, 4, 3))
    Sc, _, _ = oracle.compose(GDN, ell, P, S, [0, 0], np.zeros(0, np.int32), init_S=S0)
    np.testing.assert_array_equal(Sc, S0)
    with pytest.raises(ValueError):
        oracle.compose(GDN, ell, P, S, [0, 1], [2])


# ----------------------------------------------------------------------------- conv

@pytest.mark.parametrize("K", [2, 4])
def test_conv_matches_numpy_convolve(K):
    rng = np.random.default_rng(90 + K)
    n, C = 37, 5
    x = rng.standard_normal((n, C))
    w = rng.uniform(-0.5, 0.5, (C, K))
    bias = rng.standard_normal(C)
    y = oracle.causal_conv(x, w, bias, 0)
    for c in range(C):
        ref = np.convolve(x[:, c], w[c, ::-1])[:n] + bias[c]
        np.testing.assert_allclose(y[:, c], ref, atol=1e-13)
    ys = oracle.causal_conv(x, w, bias, 1)
    np.testing.assert_allclose(ys, y / (1.0 + np.exp(-y)), atol=1e-13)


def test_conv_warmup_window_identity():
    """The conv outputs at a segment's first K-1 positions depend only on the
    previous K-1 raw inputs and the segment's own first K-1 inputs; from
    position K-1 on they do not depend on the previous segment at all."""
    rng = np.random.default_rng(95)
    K, C = 4, 6
    lens = [9, 5, 12]
    offs = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((int(offs[-1]), C))
    w = rng.uniform(-0.5, 0.5, (C, K))
    y_full = oracle.causal_conv(x, w, None, 1)
    for s in range(1, len(lens)):
        a, e = offs[s], offs[s + 1]
        window = np.concatenate([x[a - (K - 1):a], x[a:a + K - 1]])
        y_win = oracle.causal_conv(window, w, None, 1)
        np.testing.assert_allclose(y_win[K - 1:], y_full[a:a + K - 1], atol=1e-13)
        y_cold = oracle.causal_conv(x[a:e], w, None, 1)
        np.testing.assert_allclose(y_cold[K - 1:], y_full[a + K - 1:e], atol=1e-13)
        # a zero tail reproduces the cold conv of the segment
        zero_win = np.concatenate([np.zeros((K - 1, C)), x[a:a + K - 1]])
        np.testing.assert_allclose(oracle.causal_conv(zero_win, w, None, 1)[K - 1:], y_cold[:K - 1], atol=1e-13)


# ----------------------------------------------------------------------------- conv variant keys / values

@pytest.mark.parametrize("act", [0, 1])
def test_conv_kv_brute_force(act):
    """conv_kv against the definition written out element by element: the causal conv
    with zero history, the activation, the split into heads, the key L2 norm."""
    rng = np.random.default_rng(70 + act)
    n, H, dk, dv, K = 7, 2, 3, 2, 3
    C = H * (dk + dv)
    x = rng.standard_normal((n, C))
    w = rng.uniform(-0.5, 0.5, (C, K))
    bias = rng.standard_normal(C)
    k, v = oracle.conv_kv(x, w, bias, act, H, dk, dv)
    for t in range(n):
        y = np.zeros(C)
        for c in range(C):
            acc = bias[c]
            for j in range(K):
                s = t - (K - 1) + j
                if s >= 0:
                    acc += w[c, j] * x[s, c]
            y[c] = acc / (1.0 + math.exp(-acc)) if act == 1 else acc
        for h in range(H):
            kk = y[h * dk:(h + 1) * dk]
            np.testing.assert_allclose(k[t, h], kk / math.sqrt(float(kk @ kk) + 1e-6), atol=1e-13)
            np.testing.assert_allclose(v[t, h], y[H * dk + h * dv:H * dk + (h + 1) * dv], atol=1e-13)
    ku, _ = oracle.conv_kv(x, w, bias, act, H, dk, dv, normalize=False)
    np.testing.assert_allclose(ku, oracle.causal_conv(x, w, bias, act)[:, :H * dk].reshape(n, H, dk), atol=1e-13)


def test_conv_kv_suffix_context_free_head_warmed():
    """The reading the conv-coupled records rest on: in a stream cut into two segments,
    the second segment's keys and values from its token K-1 on equal those of the
    segment alone (zero history), and its first K-1 equal the conv over the first
    segment's last K-1 raw inputs followed by its own; with zero history instead the
    first K-1 differ."""
    rng = np.random.default_rng(77)
    H, dk, dv, K = 2, 4, 3, 4
    C = H * (dk + dv)
    n1, n2 = 9, 8
    x = rng.standard_normal((n1 + n2, C))
    w = rng.uniform(-0.5, 0.5, (C, K))
    k, v = oracle.conv_kv(x, w, None, 1, H, dk, dv)
    k2, v2 = oracle.conv_kv(x[n1:], w, None, 1, H, dk, dv)
    np.testing.assert_allclose(k[n1 + K - 1:], k2[K - 1:], atol=1e-13)
    np.testing.assert_allclose(v[n1 + K - 1:], v2[K - 1:], atol=1e-13)
    kw, vw = oracle.conv_kv(x[n1 - (K - 1):], w, None, 1, H, dk, dv)
    np.testing.assert_allclose(k[n1:n1 + K - 1], kw[K - 1:2 * (K - 1)], atol=1e-13)
    np.testing.assert_allclose(v[n1:n1 + K - 1], vw[K - 1:2 * (K - 1)], atol=1e-13)
    assert np.max(np.abs(k[n1:n1 + K - 1] - k2[:K - 1])) > 1e-2


# ----------------------------------------------------------------------------- KDA special cases

def test_kda_without_decay_is_gdn_without_decay():
    """alpha = 1: (I - beta k k^T) diag(1) is the ungated delta rule, as GDN with log alpha = 0."""
    n, H, dk, dv = 29, 2, 6, 5
    k, v, b, la = rand_inputs(KDA, n, H, dk, dv, 80)
    ell_k, P_k, S_k = oracle.build_segments(KDA, k, v, np.zeros((n, H, dk)), [0, n], beta=b)
    ell_g, P_g, S_g = oracle.build_segments(GDN, k, v, np.zeros((n, H)), [0, n], beta=b)
    np.testing.assert_allclose(P_k, P_g, atol=1e-14)
    np.testing.assert_allclose(S_k, S_g, atol=1e-14)
    assert np.all(ell_k == 0.0) and np.all(ell_g == 0.0)


def test_kda_without_writes_is_the_product_of_gates():
    """beta = 0: A_t = diag(alpha_t), so T_C = diag(prod_t alpha_t) and nothing is written."""
    n, H, dk, dv = 21, 2, 5, 3
    k, v, _, la = rand_inputs(KDA, n, H, dk, dv, 81, decay=0.2)
    ell, P, S = oracle.build_segments(KDA, k, v, la, [0, n], beta=np.zeros((n, H)))
    for h in range(H):
        np.testing.assert_allclose(P[0, h], np.diag(np.exp(la[:, h].sum(axis=0))), atol=1e-14)
    assert np.all(S == 0.0)


def test_kda_channel_keys_closed_form():
    """Keys along coordinate axes: each A_t is diagonal, entry i scaled by alpha_{t,i} and,
    on the key's own axis, by (1 - beta_t); S_n = sum_t (prod_{s>t} A_s) beta_t k_t v_t^T."""
    n, dk, dv = 17, 4, 3
    rng = np.random.default_rng(82)
    axes = rng.integers(0, dk, size=n)
    k = np.zeros((n, 1, dk))
    k[np.arange(n), 0, axes] = 1.0
    v = rng.standard_normal((n, 1, dv))
    b = rng.uniform(0.1, 0.9, size=(n, 1))
    la = -0.3 * rng.uniform(0.0, 1.0, size=(n, 1, dk))
    _, P, S = oracle.build_segments(KDA, k, v, la, [0, n], beta=b)
    diag = np.ones(dk)
    S_cf = np.zeros((dk, dv))
    for t in range(n):
        a = np.exp(la[t, 0])
        a[axes[t]] *= 1.0 - b[t, 0]
        diag *= a
        S_cf = a[:, None] * S_cf
        S_cf[axes[t]] += b[t, 0] * v[t, 0]
    np.testing.assert_allclose(P[0, 0], np.diag(diag), atol=1e-14)
    np.testing.assert_allclose(S[0, 0], S_cf, atol=1e-13)


# ----------------------------------------------------------------------------- in-segment outputs
# o_t = S_t^T q_t from the state right after token t: the chunked prefill forward's
# readout, with the records as side-outputs (besthub article, paragraph 7).

def test_golden_gdn_two_token_outputs():
    g = _load("gdn_two_tokens_outputs.json")
    toks = g["tokens"]
    k = np.array([t["k"] for t in toks])[:, None, :]
    v = np.array([t["v"] for t in toks])[:, None, :]
    q = np.array([t["q"] for t in toks])[:, None, :]
    b = np.array([[t["beta"]] for t in toks])
    la = np.log(np.array([[t["alpha"]] for t in toks]))
    o, ell, P, S = oracle.forward(GDN, k, v, q, la, [0, 2], beta=b)
    np.testing.assert_allclose(o[:, 0], g["expected"]["o"], atol=1e-12)
    # the records are the build's, bit for bit
    ell_b, P_b, S_b = oracle.build_segments(GDN, k, v, la, [0, 2], beta=b)
    assert np.array_equal(ell, ell_b) and np.array_equal(P, P_b) and np.array_equal(S, S_b)


@pytest.mark.parametrize("family", [SCALAR, DIAGONAL, GDN, KDA])
def test_outputs_single_token(family):
    """From a zero state one token writes beta k v^T, so o = beta (q . k) v."""
    k, v, b, la = rand_inputs(family, 1, 2, 5, 3, 2101)
    q = np.random.default_rng(2102).standard_normal((1, 2, 5))
    o, _, _, _ = oracle.forward(family, k, v, q, la, [0, 1], beta=b)
    for h in range(2):
        want = b[0, h] * float(q[0, h] @ k[0, h]) * v[0, h]
        np.testing.assert_allclose(o[0, h], want, rtol=1e-13, atol=1e-14)


def test_outputs_gdn_orthonormal_keys_closed_form():
    """Orthonormal keys commute through the projections, so
    S_t = sum_{s<=t} e^{g_t - g_s} beta_s k_s v_s^T and
    o_t = sum_{s<=t} e^{g_t - g_s} beta_s (k_s . q_t) v_s."""
    n, d, dv = 8, 12, 5
    rng = np.random.default_rng(2103)
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Q[:n][:, None, :]
    v = rng.standard_normal((n, 1, dv))
    q = rng.standard_normal((n, 1, d))
    b = rng.uniform(0.1, 0.9, size=(n, 1))
    la = -rng.uniform(0.0, 0.3, size=(n, 1))
    o, _, _, _ = oracle.forward(GDN, k, v, q, la, [0, n], beta=b)
    g = np.cumsum(la[:, 0])
    for t in range(n):
        want = sum(math.exp(g[t] - g[s]) * b[s, 0] * float(k[s, 0] @ q[t, 0]) * v[s, 0] for s in range(t + 1))
        np.testing.assert_allclose(o[t, 0], want, rtol=1e-12, atol=1e-13)


def test_outputs_scalar_and_diagonal_closed_forms():
    """Scalar: o_t = sum_{s<=t} gamma^{t-s} (k_s . q_t) v_s (retention); diagonal:
    o_t = sum_{s<=t} ((q_t * prod_{s<r<=t} alpha_r) . k_s) v_s (gated linear attention)."""
    n, d, dv = 9, 4, 3
    rng = np.random.default_rng(2104)
    k, v, q = (rng.standard_normal((n, 1, d)), rng.standard_normal((n, 1, dv)), rng.standard_normal((n, 1, d)))
    lg = math.log(0.9)
    o, _, _, _ = oracle.forward(SCALAR, k, v, q, np.full((n, 1), lg), [0, n])
    for t in range(n):
        want = sum(0.9 ** (t - s) * float(k[s, 0] @ q[t, 0]) * v[s, 0] for s in range(t + 1))
        np.testing.assert_allclose(o[t, 0], want, rtol=1e-12, atol=1e-13)
    la = -rng.uniform(0.0, 0.5, size=(n, 1, d))
    o, _, _, _ = oracle.forward(DIAGONAL, k, v, q, la, [0, n])
    for t in range(n):
        want = np.zeros(dv)
        for s in range(t + 1):
            decay = np.exp(la[s + 1:t + 1, 0].sum(axis=0))
            want += float((q[t, 0] * decay) @ k[s, 0]) * v[s, 0]
        np.testing.assert_allclose(o[t, 0], want, rtol=1e-12, atol=1e-13)


def test_outputs_plain_linear_attention():
    """No decay, no delta term (beta = 1 on the scalar family): causal linear
    attention, O = tril(Q K^T) V."""
    n, d, dv = 11, 6, 4
    rng = np.random.default_rng(2105)
    k, v, q = (rng.standard_normal((n, 1, d)), rng.standard_normal((n, 1, dv)), rng.standard_normal((n, 1, d)))
    o, _, _, _ = oracle.forward(SCALAR, k, v, q, np.zeros((n, 1)), [0, n])
    want = np.tril(q[:, 0] @ k[:, 0].T) @ v[:, 0]
    np.testing.assert_allclose(o[:, 0], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("family", [SCALAR, DIAGONAL, GDN, KDA])
def test_outputs_brute_force_dense_states(family):
    """Every token's state by dense products of the A_t matrices, read out with q_t."""
    n, H, dk, dv = 10, 2, 4, 3
    k, v, b, la = rand_inputs(family, n, H, dk, dv, 2106, decay=0.3)
    q = np.random.default_rng(2107).standard_normal((n, H, dk))
    offs = [0, 4, 4, 10]                     # an empty segment in the middle
    o, _, _, _ = oracle.forward(family, k, v, q, la, offs, beta=b)
    for h in range(H):
        for s in range(3):
            for t in range(offs[s], offs[s + 1]):
                sl = slice(offs[s], t + 1)
                _, St = brute_force(family, k[sl, h], v[sl, h], one_head(b, h)[sl] if b is not None else None,
                                    la[sl, h])
                np.testing.assert_allclose(o[t, h], St.T @ q[t, h], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("family", [SCALAR, DIAGONAL, GDN, KDA])
def test_outputs_from_a_start_state_compose(family):
    """From a start state S_0 the outputs are (T_{<=t} S_0 + S_t(0))^T q_t, where
    T_{<=t} and S_t(0) are the record of the segment's first t+1 tokens: the
    composition law read out token by token."""
    n, H, dk, dv = 7, 2, 4, 3
    k, v, b, la = rand_inputs(family, n, H, dk, dv, 2108, decay=0.2)
    rng = np.random.default_rng(2109)
    q = rng.standard_normal((n, H, dk))
    S0 = rng.standard_normal((1, H, dk, dv))
    o, _, _, _ = oracle.forward(family, k, v, q, la, [0, n], beta=b, init_S=S0)
    o0, _, _, _ = oracle.forward(family, k, v, q, la, [0, n], beta=b)
    for t in range(n):
        ell, P, _ = oracle.build_segments(family, k[:t + 1], v[:t + 1], la[:t + 1], [0, t + 1],
                                          beta=None if b is None else b[:t + 1])
        for h in range(H):
            T = record_T(family, ell[0, h], None if P is None else P[0, h], dk)
            want = o0[t, h] + (T @ S0[0, h]).T @ q[t, h]
            np.testing.assert_allclose(o[t, h], want, rtol=1e-11, atol=1e-12)


def test_outputs_last_token_reads_the_record():
    """The last output of a segment is its zero-start record read out: o_last = S^T q_last."""
    n, H, d = 70, 3, 6
    k, v, b, la = rand_inputs(GDN, n, H, d, d, 2110)
    q = np.random.default_rng(2111).standard_normal((n, H, d))
    offs = [0, 33, 70]
    o, _, _, S = oracle.forward(GDN, k, v, q, la, offs, beta=b)
    for s in range(2):
        for h in range(H):
            np.testing.assert_allclose(o[offs[s + 1] - 1, h], S[s, h].T @ q[offs[s + 1] - 1, h], rtol=1e-13)
