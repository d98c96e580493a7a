"""fp64 CPU oracle for the HYPIC linear-layer segment cache (ctypes over hypic_oracle.c).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library ``hybrid_prefill_amd`` and never imports it.

What it computes (pages: "HYPIC: Cache Acceleration for Hybrid Attention
Models", section "Core Approach"; "Cut First-Token Latency by 3.25x ...",
paragraph 4; the podcast companion page, sections "The transition operator:
compose, don't add" and "Family comparison"):

* ``forward`` -- the same records plus every token's in-segment output
  ``o_t = S_t^T q_t`` (the chunked prefill forward's definition).
* ``build_segments`` -- per segment and head, the record ``(ell, P, S)`` of the
  recurrence ``S_t = A_t S_{t-1} + beta_t k_t v_t^T`` from ``S_0 = 0``, with
  ``T_C = e^ell P`` (KDA, ``A_t = (I - beta k k^T) diag(alpha_t)``: ``ell = 0``,
  ``P = T_C``), token by token in fp64.
* ``compose`` -- ``S <- T_i S + S_i`` over a chain of pool records in prompt order.
* ``causal_conv`` -- the full causal depthwise short convolution over a raw stream.
* ``conv_kv`` -- a conv variant's keys and values over a raw stream: the causal
  conv and activation, the channels split per head, each key L2-normalised.

Every function takes numpy arrays; inputs are upcast to fp64 exactly (bf16 and
fp32 values are representable in fp64), so the oracle sees the exact bytes the
GPU saw.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
closed forms, hand-worked golden examples, a dense brute-force product and
invariants; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

SCALAR, DIAGONAL, GDN, KDA = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hypic_oracle.c")
_DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")
SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
# HYPIC_ORACLE_LIB names another build of the oracle (the sanitized one, see build_library)
_LIB_PATH = os.environ.get("HYPIC_ORACLE_LIB") or _DEFAULT_LIB
_lib = None


def build_library(sanitize: bool = False) -> str:
    """Compile ``hypic_oracle.c`` with gcc (-O2, OpenMP) into ``oracle/liboracle.so``; with
    sanitize, an AddressSanitizer + UndefinedBehaviorSanitizer build (abort on the first
    report) into ``oracle/liboracle_san.so``, loaded by a process that preloads gcc's
    libasan and libubsan."""
    out = SAN_LIB if sanitize else _DEFAULT_LIB
    tmp = out + ".tmp"
    extra = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"]
    cmd = ["gcc", *extra, "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_PATH == _DEFAULT_LIB and (not os.path.exists(_LIB_PATH) or
                                      os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build_library()
    lib = ctypes.CDLL(_LIB_PATH)
    d, i64, i32, ci = (ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                       ctypes.POINTER(ctypes.c_int32), ctypes.c_int)
    lib.oracle_build_segments.argtypes = [ci, ci, ci, ci, ci, i64, d, d, d, d, d, d, d, d]
    lib.oracle_build_segments.restype = ci
    lib.oracle_forward.argtypes = [ci, ci, ci, ci, ci, i64, d, d, d, d, d, d, d, d, d, d]
    lib.oracle_forward.restype = ci
    lib.oracle_compose.argtypes = [ci, ci, ci, ci, ctypes.c_int64, d, d, d, ci, i64, i32, d, d, d, d]
    lib.oracle_compose.restype = ci
    lib.oracle_causal_conv.argtypes = [ctypes.c_int64, ci, ci, d, d, d, ci, d]
    lib.oracle_causal_conv.restype = ci
    lib.oracle_num_threads.restype = ci
    lib.oracle_set_num_threads.argtypes = [ci]
    _lib = lib
    return lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def _f64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def build_segments(family: int, k, v, log_alpha, seg_offsets, beta=None, init_S=None,
                   want_P: bool = True) -> Tuple[np.ndarray, Optional[np.ndarray], np.ndarray]:
    """Records of every segment and head of a packed stream.

    k [N,H,dk], v [N,H,dv], beta [N,H] or None (= 1), log_alpha [N,H] (scalar,
    GDN) or [N,H,dk] (diagonal), seg_offsets [num_segments+1].  init_S
    [num_segments,H,dk,dv] or None (zero start).
    Returns ell [segs,H] (or [segs,H,dk]), P [segs,H,dk,dk] (GDN and want_P, else
    None) and S [segs,H,dk,dv], all fp64.
    """
    lib = _load()
    k, v, la, b, s0 = _f64(k), _f64(v), _f64(log_alpha), _f64(beta), _f64(init_S)
    offs = np.ascontiguousarray(np.asarray(seg_offsets, dtype=np.int64))
    N, H, dk = k.shape
    dv = v.shape[2]
    nseg = offs.shape[0] - 1
    assert v.shape[:2] == (N, H)
    if family == DIAGONAL:
        assert la.shape == (N, H, dk)
        ell = np.zeros((nseg, H, dk))
    elif family == KDA:
        assert la.shape == (N, H, dk)
        ell = np.zeros((nseg, H))
    else:
        assert la.shape == (N, H)
        ell = np.zeros((nseg, H))
    if b is not None:
        assert b.shape == (N, H)
    P = np.zeros((nseg, H, dk, dk)) if (family in (GDN, KDA) and want_P) else None
    S = np.zeros((nseg, H, dk, dv))
    rc = lib.oracle_build_segments(family, H, dk, dv, nseg, _ptr(offs, ctypes.c_int64),
                                   _ptr(k), _ptr(v), _ptr(b), _ptr(la), _ptr(s0),
                                   _ptr(ell), _ptr(P), _ptr(S))
    if rc != 0:
        raise ValueError("oracle_build_segments: bad argument")
    return ell, P, S


def forward(family: int, k, v, q, log_alpha, seg_offsets, beta=None, init_S=None, want_P: bool = True):
    """In-segment outputs and records of a packed stream: the chunked prefill forward's
    definition, token by token.

    As build_segments, plus q [N,H,dk]: o [N,H,dv] with o[t,h] = S_t^T q_t, S_t the
    head's state right after token t, the recurrence restarting at each segment's
    first token from init_S[s] (or 0).  Returns (o, ell, P, S).
    """
    lib = _load()
    k, v, qq, la, b, s0 = _f64(k), _f64(v), _f64(q), _f64(log_alpha), _f64(beta), _f64(init_S)
    offs = np.ascontiguousarray(np.asarray(seg_offsets, dtype=np.int64))
    N, H, dk = k.shape
    dv = v.shape[2]
    nseg = offs.shape[0] - 1
    assert v.shape[:2] == (N, H) and qq.shape == (N, H, dk)
    if family in (DIAGONAL, KDA):
        assert la.shape == (N, H, dk)
    else:
        assert la.shape == (N, H)
    if b is not None:
        assert b.shape == (N, H)
    ell = np.zeros((nseg, H, dk)) if family == DIAGONAL else np.zeros((nseg, H))
    P = np.zeros((nseg, H, dk, dk)) if (family in (GDN, KDA) and want_P) else None
    S = np.zeros((nseg, H, dk, dv))
    o = np.zeros((N, H, dv))
    rc = lib.oracle_forward(family, H, dk, dv, nseg, _ptr(offs, ctypes.c_int64), _ptr(k), _ptr(v), _ptr(qq),
                            _ptr(b), _ptr(la), _ptr(s0), _ptr(ell), _ptr(P), _ptr(S), _ptr(o))
    if rc != 0:
        raise ValueError("oracle_forward: bad argument")
    return o, ell, P, S


def compose(family: int, pool_ell, pool_P, pool_S, chain_offsets, chain_slots, init_S=None,
            want_P: bool = False):
    """Compose pool records along chains (prompt order).

    pool_ell [slots,H] (or [slots,H,dk]), pool_P [slots,H,dk,dk] (GDN; else
    None), pool_S [slots,H,dk,dv]; chain r = chain_slots[off[r]:off[r+1]].
    Returns (S [R,H,dk,dv], ell [R,H] or [R,H,dk], P [R,H,dk,dk] or None).
    """
    lib = _load()
    pe, pP, pS, s0 = _f64(pool_ell), _f64(pool_P), _f64(pool_S), _f64(init_S)
    offs = np.ascontiguousarray(np.asarray(chain_offsets, dtype=np.int64))
    slots = np.ascontiguousarray(np.asarray(chain_slots, dtype=np.int32))
    nslots, H, dk, dv = pS.shape
    R = offs.shape[0] - 1
    out_S = np.zeros((R, H, dk, dv))
    out_ell = np.zeros((R, H, dk)) if family == DIAGONAL else np.zeros((R, H))
    out_P = np.zeros((R, H, dk, dk)) if (family in (GDN, KDA) and want_P) else None
    rc = lib.oracle_compose(family, H, dk, dv, nslots, _ptr(pe), _ptr(pP), _ptr(pS), R,
                            _ptr(offs, ctypes.c_int64), _ptr(slots, ctypes.c_int32),
                            _ptr(s0), _ptr(out_S), _ptr(out_ell), _ptr(out_P))
    if rc != 0:
        raise ValueError("oracle_compose: bad argument")
    return out_S, out_ell, out_P


def causal_conv(x, w, bias=None, act: int = 0) -> np.ndarray:
    """Causal depthwise conv over a raw stream x [n,C] with w [C,K], zero history."""
    lib = _load()
    x, w, b = _f64(x), _f64(w), _f64(bias)
    n, C = x.shape
    K = w.shape[1]
    y = np.zeros((n, C))
    rc = lib.oracle_causal_conv(n, C, K, _ptr(x), _ptr(w), _ptr(b), int(act), _ptr(y))
    if rc != 0:
        raise ValueError("oracle_causal_conv: bad argument")
    return y


def rel_fro(x, ref) -> float:
    """||x - ref||_F / ||ref||_F, or the absolute norm when ref is all zero."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = float(np.linalg.norm((x - ref).ravel()))
    den = float(np.linalg.norm(ref.ravel()))
    return num / den if den > 0 else num


def conv_kv(x, w, bias, act: int, H: int, dk: int, dv: int, normalize: bool = True, eps: float = 1e-6):
    """Keys and values of a conv variant over a raw stream x [n, C] (C = H (dk + dv),
    zero history at its start): the causal conv and activation of causal_conv, the
    channels split into keys [n, H, dk] and values [n, H, dv], each head's key
    divided by sqrt(|k|^2 + eps) (besthub article, paragraph 4: the convolution
    state the warm-up keeps aligned is this conv's)."""
    y = causal_conv(x, w, bias, act)
    n = y.shape[0]
    k = y[:, :H * dk].reshape(n, H, dk)
    v = y[:, H * dk:].reshape(n, H, dv).copy()
    if normalize:
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    return k, v
