"""Shared helpers of the GPU parity tests: run the HIP path, read back the exact
bytes it saw, and evaluate the fp64 oracle on chosen (segment, head) units."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import hybrid_prefill_amd as hp
import oracle
from oracle import rel_fro

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def dev_i64(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.int64)).to("cuda")


def dev_i32(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).to("cuda")


def full_log_alpha(family, la: torch.Tensor, N: int, H: int) -> np.ndarray:
    """The per-token log decay the oracle needs ([N,H] or [N,H,d_k]), fp64."""
    if la is None:
        return np.zeros((N, H))
    a = np64(la)
    if family != oracle.DIAGONAL and a.ndim == 1:     # per-head constant
        return np.broadcast_to(a, (N, H)).copy()
    return a


def oracle_unit(family, k, v, la_full, beta, t0, t1, h, init_S=None):
    """Oracle record of tokens [t0,t1) of head h (inputs: fp64 numpy full arrays)."""
    sl = slice(t0, t1)
    b = None if beta is None else beta[sl, h:h + 1]
    la = la_full[sl, h:h + 1]
    s0 = None if init_S is None else init_S[None, None]
    ell, P, S = oracle.build_segments(family, k[sl, h:h + 1], v[sl, h:h + 1], la, [0, t1 - t0],
                                      beta=b, init_S=s0)
    return ell[0, 0], (None if P is None else P[0, 0]), S[0, 0]


def record_errors(family, ell_g, P_g, S_g, ell_r, P_r, S_r):
    """(S error, T error, |ell| error) of one record against the oracle's."""
    eS = rel_fro(S_g, S_r)
    dl = float(np.max(np.abs(np.asarray(ell_g, dtype=np.float64) - ell_r)))
    if family == oracle.GDN:
        # e^{ell_g} P_g vs e^{ell_r} P_r, scaled by e^{-ell_r} (no underflow)
        eT = rel_fro(math.exp(float(ell_g) - float(ell_r)) * P_g, P_r)
    elif family == oracle.SCALAR:
        eT = abs(math.expm1(float(ell_g) - float(ell_r)))
    else:
        eT = float(np.max(np.abs(np.expm1(np.asarray(ell_g, dtype=np.float64) - ell_r))))
    return eS, eT, dl


def composed_P_errors(ell_g, P_g, ell_r, P_r):
    """(P error, ell error) of a composed operator T = e^ell P against a reference
    (ell_r, P_r).  The compose may move an exact power of two 2^k from P into ell
    (renormalisation against underflow), so k = round((ell_g - ell_r) / ln 2) is taken
    out first: P error = |2^k P_g - P_r| / |P_r|, ell error = |ell_g - ell_r - k ln 2|."""
    d = float(ell_g) - float(ell_r)
    k = int(round(d / math.log(2.0)))
    return rel_fro(np.ldexp(np.asarray(P_g, dtype=np.float64), k), P_r), abs(d - k * math.log(2.0))
