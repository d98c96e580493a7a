"""Python binding of libhypic (ctypes): argument marshalling only.

Every step of the hot path runs in the HIP kernels of ``libhypic.so``; this
module only turns torch tensors into device pointers, strides and the current
HIP stream, and allocates outputs the caller did not pass.  The names follow
the C ABI in ``include/hypic.h``:

* :func:`build_segment`  -- records ``(ell, P, S)`` of segments into pool slots
* :func:`prefill_segment` -- the chunked prefill forward's in-segment outputs
  ``o_t = S_t^T q_t``, with the records as optional side-outputs
* :func:`compose_chain`  -- fold pool records along request chains
* :func:`compose_chain_heads` -- the same with a few tokens applied to the state
  before each record (the warmed first tokens of reused conv-variant segments)
* :func:`conv_warmup`    -- short-conv outputs at segment starts with the
  previous segment's tail as conv state
* :func:`conv_kv`        -- keys and values of chosen tokens of a conv variant
  (causal conv over given window rows, activation, per-head key L2 norm)

There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

SCALAR, DIAGONAL, GDN, KDA = 0, 1, 2, 3
F32, BF16 = 0, 1
EFLAG_SLOT_OUT_OF_RANGE = 0x1
EFLAG_BAD_OFFSETS = 0x2

_HERE = os.path.dirname(os.path.abspath(__file__))
# HYPIC_LIB names another build of the same library (the host-sanitized copy that the
# sanitizer test loads); by default the in-tree libhypic.so
LIB_PATH = os.environ.get("HYPIC_LIB") or os.path.join(_HERE, "libhypic.so")
_lib = None


class HypicError(RuntimeError):
    pass


class _Pool(ctypes.Structure):
    _fields_ = [("family", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("num_slots", ctypes.c_int64),
                ("log_scale", ctypes.c_void_p), ("P", ctypes.c_void_p), ("S", ctypes.c_void_p)]


class _Segments(ctypes.Structure):
    _fields_ = [("family", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("num_segments", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("num_tokens", ctypes.c_int64),
                ("seg_offsets", ctypes.c_void_p),
                ("k", ctypes.c_void_p), ("k_stride_t", ctypes.c_int64), ("k_stride_h", ctypes.c_int64),
                ("v", ctypes.c_void_p), ("v_stride_t", ctypes.c_int64), ("v_stride_h", ctypes.c_int64),
                ("beta", ctypes.c_void_p), ("beta_stride_t", ctypes.c_int64), ("beta_stride_h", ctypes.c_int64),
                ("log_alpha", ctypes.c_void_p), ("la_stride_t", ctypes.c_int64), ("la_stride_h", ctypes.c_int64)]


EXPORTED = ("hypic_build_segment", "hypic_prefill_segment", "hypic_compose_chain", "hypic_compose_chain_heads", "hypic_conv_warmup",
            "hypic_conv_kv", "hypic_status_string", "hypic_abi_version")


def lib():
    """Load libhypic.so (built in-tree by ``hybrid_prefill_amd._build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise HypicError(f"{LIB_PATH} is missing: build it with `python -m hybrid_prefill_amd._build` "
                         "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.hypic_build_segment.argtypes = [ctypes.POINTER(_Segments), ctypes.POINTER(_Pool), vp, vp, vp]
    L.hypic_build_segment.restype = i32
    L.hypic_prefill_segment.argtypes = [ctypes.POINTER(_Segments), vp, i64, i64, vp, i64, i64, i32,
                                        ctypes.POINTER(_Pool), vp, vp, vp]
    L.hypic_prefill_segment.restype = i32
    L.hypic_compose_chain.argtypes = [ctypes.POINTER(_Pool), i32, vp, vp, i64, vp, vp, vp, vp, vp, vp]
    L.hypic_compose_chain.restype = i32
    L.hypic_conv_warmup.argtypes = [i32, i32, i32, i32, vp, i64, vp, vp, i64, vp, vp, vp, i32, vp, vp, vp]
    L.hypic_conv_warmup.restype = i32
    L.hypic_conv_kv.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, vp, i32, i32, i32, vp, vp,
                                vp, i64, vp, vp, vp, vp, vp, vp]
    L.hypic_conv_kv.restype = i32
    L.hypic_compose_chain_heads.argtypes = [ctypes.POINTER(_Pool), i32, vp, vp, i64, vp, i64, vp, vp, vp, vp,
                                            vp, vp, vp, vp, vp]
    L.hypic_compose_chain_heads.restype = i32
    L.hypic_status_string.argtypes = [i32]
    L.hypic_status_string.restype = ctypes.c_char_p
    L.hypic_abi_version.restype = i32
    _lib = L
    return L


def _check(rc: int, what: str) -> None:
    if rc != 0:
        msg = lib().hypic_status_string(rc).decode()
        raise HypicError(f"{what}: {msg} (status {rc})")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise HypicError(f"unsupported dtype {t.dtype} (fp32 or bf16)")


def _device_check(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise HypicError("every tensor must be on the GPU")


def _shape(name: str, t: Optional[torch.Tensor], want) -> None:
    """The C ABI receives no sizes for most tensors, so a tensor of the wrong shape would
    become an out-of-bounds device access: every shape is checked here, before the call."""
    if t is not None and tuple(t.shape) != tuple(want):
        raise HypicError(f"{name} has shape {tuple(t.shape)}, expected {tuple(want)}")


def _flag(err_flag: Optional[torch.Tensor]) -> None:
    """The error word is one 32-bit device word the kernels OR into."""
    if err_flag is not None and (err_flag.dtype != torch.int32 or err_flag.numel() < 1
                                 or not err_flag.is_contiguous()):
        raise HypicError("err_flag must be a contiguous int32 tensor with at least one element")


@dataclass
class Pool:
    """Caller-owned segment pool: per (slot, head) record (log_scale, P, S), fp32."""
    family: int
    num_heads: int
    d_k: int
    d_v: int
    log_scale: torch.Tensor          # [slots,H] or [slots,H,d_k] (diagonal)
    S: torch.Tensor                  # [slots,H,d_k,d_v]
    P: Optional[torch.Tensor] = None  # [slots,H,d_k,d_k] (GDN)

    @property
    def num_slots(self) -> int:
        return self.S.shape[0]

    @staticmethod
    def allocate(family: int, num_slots: int, num_heads: int, d_k: int, d_v: int, device="cuda",
                 fill: Optional[float] = None) -> "Pool":
        ls_shape = (num_slots, num_heads, d_k) if family == DIAGONAL else (num_slots, num_heads)
        mk = (lambda s: torch.full(s, fill, dtype=torch.float32, device=device)) if fill is not None \
            else (lambda s: torch.empty(s, dtype=torch.float32, device=device))
        P = mk((num_slots, num_heads, d_k, d_k)) if family in (GDN, KDA) else None
        return Pool(family, num_heads, d_k, d_v, mk(ls_shape), mk((num_slots, num_heads, d_k, d_v)), P)

    def _validate(self) -> None:
        """dtype, layout and full shape of every pool tensor (no device access)."""
        for t in (self.log_scale, self.S, self.P):
            if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
                raise HypicError("pool tensors must be contiguous fp32")
        n, H, dk, dv = self.S.shape[0], self.num_heads, self.d_k, self.d_v
        _shape("pool.S", self.S, (n, H, dk, dv))
        _shape("pool.log_scale", self.log_scale, (n, H, dk) if self.family == DIAGONAL else (n, H))
        if self.family in (GDN, KDA):
            if self.P is None:
                raise HypicError("a GDN / KDA pool needs P")
            _shape("pool.P", self.P, (n, H, dk, dk))
        elif self.P is not None:
            raise HypicError("only GDN / KDA pools hold P")

    def _c(self) -> _Pool:
        self._validate()
        _device_check(self.log_scale, self.S, self.P)
        return _Pool(self.family, self.num_heads, self.d_k, self.d_v, self.num_slots,
                     _ptr(self.log_scale), _ptr(self.P), _ptr(self.S))


def _segments(family: int, k: torch.Tensor, v: torch.Tensor, log_alpha: Optional[torch.Tensor],
              seg_offsets: torch.Tensor, beta: Optional[torch.Tensor]) -> _Segments:
    """Shape and dtype checks of a packed token stream, then its C descriptor (no device access)."""
    if k.dtype != v.dtype:
        raise HypicError("k and v must share a dtype")
    if k.dim() != 3 or v.dim() != 3 or k.stride(2) != 1 or v.stride(2) != 1:
        raise HypicError("k, v must be [N,H,d] with unit channel stride")
    if seg_offsets.dtype != torch.int64 or seg_offsets.dim() != 1 or seg_offsets.numel() < 1:
        raise HypicError("seg_offsets must be 1-D int64 with num_segments + 1 entries")
    N, H, dk = k.shape
    dv = v.shape[2]
    _shape("v", v, (N, H, dv))
    la_st = la_sh = 0
    if log_alpha is not None:
        if log_alpha.dtype != torch.float32:
            raise HypicError("log_alpha must be fp32")
        if family in (DIAGONAL, KDA):
            _shape("log_alpha", log_alpha, (N, H, dk))
            if log_alpha.stride(2) != 1:
                raise HypicError("per-channel log_alpha must be [N,H,d_k] with unit channel stride")
            la_st, la_sh = log_alpha.stride(0), log_alpha.stride(1)
        elif log_alpha.dim() == 1:
            _shape("log_alpha", log_alpha, (H,))
            la_st, la_sh = 0, log_alpha.stride(0)
        else:
            _shape("log_alpha", log_alpha, (N, H))
            la_st, la_sh = log_alpha.stride(0), log_alpha.stride(1)
    b_st = b_sh = 0
    if beta is not None:
        if beta.dtype != torch.float32:
            raise HypicError("beta must be fp32 [N,H]")
        _shape("beta", beta, (N, H))
        b_st, b_sh = beta.stride(0), beta.stride(1)
    return _Segments(family, H, dk, dv, seg_offsets.numel() - 1, _dtype_code(k), N,
                     _ptr(seg_offsets),
                     _ptr(k), k.stride(0), k.stride(1),
                     _ptr(v), v.stride(0), v.stride(1),
                     _ptr(beta), b_st, b_sh,
                     _ptr(log_alpha), la_st, la_sh)


def _pool_for(pool: Pool, family: int, H: int, dk: int, dv: int, dst_slots: torch.Tensor, nseg: int) -> None:
    pool._validate()
    if (pool.family, pool.num_heads, pool.d_k, pool.d_v) != (family, H, dk, dv):
        raise HypicError(f"pool (family {pool.family}, H={pool.num_heads}, d_k={pool.d_k}, d_v={pool.d_v}) "
                         f"does not match the stream (family {family}, H={H}, d_k={dk}, d_v={dv})")
    if dst_slots.dtype != torch.int32:
        raise HypicError("dst_slots must be int32")
    _shape("dst_slots", dst_slots, (nseg,))


def build_segment(family: int, k: torch.Tensor, v: torch.Tensor, log_alpha: Optional[torch.Tensor],
                  seg_offsets: torch.Tensor, pool: Pool, dst_slots: torch.Tensor,
                  beta: Optional[torch.Tensor] = None, err_flag: Optional[torch.Tensor] = None,
                  stream=None) -> None:
    """hypic_build_segment: records of every segment of a packed stream into pool slots.

    k [N,H,d_k], v [N,H,d_v] (bf16 or fp32, unit channel stride); log_alpha
    [N,H] (scalar, GDN), [H] broadcast per head (constant decay) or [N,H,d_k]
    (diagonal), fp32, or None (no decay); beta [N,H] fp32 or None (= 1);
    seg_offsets device int64 [S+1]; dst_slots device int32 [S].
    """
    seg = _segments(family, k, v, log_alpha, seg_offsets, beta)
    _pool_for(pool, family, seg.num_heads, seg.d_k, seg.d_v, dst_slots, seg.num_segments)
    _flag(err_flag)
    _device_check(k, v, log_alpha, seg_offsets, dst_slots, beta, err_flag)
    cpool = pool._c()
    rc = lib().hypic_build_segment(ctypes.byref(seg), ctypes.byref(cpool), _ptr(dst_slots),
                                   _ptr(err_flag), _stream(stream))
    _check(rc, "hypic_build_segment")


def prefill_segment(family: int, k: torch.Tensor, v: torch.Tensor, q: Optional[torch.Tensor],
                    log_alpha: Optional[torch.Tensor], seg_offsets: torch.Tensor,
                    beta: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    out_dtype=torch.float32, pool: Optional[Pool] = None,
                    dst_slots: Optional[torch.Tensor] = None, outputs: bool = True,
                    err_flag: Optional[torch.Tensor] = None, stream=None) -> Optional[torch.Tensor]:
    """hypic_prefill_segment: the chunked prefill forward of every segment (zero state
    at each segment's first token), o_t = S_t^T q_t for every token, and with a pool
    the records (ell, P, S) into dst_slots as build_segment writes them.

    q [N,H,d_k] in k's dtype; out [N,H,d_v] fp32 or bf16 (allocated when None).
    outputs=False: the records alone (q and out unused).  Returns out (or None).
    """
    seg = _segments(family, k, v, log_alpha, seg_offsets, beta)
    N, H, dk, dv = seg.num_tokens, seg.num_heads, seg.d_k, seg.d_v
    if pool is not None:
        if dst_slots is None:
            raise HypicError("a pool needs dst_slots")
        _pool_for(pool, family, H, dk, dv, dst_slots, seg.num_segments)
    elif not outputs:
        raise HypicError("nothing to compute: no outputs and no pool")
    q_st = q_sh = o_st = o_sh = 0
    o_code = F32
    if outputs:
        if q is None:
            raise HypicError("outputs need q")
        if q.dtype != k.dtype or q.dim() != 3 or q.stride(2) != 1:
            raise HypicError("q must be [N,H,d_k] in k's dtype with unit channel stride")
        _shape("q", q, (N, H, dk))
        if out is None:
            out = torch.empty((N, H, dv), dtype=out_dtype, device=k.device)
        if out.dim() != 3 or out.stride(2) != 1:
            raise HypicError("out must be [N,H,d_v] with unit channel stride")
        _shape("out", out, (N, H, dv))
        o_code = _dtype_code(out)
        q_st, q_sh, o_st, o_sh = q.stride(0), q.stride(1), out.stride(0), out.stride(1)
    else:
        q = out = None
    _flag(err_flag)
    _device_check(k, v, q, out, log_alpha, seg_offsets, dst_slots, beta, err_flag)
    cpool = pool._c() if pool is not None else None
    rc = lib().hypic_prefill_segment(ctypes.byref(seg), _ptr(q), q_st, q_sh, _ptr(out), o_st, o_sh, o_code,
                                     None if cpool is None else ctypes.byref(cpool),
                                     _ptr(dst_slots) if pool is not None else None, _ptr(err_flag),
                                     _stream(stream))
    _check(rc, "hypic_prefill_segment")
    return out


def _compose_shapes(pool: Pool, R: int, init_S, out_S, out_log_scale, out_P=None) -> None:
    H, dk, dv = pool.num_heads, pool.d_k, pool.d_v
    _shape("init_S", init_S, (R, H, dk, dv))
    _shape("out_S", out_S, (R, H, dk, dv))
    _shape("out_log_scale", out_log_scale, (R, H, dk) if pool.family == DIAGONAL else (R, H))
    if out_P is not None and pool.family not in (GDN, KDA):
        raise HypicError("out_P needs a GDN / KDA pool")
    if out_P is not None and out_log_scale is None:
        raise HypicError("out_P needs out_log_scale (the composed operator is e^ell P)")
    _shape("out_P", out_P, (R, H, dk, dk))


def compose_chain(pool: Pool, chain_offsets: torch.Tensor, chain_slots: torch.Tensor,
                  init_S: Optional[torch.Tensor] = None, out_S: Optional[torch.Tensor] = None,
                  out_log_scale: Optional[torch.Tensor] = None, out_P: Optional[torch.Tensor] = None,
                  err_flag: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """hypic_compose_chain: S <- T_i S + S_i along each chain; returns out_S [R,H,d_k,d_v]."""
    if chain_offsets.dtype != torch.int64 or chain_slots.dtype != torch.int32:
        raise HypicError("chain_offsets must be int64 and chain_slots int32")
    if chain_offsets.dim() != 1 or chain_offsets.numel() < 1 or chain_slots.dim() != 1:
        raise HypicError("chain_offsets must be 1-D [R+1] and chain_slots 1-D")
    R = chain_offsets.numel() - 1
    if out_S is None:
        out_S = torch.empty((R, pool.num_heads, pool.d_k, pool.d_v), dtype=torch.float32,
                            device=pool.S.device)
    for t in (init_S, out_S, out_log_scale, out_P):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise HypicError("state tensors must be contiguous fp32")
    pool._validate()
    _compose_shapes(pool, R, init_S, out_S, out_log_scale, out_P)
    _flag(err_flag)
    _device_check(chain_offsets, chain_slots, init_S, out_S, out_log_scale, out_P, err_flag)
    cpool = pool._c()
    rc = lib().hypic_compose_chain(ctypes.byref(cpool), R, _ptr(chain_offsets), _ptr(chain_slots),
                                   chain_slots.numel(), _ptr(init_S), _ptr(out_S), _ptr(out_log_scale),
                                   _ptr(out_P), _ptr(err_flag), _stream(stream))
    _check(rc, "hypic_compose_chain")
    return out_S


def compose_chain_heads(pool: Pool, chain_offsets: torch.Tensor, chain_slots: torch.Tensor,
                        head_offsets: torch.Tensor, head_k: torch.Tensor, head_v: torch.Tensor,
                        head_beta: torch.Tensor, head_log_alpha: torch.Tensor,
                        init_S: Optional[torch.Tensor] = None, out_S: Optional[torch.Tensor] = None,
                        out_log_scale: Optional[torch.Tensor] = None, err_flag: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """hypic_compose_chain_heads: each chain entry applies its head tokens, then folds its
    record; head_k [T,H,d_k], head_v [T,H,d_v], head_beta / head_log_alpha [T,H] fp32."""
    if chain_offsets.dtype != torch.int64 or chain_slots.dtype != torch.int32 or head_offsets.dtype != torch.int64:
        raise HypicError("chain_offsets / head_offsets must be int64 and chain_slots int32")
    if chain_offsets.dim() != 1 or chain_offsets.numel() < 1 or chain_slots.dim() != 1:
        raise HypicError("chain_offsets must be 1-D [R+1] and chain_slots 1-D")
    _shape("head_offsets", head_offsets, (chain_slots.numel() + 1,))
    T = head_k.shape[0]
    H, dk, dv = pool.num_heads, pool.d_k, pool.d_v
    _shape("head_k", head_k, (T, H, dk))
    _shape("head_v", head_v, (T, H, dv))
    _shape("head_beta", head_beta, (T, H))
    _shape("head_log_alpha", head_log_alpha, (T, H))
    for t_ in (head_k, head_v, head_beta, head_log_alpha):
        if t_.dtype != torch.float32 or not t_.is_contiguous():
            raise HypicError("head tensors must be contiguous fp32 with one row per head token")
    R = chain_offsets.numel() - 1
    if out_S is None:
        out_S = torch.empty((R, pool.num_heads, pool.d_k, pool.d_v), dtype=torch.float32, device=pool.S.device)
    for t_ in (init_S, out_S, out_log_scale):
        if t_ is not None and (t_.dtype != torch.float32 or not t_.is_contiguous()):
            raise HypicError("state tensors must be contiguous fp32")
    pool._validate()
    _compose_shapes(pool, R, init_S, out_S, out_log_scale)
    _flag(err_flag)
    _device_check(chain_offsets, chain_slots, head_offsets, head_k, head_v, head_beta, head_log_alpha,
                  init_S, out_S, out_log_scale, err_flag)
    cpool = pool._c()
    none = T == 0
    rc = lib().hypic_compose_chain_heads(ctypes.byref(cpool), R, _ptr(chain_offsets), _ptr(chain_slots),
                                         chain_slots.numel(), _ptr(head_offsets), T,
                                         None if none else _ptr(head_k), None if none else _ptr(head_v),
                                         None if none else _ptr(head_beta), None if none else _ptr(head_log_alpha),
                                         _ptr(init_S), _ptr(out_S), _ptr(out_log_scale), _ptr(err_flag),
                                         _stream(stream))
    _check(rc, "hypic_compose_chain_heads")
    return out_S


def conv_warmup(tails: torch.Tensor, heads: torch.Tensor, weight: torch.Tensor,
                bias: Optional[torch.Tensor] = None, activation: int = 0,
                tail_index: Optional[torch.Tensor] = None, head_index: Optional[torch.Tensor] = None,
                num_boundaries: Optional[int] = None, out: Optional[torch.Tensor] = None,
                err_flag: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """hypic_conv_warmup: tails/heads [rows,K-1,C] raw inputs, weight [C,K]; returns out [B,K-1,C] fp32."""
    if tails.dtype != heads.dtype or not tails.is_contiguous() or not heads.is_contiguous():
        raise HypicError("tails and heads must be contiguous and share a dtype")
    if weight.dim() != 2:
        raise HypicError("weight must be [C,K]")
    C, K = weight.shape
    if weight.dtype != torch.float32 or not weight.is_contiguous():
        raise HypicError("weight must be contiguous fp32 [C,K]")
    if tails.dim() != 3 or heads.dim() != 3 or tails.shape[1:] != (K - 1, C) or heads.shape[1:] != (K - 1, C):
        raise HypicError("tails/heads must be [rows, K-1, C]")
    for ix in (tail_index, head_index):
        if ix is not None and (ix.dtype != torch.int32 or ix.dim() != 1 or not ix.is_contiguous()):
            raise HypicError("indices must be contiguous 1-D int32")
    if num_boundaries is None:
        num_boundaries = tail_index.numel() if tail_index is not None else (
            head_index.numel() if head_index is not None else tails.shape[0])
    for name, ix, table in (("tail_index", tail_index, tails), ("head_index", head_index, heads)):
        n_have = ix.numel() if ix is not None else table.shape[0]
        if n_have < num_boundaries:
            raise HypicError(f"{name if ix is not None else name[:4] + 's'} covers {n_have} boundaries, "
                             f"needs {num_boundaries}")
    _shape("bias", bias, (C,))
    if bias is not None and (bias.dtype != torch.float32 or not bias.is_contiguous()):
        raise HypicError("bias must be contiguous fp32 [C]")
    if out is None:
        out = torch.empty((num_boundaries, K - 1, C), dtype=torch.float32, device=weight.device)
    _shape("out", out, (num_boundaries, K - 1, C))
    if out.dtype != torch.float32 or not out.is_contiguous():
        raise HypicError("out must be contiguous fp32 [B, K-1, C]")
    _flag(err_flag)
    _device_check(tails, heads, weight, bias, tail_index, head_index, out, err_flag)
    rc = lib().hypic_conv_warmup(num_boundaries, C, K, _dtype_code(tails),
                                 _ptr(tails), tails.shape[0], _ptr(tail_index),
                                 _ptr(heads), heads.shape[0], _ptr(head_index),
                                 _ptr(weight), _ptr(bias), int(activation), _ptr(out), _ptr(err_flag),
                                 _stream(stream))
    _check(rc, "hypic_conv_warmup")
    return out


def conv_kv(x: torch.Tensor, window: torch.Tensor, weight: torch.Tensor, num_heads: int, d_k: int, d_v: int,
            bias: Optional[torch.Tensor] = None, activation: int = 1, normalize_k: bool = True,
            out_dtype=torch.bfloat16, src_token: Optional[torch.Tensor] = None,
            beta: Optional[torch.Tensor] = None, log_alpha: Optional[torch.Tensor] = None,
            err_flag: Optional[torch.Tensor] = None, stream=None):
    """hypic_conv_kv: x [rows, C] raw inputs, window [T, K] int32 rows (-1 = zero), weight [C, K].
    Returns (k [T, H, d_k], v [T, H, d_v]) and, with src_token, (beta [T, H], log_alpha [T, H])."""
    if weight.dim() != 2:
        raise HypicError("weight must be [C, K]")
    C, K = weight.shape
    if C != num_heads * (d_k + d_v):
        raise HypicError("weight must have H (d_k + d_v) channels")
    if not x.is_contiguous() or x.dim() != 2 or x.shape[1] != C:
        raise HypicError("x must be contiguous [rows, C]")
    if weight.dtype != torch.float32 or not weight.is_contiguous():
        raise HypicError("weight must be contiguous fp32 [C, K]")
    if window.dtype != torch.int32 or not window.is_contiguous() or window.dim() != 2 or window.shape[1] != K:
        raise HypicError("window must be contiguous int32 [T, K]")
    T = window.shape[0]
    for t_ in (beta, log_alpha):
        if t_ is not None and (t_.dtype != torch.float32 or not t_.is_contiguous() or t_.shape[-1] != num_heads):
            raise HypicError("beta / log_alpha must be contiguous fp32 [N, H]")
    if src_token is not None and (src_token.dtype != torch.int32 or src_token.numel() != T
                                  or not src_token.is_contiguous()):
        raise HypicError("src_token must be contiguous int32 [T]")
    if beta is not None and log_alpha is not None and beta.shape != log_alpha.shape:
        raise HypicError("beta and log_alpha must both be [N, H]")
    for t_ in (beta, log_alpha):
        if t_ is not None and t_.dim() != 2:
            raise HypicError("beta / log_alpha must be contiguous fp32 [N, H]")
    _shape("bias", bias, (C,))
    if bias is not None and (bias.dtype != torch.float32 or not bias.is_contiguous()):
        raise HypicError("bias must be contiguous fp32 [C]")
    _flag(err_flag)
    _device_check(x, window, weight, bias, src_token, beta, log_alpha, err_flag)
    dev = weight.device
    k = torch.empty((T, num_heads, d_k), dtype=out_dtype, device=dev)
    v = torch.empty((T, num_heads, d_v), dtype=out_dtype, device=dev)
    b_out = la_out = None
    n_src = 0
    if src_token is not None:
        b_out = torch.empty((T, num_heads), dtype=torch.float32, device=dev)
        la_out = torch.empty((T, num_heads), dtype=torch.float32, device=dev)
        n_src = (beta if beta is not None else log_alpha).shape[0] if (beta is not None or log_alpha is not None) \
            else 2 ** 31 - 1
    rc = lib().hypic_conv_kv(T, num_heads, d_k, d_v, K, _dtype_code(x), _ptr(x), x.shape[0], _ptr(window),
                             _ptr(weight), _ptr(bias), int(activation), int(bool(normalize_k)),
                             F32 if out_dtype == torch.float32 else BF16, _ptr(k), _ptr(v),
                             _ptr(src_token), n_src, _ptr(beta), _ptr(log_alpha), _ptr(b_out), _ptr(la_out),
                             _ptr(err_flag), _stream(stream))
    _check(rc, "hypic_conv_kv")
    return (k, v) if src_token is None else (k, v, b_out, la_out)
