"""Host-side checks of the C ABI (no GPU needed, no compute call).

* libhypic.so loads and exports every function include/hypic.h declares;
* synchronous argument validation rejects bad calls before any HIP call.
"""
import ctypes
import os
import re

import pytest

import hybrid_prefill_amd as hp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hypic.h")

INVALID, UNSUPPORTED = 1, 2


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(hypic_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hp.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return hp.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(hp.EXPORTED) <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in hypic.h but not exported"


def test_version_and_status_strings(L):
    assert L.hypic_abi_version() == 1
    assert L.hypic_status_string(0) == b"ok"
    assert L.hypic_status_string(1) == b"invalid argument"
    assert L.hypic_status_string(2) == b"unsupported configuration"
    assert L.hypic_status_string(3) == b"HIP launch error"
    assert L.hypic_status_string(99) == b"unknown status"


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def pool(family=hp.GDN, H=2, dk=64, dv=64, slots=4, P=True):
    return hp._Pool(family, H, dk, dv, slots, FAKE, FAKE if P else None, FAKE)


def segs(family=hp.GDN, H=2, dk=64, dv=64, nseg=1, dtype=hp.BF16, N=10, **kw):
    s = hp._Segments(family, H, dk, dv, nseg, dtype, N, FAKE, FAKE, 64 * H, 64, FAKE, 64 * H, 64,
                     None, 0, 0, FAKE, H, 1)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def build(L, s, p, slots=FAKE):
    return L.hypic_build_segment(ctypes.byref(s) if s is not None else None,
                                 ctypes.byref(p) if p is not None else None, slots, None, None)


def test_build_validation(L):
    assert build(L, None, pool()) == INVALID
    assert build(L, segs(), None) == INVALID
    assert build(L, segs(dk=96), pool(dk=96)) == UNSUPPORTED
    assert build(L, segs(dv=32), pool(dv=32)) == UNSUPPORTED
    assert build(L, segs(family=7), pool()) == UNSUPPORTED
    assert build(L, segs(dtype=5), pool()) == UNSUPPORTED
    assert build(L, segs(family=hp.SCALAR), pool()) == INVALID          # family mismatch
    assert build(L, segs(H=3), pool()) == INVALID                       # head count mismatch
    assert build(L, segs(), pool(P=False)) == INVALID                   # GDN pool needs P
    assert build(L, segs(family=hp.SCALAR), pool(family=hp.SCALAR)) == INVALID  # P given for scalar
    assert build(L, segs(nseg=-1), pool()) == INVALID
    assert build(L, segs(N=-5), pool()) == INVALID
    assert build(L, segs(seg_offsets=None), pool()) == INVALID
    assert build(L, segs(), pool(), slots=None) == INVALID
    assert build(L, segs(k=None), pool()) == INVALID
    assert build(L, segs(k_stride_t=-1), pool()) == INVALID
    # nothing to do is not an error and launches nothing
    assert build(L, segs(nseg=0), pool()) == 0


def test_compose_validation(L):
    p = pool()
    c = L.hypic_compose_chain
    assert c(None, 1, FAKE, FAKE, 1, None, FAKE, None, None, None, None) == INVALID
    assert c(ctypes.byref(p), -1, FAKE, FAKE, 1, None, FAKE, None, None, None, None) == INVALID
    assert c(ctypes.byref(p), 1, None, FAKE, 1, None, FAKE, None, None, None, None) == INVALID
    assert c(ctypes.byref(p), 1, FAKE, FAKE, 1, None, None, None, None, None, None) == INVALID
    assert c(ctypes.byref(p), 1, FAKE, None, 3, None, FAKE, None, None, None, None) == INVALID
    assert c(ctypes.byref(p), 1, FAKE, FAKE, -2, None, FAKE, None, None, None, None) == INVALID
    ps = pool(family=hp.SCALAR, P=False)
    assert c(ctypes.byref(ps), 1, FAKE, FAKE, 1, None, FAKE, None, FAKE, None, None) == INVALID  # out_P for scalar
    assert c(ctypes.byref(p), 1, FAKE, FAKE, 1, None, FAKE, None, FAKE, None, None) == INVALID   # out_P without ell
    pbad = pool(dk=32)
    assert c(ctypes.byref(pbad), 1, FAKE, FAKE, 1, None, FAKE, None, None, None, None) == UNSUPPORTED
    assert c(ctypes.byref(p), 0, None, None, 0, None, None, None, None, None, None) == 0


def test_conv_validation(L):
    c = L.hypic_conv_warmup
    ok = dict(B=2, C=8, K=4, dt=hp.BF16, tails=FAKE, nt=2, ti=None, heads=FAKE, nh=2, hi=None,
              w=FAKE, b=None, act=0, out=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return c(a["B"], a["C"], a["K"], a["dt"], a["tails"], a["nt"], a["ti"], a["heads"], a["nh"],
                 a["hi"], a["w"], a["b"], a["act"], a["out"], None, None)

    assert call(K=1) == UNSUPPORTED
    assert call(K=9) == UNSUPPORTED
    assert call(dt=3) == UNSUPPORTED
    assert call(act=2) == UNSUPPORTED
    assert call(C=0) == INVALID
    assert call(B=-1) == INVALID
    assert call(tails=None) == INVALID
    assert call(w=None) == INVALID
    assert call(out=None) == INVALID
    assert call(nt=1) == INVALID        # fewer tails than boundaries and no index
    assert call(B=0) == 0


def test_ctypes_layout_matches_header(tmp_path):
    """The binding's ctypes structs have the C header's field offsets and sizes."""
    import subprocess
    src = tmp_path / "layout.c"
    fields = {"hypic_pool": [f for f, _ in hp._Pool._fields_],
              "hypic_segments": [f for f, _ in hp._Segments._fields_]}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "hypic.h"', "int main(void) {"]
    for T, fs in fields.items():
        for f in fs:
            lines.append(f'printf("{T} {f} %zu\\n", offsetof({T}, {f}));')
        lines.append(f'printf("{T} __size %zu\\n", sizeof({T}));')
    lines.append("return 0; }")
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    types = {"hypic_pool": hp._Pool, "hypic_segments": hp._Segments}
    n = 0
    for line in filter(None, out):
        T, f, off = line.split()
        want = ctypes.sizeof(types[T]) if f == "__size" else getattr(types[T], f).offset
        assert want == int(off), (T, f, want, off)
        n += 1
    assert n == sum(len(v) + 1 for v in fields.values())


def test_conv_kv_validation(L):
    c = L.hypic_conv_kv
    ok = dict(T=3, H=2, dk=4, dv=4, K=4, dt=hp.BF16, x=FAKE, rows=10, win=FAKE, w=FAKE, b=None, act=1,
              norm=1, odt=hp.BF16, k=FAKE, v=FAKE, src=None, nsrc=0, beta=None, la=None, bo=None, lo=None)

    def call(**kw):
        a = dict(ok, **kw)
        return c(a["T"], a["H"], a["dk"], a["dv"], a["K"], a["dt"], a["x"], a["rows"], a["win"], a["w"], a["b"],
                 a["act"], a["norm"], a["odt"], a["k"], a["v"], a["src"], a["nsrc"], a["beta"], a["la"],
                 a["bo"], a["lo"], None, None)

    assert call(K=0) == UNSUPPORTED
    assert call(K=9) == UNSUPPORTED
    assert call(dt=5) == UNSUPPORTED
    assert call(odt=5) == UNSUPPORTED
    assert call(act=3) == UNSUPPORTED
    assert call(H=65, dk=128, dv=128) == UNSUPPORTED     # conv row larger than the LDS row (16384)
    assert call(T=-1) == INVALID
    assert call(H=0) == INVALID
    assert call(x=None) == INVALID
    assert call(win=None) == INVALID
    assert call(k=None) == INVALID
    assert call(src=FAKE) == INVALID                     # src_token without beta_out / la_out
    assert call(T=0) == 0


def test_compose_chain_heads_validation(L):
    c = L.hypic_compose_chain_heads
    p = pool(dk=128, dv=128)

    def call(pp=p, R=1, offs=FAKE, slots=FAKE, ns=1, hoffs=FAKE, T=3, hk=FAKE, hv=FAKE, hb=FAKE, hl=FAKE,
             out=FAKE):
        return c(ctypes.byref(pp), R, offs, slots, ns, hoffs, T, hk, hv, hb, hl, None, out, None, None, None)

    # every call below fails validation before any launch
    assert call(pp=pool(dk=64, dv=64)) == UNSUPPORTED                       # fused compose: d = 128 only
    assert call(pp=pool(family=hp.SCALAR, dk=128, dv=128, P=False)) == UNSUPPORTED
    assert call(T=1 << 27) == UNSUPPORTED
    assert call(T=-1) == INVALID
    assert call(hoffs=None) == INVALID
    assert call(hk=None) == INVALID
    assert call(hl=None) == INVALID
    assert call(out=None) == INVALID
    assert call(T=0) == INVALID                                             # no tokens, but head pointers given
    assert call(R=0) == 0


# ----------------------------------------------------------------------------- binding shape checks
# The C ABI receives no sizes for most tensors, so the binding checks every shape before
# the call.  These run on CPU tensors: a wrong shape raises before the device check, a
# right one reaches the device check (the tensors are not on the GPU).

import torch  # noqa: E402


def _raises(fn, match):
    with pytest.raises(hp.HypicError, match=match):
        fn()


def test_build_segment_shape_checks():
    N, H, d = 10, 2, 64
    k = torch.zeros((N, H, d), dtype=torch.bfloat16)
    v = torch.zeros((N, H, d), dtype=torch.bfloat16)
    la = torch.zeros((N, H))
    beta = torch.zeros((N, H))
    offs = torch.tensor([0, 4, 10])
    slots = torch.tensor([0, 1], dtype=torch.int32)
    pool = hp.Pool.allocate(hp.GDN, 3, H, d, d, device="cpu")
    ok = dict(family=hp.GDN, k=k, v=v, log_alpha=la, seg_offsets=offs, pool=pool, dst_slots=slots, beta=beta)

    def call(**kw):
        return lambda: hp.build_segment(**dict(ok, **kw))

    _raises(call(), "on the GPU")                                            # shapes fine
    _raises(call(v=torch.zeros((N, H + 1, d), dtype=torch.bfloat16)), "v has shape")
    _raises(call(v=torch.zeros((N - 1, H, d), dtype=torch.bfloat16)), "v has shape")
    _raises(call(log_alpha=torch.zeros((N, H, d))), "log_alpha has shape")  # 3-D gates for GDN
    _raises(call(log_alpha=torch.zeros((N - 2, H))), "log_alpha has shape")
    _raises(call(log_alpha=torch.zeros((H + 1,))), "log_alpha has shape")
    _raises(call(beta=torch.zeros((N, H + 1))), "beta has shape")
    _raises(call(dst_slots=torch.tensor([0], dtype=torch.int32)), "dst_slots has shape")
    _raises(call(err_flag=torch.zeros(1, dtype=torch.int64)), "err_flag")
    _raises(call(pool=hp.Pool.allocate(hp.GDN, 3, H + 1, d, d, device="cpu")), "does not match")
    _raises(call(pool=hp.Pool.allocate(hp.SCALAR, 3, H, d, d, device="cpu")), "does not match")
    bad = hp.Pool.allocate(hp.GDN, 3, H, d, d, device="cpu")
    bad.P = torch.zeros((3, H, d, d + 1))
    _raises(call(pool=bad), "pool.P has shape")
    bad = hp.Pool.allocate(hp.GDN, 3, H, d, d, device="cpu")
    bad.log_scale = torch.zeros((3, H, d))
    _raises(call(pool=bad), "pool.log_scale has shape")
    # diagonal: per-channel gates [N,H,d_k]; a diagonal pool's log_scale is [slots,H,d_k]
    dpool = hp.Pool.allocate(hp.DIAGONAL, 3, H, d, d, device="cpu")
    _raises(call(family=hp.DIAGONAL, pool=dpool, beta=None, log_alpha=torch.zeros((N, H, d))), "on the GPU")
    _raises(call(family=hp.DIAGONAL, pool=dpool, beta=None, log_alpha=torch.zeros((N, H))), "log_alpha has shape")
    dpool.log_scale = torch.zeros((3, H))
    _raises(call(family=hp.DIAGONAL, pool=dpool, beta=None, log_alpha=torch.zeros((N, H, d))),
            "pool.log_scale has shape")


def test_prefill_segment_shape_checks():
    """hypic_prefill_segment's binding: q and out against [N,H,d_k] / [N,H,d_v], q in
    k's dtype, a pool needs dst_slots, and a call that computes nothing is refused, all
    before any device work."""
    N, H, d = 10, 2, 128
    k = torch.zeros((N, H, d), dtype=torch.bfloat16)
    v = torch.zeros((N, H, d), dtype=torch.bfloat16)
    q = torch.zeros((N, H, d), dtype=torch.bfloat16)
    la = torch.zeros((N, H))
    offs = torch.tensor([0, 4, 10])
    slots = torch.tensor([0, 1], dtype=torch.int32)
    pool = hp.Pool.allocate(hp.GDN, 3, H, d, d, device="cpu")
    ok = dict(family=hp.GDN, k=k, v=v, q=q, log_alpha=la, seg_offsets=offs)

    def call(**kw):
        return lambda: hp.prefill_segment(**dict(ok, **kw))

    _raises(call(out=torch.zeros((N, H, d))), "on the GPU")                         # shapes fine
    _raises(call(out=torch.zeros((N, H, d)), pool=pool, dst_slots=slots), "on the GPU")
    _raises(call(q=torch.zeros((N, H + 1, d), dtype=torch.bfloat16)), "q has shape")
    _raises(call(q=torch.zeros((N - 1, H, d), dtype=torch.bfloat16)), "q has shape")
    _raises(call(q=torch.zeros((N, H, d))), "q must be")                            # fp32 q, bf16 k
    _raises(call(q=None), "outputs need q")
    _raises(call(out=torch.zeros((N, H, d + 1))), "out has shape")
    _raises(call(out=torch.zeros((N, H, 2 * d))[:, :, ::2]), "unit channel stride")
    _raises(call(pool=pool), "needs dst_slots")
    _raises(call(pool=pool, dst_slots=torch.tensor([0], dtype=torch.int32)), "dst_slots has shape")
    _raises(call(outputs=False), "nothing to compute")
    _raises(call(out=torch.zeros((N, H, d)), err_flag=torch.zeros(1, dtype=torch.int64)), "err_flag")


def test_compose_shape_checks():
    H, d, R = 2, 64, 3
    pool = hp.Pool.allocate(hp.GDN, 4, H, d, d, device="cpu")
    offs = torch.tensor([0, 1, 2, 3])
    ids = torch.tensor([0, 1, 2], dtype=torch.int32)
    ok = dict(pool=pool, chain_offsets=offs, chain_slots=ids, out_S=torch.zeros((R, H, d, d)))

    def call(**kw):
        return lambda: hp.compose_chain(**dict(ok, **kw))

    _raises(call(), "on the GPU")
    _raises(call(out_S=torch.zeros((R - 1, H, d, d))), "out_S has shape")
    _raises(call(init_S=torch.zeros((R, H, d, d - 1))), "init_S has shape")
    _raises(call(out_log_scale=torch.zeros((R, H, d))), "out_log_scale has shape")
    _raises(call(out_log_scale=torch.zeros((R, H)), out_P=torch.zeros((R, H, d, 2 * d))), "out_P has shape")
    _raises(call(out_P=torch.zeros((R, H, d, d))), "out_P needs out_log_scale")
    spool = hp.Pool.allocate(hp.SCALAR, 4, H, d, d, device="cpu")
    _raises(call(pool=spool, out_P=torch.zeros((R, H, d, d))), "out_P needs")
    dpool = hp.Pool.allocate(hp.DIAGONAL, 4, H, d, d, device="cpu")
    _raises(call(pool=dpool, out_log_scale=torch.zeros((R, H))), "out_log_scale has shape")
    _raises(call(pool=dpool, out_log_scale=torch.zeros((R, H, d))), "on the GPU")
    # the fused head-token compose
    T = 5
    hk = dict(pool=pool, chain_offsets=offs, chain_slots=ids, head_offsets=torch.tensor([0, 2, 4, 5]),
              head_k=torch.zeros((T, H, d)), head_v=torch.zeros((T, H, d)), head_beta=torch.zeros((T, H)),
              head_log_alpha=torch.zeros((T, H)))

    def hcall(**kw):
        return lambda: hp.compose_chain_heads(**dict(hk, **kw))

    _raises(hcall(), "on the GPU")
    _raises(hcall(head_offsets=torch.tensor([0, 2, 5])), "head_offsets has shape")
    _raises(hcall(head_v=torch.zeros((T, H, d + 1))), "head_v has shape")
    _raises(hcall(head_beta=torch.zeros((T - 1, H))), "head_beta has shape")
    _raises(hcall(head_log_alpha=torch.zeros((T, H + 1))), "head_log_alpha has shape")
    _raises(hcall(out_S=torch.zeros((R, H, d, d + 2))), "out_S has shape")


def test_conv_shape_checks():
    C, K, rows = 16, 4, 5
    tails = torch.zeros((rows, K - 1, C), dtype=torch.bfloat16)
    heads = torch.zeros((rows, K - 1, C), dtype=torch.bfloat16)
    w = torch.zeros((C, K))
    ok = dict(tails=tails, heads=heads, weight=w)

    def call(**kw):
        return lambda: hp.conv_warmup(**dict(ok, **kw))

    _raises(call(), "on the GPU")
    _raises(call(bias=torch.zeros(C + 1)), "bias has shape")
    _raises(call(out=torch.zeros((rows, K - 1, C + 1))), "out has shape")
    _raises(call(heads=torch.zeros((rows, K, C), dtype=torch.bfloat16)), "K-1, C")
    _raises(call(num_boundaries=rows + 1), "covers")
    _raises(call(tail_index=torch.zeros(2, dtype=torch.int32), num_boundaries=3), "tail_index covers")
    # conv keys and values: C = H (d_k + d_v) channels
    H, dk, dv, T = 2, 4, 4, 3
    Cv = H * (dk + dv)
    kv = dict(x=torch.zeros((7, Cv), dtype=torch.bfloat16), window=torch.zeros((T, K), dtype=torch.int32),
              weight=torch.zeros((Cv, K)), num_heads=H, d_k=dk, d_v=dv)

    def kcall(**kw):
        return lambda: hp.conv_kv(**dict(kv, **kw))

    _raises(kcall(), "on the GPU")
    _raises(kcall(weight=torch.zeros((Cv + 1, K))), "H \\(d_k \\+ d_v\\) channels")
    _raises(kcall(window=torch.zeros((T, K + 1), dtype=torch.int32)), "window")
    _raises(kcall(bias=torch.zeros(Cv - 1)), "bias has shape")
    _raises(kcall(src_token=torch.zeros(T + 1, dtype=torch.int32)), "src_token")
    _raises(kcall(src_token=torch.zeros(T, dtype=torch.int32), beta=torch.zeros((5, H)),
                  log_alpha=torch.zeros((6, H))), "both be")
