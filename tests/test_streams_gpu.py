"""Two independent build + compose pipelines on two streams at once give, bit for bit,
what each gives alone.

The library keeps no global mutable state and every call is asynchronous on the
caller's stream, so concurrent calls on different streams (default priority) may
interleave their kernels on the device in any order without changing any output.
The same kernels run either way, so the bar is bit-exact.
"""
import numpy as np
import pytest
import torch

import hybrid_prefill_amd as hp
import synth
from parity_util import say

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hp.lib()
    yield
    torch.cuda.synchronize()


def _pipeline(H, lens, seed):
    st = synth.gdn_stream(lens, H, D, D, torch.bfloat16, seed, 0.1, "cuda")
    offs = torch.as_tensor(st.seg_offsets).cuda()
    nseg = len(lens)
    slots = torch.as_tensor(np.random.default_rng(seed).permutation(nseg).astype(np.int32)).cuda()
    chain = torch.tensor([0, nseg], dtype=torch.int64, device="cuda")
    pool = hp.Pool.allocate(hp.GDN, nseg, H, D, D, device="cuda", fill=0.0)
    out_S = torch.zeros((1, H, D, D), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run():
        hp.build_segment(hp.GDN, st.k, st.v, st.log_alpha, offs, pool, slots, beta=st.beta, err_flag=err)
        hp.compose_chain(pool, chain, slots, out_S=out_S, err_flag=err)

    def outputs():
        return [t.clone() for t in (pool.log_scale, pool.P, pool.S, out_S)]

    return run, outputs, (pool, out_S, err)


def test_two_streams_match_one_at_a_time():
    a_run, a_out, a_bufs = _pipeline(32, [2048, 700, 1500, 64], 901)
    b_run, b_out, b_bufs = _pipeline(4, [300, 2049, 1, 129, 5000], 902)
    a_run(); b_run()
    torch.cuda.synchronize()
    ref_a, ref_b = a_out(), b_out()
    for bufs in (a_bufs, b_bufs):
        for t in bufs[:2]:
            for x in ((t.log_scale, t.P, t.S) if isinstance(t, hp.Pool) else (t,)):
                x.fill_(12345.0)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            a_run()
        with torch.cuda.stream(s2):
            b_run()
    torch.cuda.current_stream().wait_stream(s1)
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    assert int(a_bufs[2].item()) == 0 and int(b_bufs[2].item()) == 0
    for got, want in zip(a_out() + b_out(), ref_a + ref_b):
        assert torch.equal(got, want)
    say("[streams] two pipelines on two streams, 3 rounds: bit-exact with one at a time")
