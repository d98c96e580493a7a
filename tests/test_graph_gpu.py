"""The main step (GDN build of every segment, then the chain's compose) replayed from a
HIP graph gives the eager result bit for bit, replay after replay.

The step is captured once with torch.cuda.graph over the library's launches; between
replays the outputs are refilled with a canary and other eager work runs on the same
stream, so a replay that read stale state or skipped a launch would show.  The same
kernels run either way, so the bar is bit-exact.
"""
import numpy as np
import pytest
import torch

import hybrid_prefill_amd as hp
import synth
from parity_util import say

pytestmark = pytest.mark.gpu
CANARY = 12345.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hp.lib()
    yield
    torch.cuda.synchronize()


def _step(st, offs, pool, slots, chain, out_S, err):
    hp.build_segment(hp.GDN, st.k, st.v, st.log_alpha, offs, pool, slots, beta=st.beta, err_flag=err)
    hp.compose_chain(pool, chain, slots, out_S=out_S, err_flag=err)


@pytest.mark.parametrize("H,lens", [(4, [300, 64, 129, 2048]), (32, [2048] * 4)])
def test_step_graph_replays_match_eager(H, lens):
    D = 128
    st = synth.gdn_stream(lens, H, D, D, torch.bfloat16, 811, 0.1, "cuda")
    offs = torch.as_tensor(st.seg_offsets).cuda()
    nseg = len(lens)
    slots = torch.as_tensor(np.random.default_rng(3).permutation(nseg).astype(np.int32)).cuda()
    chain = torch.tensor([0, nseg], dtype=torch.int64, device="cuda")
    pool = hp.Pool.allocate(hp.GDN, nseg, H, D, D, device="cuda", fill=CANARY)
    out_S = torch.full((1, H, D, D), CANARY, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    _step(st, offs, pool, slots, chain, out_S, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = [t.clone() for t in (pool.log_scale, pool.P, pool.S, out_S)]

    # capture (the side-stream warm-up torch asks for, then the graph)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(st, offs, pool, slots, chain, out_S, err)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(st, offs, pool, slots, chain, out_S, err)
    torch.cuda.synchronize()

    other = hp.Pool.allocate(hp.GDN, nseg, H, D, D, device="cuda")
    for rep in range(3):
        for t in (pool.log_scale, pool.P, pool.S, out_S):
            t.fill_(CANARY)
        # eager work of the program's own between replays
        hp.build_segment(hp.GDN, st.k, st.v, st.log_alpha, offs, other, slots, beta=st.beta, err_flag=err)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        for got, want, name in zip((pool.log_scale, pool.P, pool.S, out_S), ref, ("log_scale", "P", "S", "out_S")):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"
        assert torch.equal(other.S, ref[2])
    say(f"[graph] H={H} lens={lens}: 3 replays bit-exact with the eager step")
    del g
