"""Host-side planning of a RAG-shaped step (no GPU): the index tables and orders that
hybrid_prefill_amd.rag.plan_step hands to the library.

Pages: besthub article "Cut First-Token Latency by 3.25x ...", paragraph 6 (cold
segments longest-processing-time first) and paragraph 4 (compose cached records;
conv warm-up at every segment boundary)."""
import numpy as np

from hybrid_prefill_amd import rag


def _plan(chains, cold):
    return rag.plan_step([np.asarray(c, dtype=np.int32) for c in chains], cold, device="cpu")


def test_cold_segments_longest_first_and_packed():
    cold = {7: 300, 2: 1024, 9: 128, 4: 1024, 5: 0}
    st = _plan([[7, 2], [9, 4, 5]], cold)
    lengths = np.diff(st.cold_offsets.numpy())
    assert list(lengths) == sorted(cold.values(), reverse=True)
    # each packed segment is the slot it is built into, with that slot's length
    for s, n in zip(st.cold_slots.numpy(), lengths):
        assert cold[int(s)] == n
    assert sorted(st.cold_slots.numpy().tolist()) == sorted(cold)
    assert st.n_cold_tokens == sum(cold.values())


def test_chains_longest_first_in_prompt_order():
    chains = [[1, 2], [3, 4, 5, 6], [7], [8, 9, 10]]
    st = _plan(chains, {})
    offs, flat = st.chain_offsets.numpy(), st.chain_slots.numpy()
    assert list(st.request_order) == [1, 3, 0, 2]
    for row, r in enumerate(st.request_order):
        assert flat[offs[row]:offs[row + 1]].tolist() == chains[r]    # prompt order kept
    assert st.n_compositions == sum(len(c) for c in chains)


def test_boundaries_are_every_adjacent_pair():
    chains = [[1, 2, 3], [4], [5, 6]]
    st = _plan(chains, {})
    pairs = list(zip(st.tail_index.numpy().tolist(), st.head_index.numpy().tolist()))
    assert pairs == [(1, 2), (2, 3), (5, 6)]
    assert list(st.boundary_request) == [0, 0, 2]


def test_empty_step():
    st = _plan([], {})
    assert st.n_cold_tokens == 0 and st.n_compositions == 0
    assert st.cold_offsets.numpy().tolist() == [0] and st.chain_offsets.numpy().tolist() == [0]
    assert st.tail_index.numel() == 0 and st.head_index.numel() == 0
