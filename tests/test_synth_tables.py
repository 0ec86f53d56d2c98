"""Host-side checks of the seeded block tables the GPU tests and bench.py build (no GPU).

Every (sequence, kv head) row must own its pages; with shared sinks, the streaming heads' sink
columns of every sequence point at one set of pages and nothing else is shared. A page used by two
rows that should not share it would let one row's append overwrite another's keys.
"""
import collections

import numpy as np
import pytest

import synth


def _used_columns(w, h):
    return synth.pages_needed(w, h)


@pytest.mark.parametrize("share", [False, True])
@pytest.mark.parametrize("sink,bs", [(4, 16), (20, 16), (70, 64), (0, 16)])
def test_pages_are_private_except_shared_sinks(share, sink, bs):
    w = synth.small("tables", batch=3, q_heads=8, kv_heads=4, head_dim=64, dtype=synth.BF16,
                    block_size=bs, sink=sink, recent=40, retrieval=(0, 2), context=300, q_len=16,
                    seed=5)
    table, n = synth.block_table(w, share_sinks=share)
    assert table.shape == (w.batch, w.num_kv_heads, w.max_blocks_per_head)
    owners = collections.defaultdict(set)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            for col in range(_used_columns(w, h)):
                page = int(table[b, h, col])
                assert 0 <= page < n
                owners[page].add((b, h, col))
    assert len(owners) == n                      # every page of the pool is used
    sb = w.sink_blocks
    for page, users in owners.items():
        if len(users) == 1:
            continue
        # only a streaming head's sink column, the same column in every sequence, may be shared
        assert share
        heads = {h for _, h, _ in users}
        cols = {c for _, _, c in users}
        assert len(heads) == 1 and len(cols) == 1
        (h,), (col,) = heads, cols
        assert h not in w.retrieval and col < sb
        assert {b for b, _, _ in users} == set(range(w.batch))
    streaming = [h for h in range(w.num_kv_heads) if h not in w.retrieval]
    saved = (w.batch - 1) * len(streaming) * sb
    private = synth.block_table(w, share_sinks=False)[1]
    assert n == (private - saved if share else private)


def test_identity_table_is_the_contiguous_static_cache():
    w = synth.gemma_2b_static_decode(batch=3, capacity=256)
    table, n = synth.block_table(w, identity=True)
    assert n == 3 * 16
    np.testing.assert_array_equal(table[:, 0, :], np.arange(48).reshape(3, 16))
