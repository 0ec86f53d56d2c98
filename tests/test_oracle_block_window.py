"""Pins for the oracle's block-granular streaming window (recent < 0).

The rule comes from the vLLM issue "Could you support Attention Sink?", ChuanhongLi's comment: a
streaming head keeps the first block of the sequence as its attention sink, drops blocks in the
middle and keeps the recent blocks, with the number of blocks per sequence capped. Pinned here by:

* a simulation of that allocation policy, token by token (a list of held blocks; a new block is
  taken when a token starts one, and past the cap the oldest block after the sink blocks is
  dropped), compared with the oracle's visible set after every token;
* hand-derived visible sets, read back through a zero query and one-hot V rows (the output is the
  mean of exactly the visible rows);
* containment between token windows: k blocks hold at least (k - 1) * block_size + 1 and at most
  k * block_size of the newest positions;
* the circular paged layout: reading the window out of a ring of pages equals reading it out of
  the contiguous cache whenever the ring holds k blocks plus the chunk;
* planted mistakes, each caught by one of the above.
"""
import numpy as np
import pytest

import oracle
from oracle import attention as oatt
from oracle import cache as ocache


def _held_after(p, *, block_size, sink_blocks, keep):
    """Positions held after tokens 0..p were appended under the block policy."""
    held = []
    for t in range(p + 1):
        n = t // block_size
        if n not in held:
            held.append(n)
            if len(held) > sink_blocks + keep:
                # the oldest block that is not a sink block leaves
                held.remove(min(x for x in held if x >= sink_blocks))
    return [t for t in range(p + 1) if t // block_size in held]


SIM = [(4, 1, 1), (4, 1, 2), (4, 1, 3), (16, 1, 2), (8, 2, 2), (4, 0, 2), (1, 1, 3), (16, 1, 5)]


@pytest.mark.parametrize("bs,sink_blocks,keep", SIM)
def test_block_window_equals_the_eviction_policy(bs, sink_blocks, keep):
    for p in range(0, 12 * bs):
        want = _held_after(p, block_size=bs, sink_blocks=sink_blocks, keep=keep)
        got = oatt.visible_positions(p, retrieval=False, sink=sink_blocks * bs, recent=-keep,
                                     block_size=bs)
        assert got.tolist() == want, (p, got.tolist(), want)


# (L, q_len, sink, blocks, block_size, visible set of each query row)
HAND = [
    (14, 1, 4, 2, 4, [{0, 1, 2, 3, 8, 9, 10, 11, 12, 13}]),   # query in block 3: blocks 2, 3 kept
    (13, 1, 4, 2, 4, [{0, 1, 2, 3, 8, 9, 10, 11, 12}]),        # first position of block 3
    (12, 1, 4, 2, 4, [set(range(12))]),                        # blocks 1, 2 kept: no gap yet
    (14, 1, 0, 1, 4, [{12, 13}]),                              # no sink, only the newest block
    (13, 1, 0, 1, 4, [{12}]),
    (18, 1, 2, 2, 4, [{0, 1, 12, 13, 14, 15, 16, 17}]),        # sink inside the first block
    (17, 3, 4, 1, 4, [{0, 1, 2, 3, 12, 13, 14}, {0, 1, 2, 3, 12, 13, 14, 15}, {0, 1, 2, 3, 16}]),
]


@pytest.mark.parametrize("L,q_len,sink,blocks,bs,sets", HAND)
def test_zero_query_averages_exactly_the_block_window(L, q_len, sink, blocks, bs, sets):
    D = 24
    q = np.zeros((1, q_len, 1, D), np.float32)
    k = np.random.default_rng(L).standard_normal((1, 1, L, D)).astype(np.float32)
    v = np.zeros((1, 1, L, D), np.float32)
    v[0, 0, np.arange(L), np.arange(L)] = 1.0
    got = oracle.attend(q, k, v, np.array([L]), np.array([0], np.uint8), sink=sink, recent=-blocks,
                        scale=0.5, dtype=0, block_size=bs)
    for i, s in enumerate(sets):
        want = np.zeros(D)
        want[sorted(s)] = 1.0 / len(s)
        np.testing.assert_allclose(got[0, i, 0], want, atol=1e-15)


@pytest.mark.parametrize("bs,blocks,sink", [(4, 1, 0), (4, 3, 4), (16, 2, 5), (8, 4, 0), (1, 6, 2)])
def test_block_window_lies_between_two_token_windows(bs, blocks, sink):
    for p in range(0, 10 * bs):
        blk = set(oatt.visible_positions(p, retrieval=False, sink=sink, recent=-blocks,
                                         block_size=bs).tolist())
        small = set(oatt.visible_positions(p, retrieval=False, sink=sink,
                                           recent=(blocks - 1) * bs + 1).tolist())
        large = set(oatt.visible_positions(p, retrieval=False, sink=sink,
                                           recent=blocks * bs).tolist())
        assert small <= blk <= large
        # the window ends at the query and starts on a block boundary (or at the sink / position 0)
        win = sorted(t for t in blk if t >= sink)
        if win:
            assert win[-1] == p and win == list(range(win[0], p + 1))
            assert win[0] % bs == 0 or win[0] == sink


def test_block_window_needs_the_block_size():
    with pytest.raises(ValueError):
        oatt.visible_positions(9, retrieval=False, sink=4, recent=-2)


def test_retrieval_heads_ignore_the_block_window():
    got = oatt.visible_positions(21, retrieval=True, sink=4, recent=-1, block_size=4)
    assert got.tolist() == list(range(22))


@pytest.mark.parametrize("calls,ring_blocks,q_len,bs,blocks", [
    ([37], 3, 1, 4, 3),        # the ring holds exactly the window
    ([5, 9, 1, 1, 30], 4, 1, 4, 2),
    ([64], 6, 16, 4, 2),       # a 16-row chunk: 2 blocks + 15 rows fit 6 pages
    ([100], 5, 20, 16, 3),
])
def test_block_window_reads_the_same_out_of_the_ring(calls, ring_blocks, q_len, bs, blocks):
    assert ring_blocks * bs >= blocks * bs + q_len - 1
    rng = np.random.default_rng(sum(calls) + 7 * ring_blocks)
    B, Hq, Hkv, D, sink = 2, 4, 2, 8, 3
    total = sum(calls)
    sb = -(-sink // bs)
    mbph = max(-(-total // bs), sb + ring_blocks)
    need = [sb + ring_blocks, mbph]                     # head 0 streaming, head 1 retrieval
    nblocks = B * sum(need)
    perm = rng.permutation(nblocks)
    table = np.zeros((B, Hkv, mbph), np.int32)
    pos = 0
    for b in range(B):
        for h in range(Hkv):
            table[b, h, :need[h]] = perm[pos:pos + need[h]]
            pos += need[h]
    kp, vp = ocache.new_pools(nblocks, bs, D, np.float32, np.nan)
    k = rng.standard_normal((B, Hkv, total, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, total, D)).astype(np.float32)
    mask = np.array([0, 1], np.uint8)
    lens = np.zeros(B, np.int64)
    for n in calls:
        kn = np.ascontiguousarray(k[:, :, lens[0]:lens[0] + n].transpose(0, 2, 1, 3))
        vn = np.ascontiguousarray(v[:, :, lens[0]:lens[0] + n].transpose(0, 2, 1, 3))
        lens = ocache.append(kp, vp, table, kn, vn, lens, mask, sink=sink, block_size=bs,
                             ring_blocks=ring_blocks, max_blocks_per_head=mbph)
    q = rng.standard_normal((B, q_len, Hq, D)).astype(np.float32)
    paged = oracle.attend_paged(q, kp, vp, table, lens, mask, sink=sink, recent=-blocks, scale=0.3,
                                dtype=0, block_size=bs, ring_blocks=ring_blocks)
    contiguous = oracle.attend(q, k, v, lens, mask, sink=sink, recent=-blocks, scale=0.3, dtype=0,
                               block_size=bs)
    assert np.isfinite(paged).all()
    np.testing.assert_allclose(paged, contiguous, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# Planted mistakes
# ------------------------------------------------------------------------------------------------
def _one_block_too_many(p, j, recent, block_size=None):
    p, j = np.asarray(p), np.asarray(j)
    if recent >= 0:
        return p - j < recent
    return j // block_size >= p // block_size + recent


def _window_by_tokens(p, j, recent, block_size=None):
    p, j = np.asarray(p), np.asarray(j)
    if recent >= 0:
        return p - j < recent
    return p - j < -recent * block_size


def _blocks_of_the_wrong_origin(p, j, recent, block_size=None):
    p, j = np.asarray(p), np.asarray(j)
    if recent >= 0:
        return p - j < recent
    return (j + 1) // block_size > (p + 1) // block_size + recent


@pytest.mark.parametrize("bug", [_one_block_too_many, _window_by_tokens, _blocks_of_the_wrong_origin])
def test_planted_block_window_bugs_are_caught(monkeypatch, bug):
    monkeypatch.setattr(oatt, "in_window", bug)
    caught = False
    for case in SIM:
        try:
            test_block_window_equals_the_eviction_policy(*case)
        except AssertionError:
            caught = True
            break
    assert caught
