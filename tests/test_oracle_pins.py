"""Pins for the CPU oracle: each check ties it to something other than itself.

* the worked slot tables printed on the vLLM issue "Could you support Attention Sink?" (golden file);
* a separately written dense brute force, swept over small shapes;
* torch's scaled_dot_product_attention on CPU in float64, with an explicit boolean mask, and its
  own is_causal mask for the retrieval-only prefill case (a textbook causal attention);
* closed forms: q = 0 gives the mean of the visible V rows (hand-derived visible sets below), a
  length-1 cache returns v0;
* invariants: a streaming head whose sink + recent covers the sequence equals a retrieval head;
  the circular paged layout gives the same outputs as the contiguous cache; cache slots beyond the
  valid length (NaN there) have no effect; repeating kv heads turns GQA into MHA without changing
  outputs.
* the row-block form (``attend_rows``, all rows of a head in one score matrix, optionally over a
  subset of the keys) against the same brute force and closed forms;
* planted mistakes: a few plausible bugs injected into a copy of the oracle must each fail a pin.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from oracle import cache as ocache
from tests.brute import brute_force

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ring_tables.txt")


def _run_oracle_f64(q, k, v, lens, ret, sink, recent, scale):
    """Run oracle.attend on float32-representable inputs (dtype tag F32)."""
    return oracle.attend(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), lens, ret,
                         sink=sink, recent=recent, scale=scale, dtype=0)


def _rand_case(rng, B, q_len, Hq, Hkv, D, Lmax):
    q = rng.standard_normal((B, q_len, Hq, D)).astype(np.float32).astype(np.float64)
    k = rng.standard_normal((B, Hkv, Lmax, D)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((B, Hkv, Lmax, D)).astype(np.float32).astype(np.float64)
    return q, k, v


# ------------------------------------------------------------------------------------------------
# Worked tables (vLLM issue "Could you support Attention Sink?")
# ------------------------------------------------------------------------------------------------
def _load_tables():
    tables, cur = {}, None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = line.strip("[]")
            tables[cur] = {"states": {}}
        elif line.startswith("sink"):
            tables[cur]["sink"] = int(line.split()[1])
        else:
            tok, body = line.split(":")
            blocks = [b.split() for b in body.split("|")]
            tables[cur]["states"][int(tok)] = [[None if x == "x" else int(x) for x in blk]
                                               for blk in blocks]
    return tables


def _simulate_inplace(sink, upto, nblocks=4, bs=4):
    """Buffer contents after appending tokens 0..upto with the page's in-place sink layout."""
    buf = [None] * (nblocks * bs)
    for t in range(upto + 1):
        s = ocache.slot_of(t, retrieval=False, sink=sink, sink_slots=sink,
                           ring_slots=nblocks * bs - sink)
        buf[s] = t
    return [buf[i * bs:(i + 1) * bs] for i in range(nblocks)]


def test_worked_ring_tables_match_page():
    tables = _load_tables()
    assert set(tables) == {"no_sink", "sink2"}
    for name, tab in tables.items():
        for tok, expect in tab["states"].items():
            assert _simulate_inplace(tab["sink"], tok) == expect, (name, tok)


def test_separate_sink_layout_uses_same_ring_index():
    # option 3 of the same page: sinks in their own page(s); the ring index (t - sink) mod ring is
    # unchanged, only the ring's first slot moves to the page boundary.
    bs, sink, rb = 4, 2, 3
    for t in range(40):
        col, row = ocache.table_position(t, retrieval=False, sink=sink, block_size=bs, ring_blocks=rb)
        if t < sink:
            assert (col, row) == (0, t)
        else:
            ring_index = (t - sink) % (rb * bs)
            assert col * bs + row == bs + ring_index
    # retrieval heads: identity
    for t in range(40):
        assert ocache.table_position(t, retrieval=True, sink=sink, block_size=bs,
                                     ring_blocks=rb) == (t // bs, t % bs)


def test_append_writes_worked_example_in_separate_sink_layout():
    # Hand-derived: sink 2, block 4, 3 ring pages (12 ring slots), 20 tokens appended one call.
    # Sinks 0,1 -> page col 0 rows 0,1. Token t >= 2 -> ring index (t-2) % 12 -> slot 4 + index.
    # Tokens 2..7 are overwritten by 14..19; the ring ends holding 8..19.
    bs, sink, rb, D = 4, 2, 3, 1
    table = np.array([[[3, 0, 2, 1]]], dtype=np.int32)     # physical pages of the one row
    kp, vp = ocache.new_pools(4, bs, D, np.float32, -1.0)
    toks = np.arange(20, dtype=np.float32).reshape(1, 20, 1, 1)
    ocache.append(kp, vp, table, toks, toks, np.array([0]), np.array([0], np.uint8), sink=sink,
                  block_size=bs, ring_blocks=rb, max_blocks_per_head=4)
    logical_rows = {0: [0, 1, -1, -1], 1: [14, 15, 16, 17], 2: [18, 19, 8, 9], 3: [10, 11, 12, 13]}
    for col, want in logical_rows.items():
        phys = table[0, 0, col]
        assert kp[phys, :, 0].tolist() == want
        assert vp[phys, 0, :].tolist() == want


# ------------------------------------------------------------------------------------------------
# Brute force and library cross-checks
# ------------------------------------------------------------------------------------------------
SWEEP = [
    # (L, q_len, sink, recent, Hq, Hkv, retrieval)
    (1, 1, 0, 1, 2, 1, (0,)),
    (7, 1, 1, 3, 2, 2, (1,)),
    (33, 1, 4, 16, 4, 2, (0,)),
    (50, 50, 4, 7, 4, 4, (0, 2)),
    (64, 17, 5, 16, 4, 1, ()),
    (96, 96, 0, 64, 2, 2, (1,)),
    (96, 3, 4, 1, 8, 2, (1,)),
    (80, 80, 16, 16, 2, 1, ()),
    (40, 12, 0, 5, 6, 3, (0, 2)),
]


@pytest.mark.parametrize("L,q_len,sink,recent,Hq,Hkv,ret", SWEEP)
def test_oracle_matches_brute_force(L, q_len, sink, recent, Hq, Hkv, ret):
    rng = np.random.default_rng(L * 1000 + q_len)
    B, D = 2, 8
    q, k, v = _rand_case(rng, B, q_len, Hq, Hkv, D, L + 5)
    lens = np.array([L, max(q_len, L - 2)])
    mask = np.zeros(Hkv, np.uint8)
    mask[list(ret)] = 1
    scale = 0.3
    got = _run_oracle_f64(q, k, v, lens, mask, sink, recent, scale)
    want = brute_force(q, k, v, lens, mask, sink, recent, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,q_len,sink,recent,Hq,Hkv,ret", SWEEP)
def test_oracle_matches_torch_sdpa_with_explicit_mask(L, q_len, sink, recent, Hq, Hkv, ret):
    rng = np.random.default_rng(7 + L)
    B, D = 1, 16
    q, k, v = _rand_case(rng, B, q_len, Hq, Hkv, D, L)
    lens = np.array([L])
    mask = np.zeros(Hkv, np.uint8)
    mask[list(ret)] = 1
    scale = 0.25
    got = _run_oracle_f64(q, k, v, lens, mask, sink, recent, scale)
    G = Hq // Hkv
    for hq in range(Hq):
        h = hq // G
        # mask built element by element from the visible-set rule as stated in words
        allowed = torch.zeros(q_len, L, dtype=torch.bool)
        for i in range(q_len):
            p = L - q_len + i
            for j in range(L):
                allowed[i, j] = j <= p and (bool(mask[h]) or j < sink or p - j < recent)
        out = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0, :, hq, :])[None], torch.from_numpy(k[0, h, :L])[None],
            torch.from_numpy(v[0, h, :L])[None], attn_mask=allowed[None], scale=scale)
        np.testing.assert_allclose(got[0, :, hq, :], out[0].numpy(), rtol=0, atol=1e-12)


def test_retrieval_prefill_equals_textbook_causal_sdpa():
    rng = np.random.default_rng(3)
    L, D, H = 70, 32, 2
    q, k, v = _rand_case(rng, 1, L, H, H, D, L)
    got = _run_oracle_f64(q, k, v, np.array([L]), np.ones(H, np.uint8), 0, 1, 1 / np.sqrt(D))
    for h in range(H):
        out = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0, :, h, :])[None], torch.from_numpy(k[0, h])[None],
            torch.from_numpy(v[0, h])[None], is_causal=True)
        np.testing.assert_allclose(got[0, :, h, :], out[0].numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# Closed forms
# ------------------------------------------------------------------------------------------------
# (L, q_len, sink, recent, retrieval, expected visible sets of the rows), derived by hand from the
# statement "sinks = the first sink positions, recent = the last recent positions up to and
# including the query, the union of the two, nothing past the query".
HAND = [
    (10, 1, 2, 3, False, [{0, 1, 7, 8, 9}]),
    (6, 1, 2, 3, False, [{0, 1, 3, 4, 5}]),          # window starts just above the sinks
    (5, 1, 2, 3, False, [{0, 1, 2, 3, 4}]),          # window meets the sinks
    (4, 1, 2, 3, False, [{0, 1, 2, 3}]),             # window overlaps the sinks
    (10, 1, 0, 3, False, [{7, 8, 9}]),
    (10, 1, 2, 1, False, [{0, 1, 9}]),
    (6, 1, 8, 2, False, [{0, 1, 2, 3, 4, 5}]),       # sink region longer than the sequence
    (10, 1, 2, 3, True, [set(range(10))]),
    (8, 3, 1, 2, False, [{0, 4, 5}, {0, 5, 6}, {0, 6, 7}]),
    (8, 3, 1, 2, True, [set(range(6)), set(range(7)), set(range(8))]),
]


@pytest.mark.parametrize("L,q_len,sink,recent,ret,sets", HAND)
def test_zero_query_averages_exactly_the_visible_rows(L, q_len, sink, recent, ret, sets):
    D = 16
    q = np.zeros((1, q_len, 1, D))
    k = np.random.default_rng(0).standard_normal((1, 1, L, D))
    v = np.zeros((1, 1, L, D))
    v[0, 0, np.arange(L), np.arange(L)] = 1.0                # one-hot V rows
    got = _run_oracle_f64(q, k, v, np.array([L]), np.array([1 if ret else 0], np.uint8), sink,
                          recent, 0.5)
    for i, s in enumerate(sets):
        want = np.zeros(D)
        want[sorted(s)] = 1.0 / len(s)
        np.testing.assert_allclose(got[0, i, 0], want, atol=1e-15)


def test_length_one_returns_v0():
    rng = np.random.default_rng(5)
    q, k, v = _rand_case(rng, 1, 1, 2, 2, 8, 1)
    got = _run_oracle_f64(q, k, v, np.array([1]), np.array([0, 1], np.uint8), 0, 1, 1.0)
    np.testing.assert_allclose(got[0, 0], v[0, :, 0, :], atol=1e-15)


def test_empty_visible_set_is_zero():
    # rows whose position would be negative (seq_len < q_len) see nothing
    q = np.ones((1, 3, 1, 4))
    k = np.ones((1, 1, 3, 4))
    v = np.ones((1, 1, 3, 4))
    got = _run_oracle_f64(q, k, v, np.array([1]), np.array([1], np.uint8), 0, 1, 1.0)
    assert (got[0, :2] == 0).all() and np.allclose(got[0, 2], 1.0)


# ------------------------------------------------------------------------------------------------
# Invariants
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("L,q_len,sink,recent", [(20, 1, 4, 16), (20, 20, 4, 16), (31, 5, 0, 31),
                                                 (12, 12, 12, 1), (40, 7, 30, 10)])
def test_streaming_with_window_covering_sequence_equals_full(L, q_len, sink, recent):
    assert sink + recent >= L
    rng = np.random.default_rng(L + sink)
    q, k, v = _rand_case(rng, 1, q_len, 2, 2, 8, L)
    a = _run_oracle_f64(q, k, v, np.array([L]), np.array([0, 0], np.uint8), sink, recent, 0.4)
    b = _run_oracle_f64(q, k, v, np.array([L]), np.array([1, 1], np.uint8), sink, recent, 0.4)
    np.testing.assert_allclose(a, b, atol=1e-13)


def _paged_roundtrip(rng, *, B, Hq, Hkv, D, bs, sink, recent, ring_blocks, ret, calls, q_len):
    """Append tokens over several calls into a shuffled, NaN-filled pool; return both outputs."""
    total = sum(calls)
    mbph = max(-(-total // bs), -(-sink // bs) + ring_blocks)
    need = [mbph if h in ret else -(-sink // bs) + ring_blocks for h in range(Hkv)]
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
    mask = np.zeros(Hkv, np.uint8)
    mask[list(ret)] = 1
    lens = np.zeros(B, np.int64)
    for n in calls:
        kn = np.ascontiguousarray(k[:, :, lens[0]:lens[0] + n].transpose(0, 2, 1, 3))
        vn = np.ascontiguousarray(v[:, :, lens[0]:lens[0] + n].transpose(0, 2, 1, 3))
        lens = ocache.append(kp, vp, table, kn, vn, lens, mask, sink=sink, block_size=bs,
                             ring_blocks=ring_blocks, max_blocks_per_head=mbph)
    q = rng.standard_normal((B, q_len, Hq, D)).astype(np.float32)
    paged = oracle.attend_paged(q, kp, vp, table, lens, mask, sink=sink, recent=recent, scale=0.3,
                                dtype=0, block_size=bs, ring_blocks=ring_blocks)
    contiguous = oracle.attend(q, k, v, lens, mask, sink=sink, recent=recent, scale=0.3, dtype=0)
    return paged, contiguous


@pytest.mark.parametrize("calls,ring_blocks,q_len,bs", [
    ([37], 3, 1, 4),          # one call longer than the ring (slot collisions inside one call)
    ([5, 9, 1, 1, 30], 3, 1, 4),
    ([64], 8, 16, 4),          # prefill-sized query block, ring >= recent + q_len - 1
    ([3, 3, 3, 3, 3, 3, 3], 2, 1, 8),
    ([100], 5, 20, 16),
])
def test_circular_paged_layout_equals_contiguous(calls, ring_blocks, q_len, bs):
    rng = np.random.default_rng(sum(calls) + ring_blocks)
    recent = min(ring_blocks * bs - q_len + 1, 11)
    paged, contiguous = _paged_roundtrip(rng, B=2, Hq=4, Hkv=2, D=8, bs=bs, sink=3, recent=recent,
                                         ring_blocks=ring_blocks, ret=(1,), calls=calls, q_len=q_len)
    assert np.isfinite(paged).all()
    np.testing.assert_allclose(paged, contiguous, atol=1e-12)


def test_shared_sink_pages_equal_private_ones_when_the_sinks_match():
    """Option 3 of the vLLM attention-sink issue keeps the sinks in blocks of their own and suggests
    reusing that block for every request that starts with the same sink tokens. Streaming heads of
    all sequences share sink pages here; with identical first sink tokens the paged result equals the
    contiguous attention, and the shared pages hold those tokens."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, D, bs, sink, ring_blocks, recent = 3, 4, 2, 8, 4, 6, 3, 9
    total = 40
    sb = -(-sink // bs)
    mbph = max(-(-total // bs), sb + ring_blocks)
    ret = (1,)
    k = rng.standard_normal((B, Hkv, total, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, total, D)).astype(np.float32)
    k[:, :, :sink] = k[0:1, :, :sink]                 # every sequence starts with the same sinks
    v[:, :, :sink] = v[0:1, :, :sink]
    table = np.zeros((B, Hkv, mbph), np.int32)
    nxt = 0
    for h in range(Hkv):
        if h in ret:
            continue
        table[:, h, :sb] = np.arange(nxt, nxt + sb)   # one set of sink pages per streaming kv head
        nxt += sb
    for b in range(B):
        for h in range(Hkv):
            lo, n = (0, mbph) if h in ret else (sb, ring_blocks)
            table[b, h, lo:lo + n] = np.arange(nxt, nxt + n)
            nxt += n
    kp, vp = ocache.new_pools(nxt, bs, D, np.float32, np.nan)
    mask = np.zeros(Hkv, np.uint8)
    mask[list(ret)] = 1
    lens = np.zeros(B, np.int64)
    for n in (5, 17, 1, 17):
        kn = np.ascontiguousarray(k[:, :, lens[0]:lens[0] + n].transpose(0, 2, 1, 3))
        vn = np.ascontiguousarray(v[:, :, lens[0]:lens[0] + n].transpose(0, 2, 1, 3))
        lens = ocache.append(kp, vp, table, kn, vn, lens, mask, sink=sink, block_size=bs,
                             ring_blocks=ring_blocks, max_blocks_per_head=mbph)
    q = rng.standard_normal((B, 2, Hq, D)).astype(np.float32)
    paged = oracle.attend_paged(q, kp, vp, table, lens, mask, sink=sink, recent=recent, scale=0.3,
                                dtype=0, block_size=bs, ring_blocks=ring_blocks)
    contiguous = oracle.attend(q, k, v, lens, mask, sink=sink, recent=recent, scale=0.3, dtype=0)
    np.testing.assert_allclose(paged, contiguous, atol=1e-12)
    # the shared pages hold the sink tokens, one copy for all sequences
    for t in range(sink):
        assert np.array_equal(kp[table[0, 0, t // bs], t % bs], k[0, 0, t])
    assert nxt == sb + B * (mbph + ring_blocks)      # private sinks would take B * sb


def test_slots_beyond_valid_length_have_no_effect():
    rng = np.random.default_rng(11)
    L, Lcap = 29, 64
    q, k, v = _rand_case(rng, 1, 3, 4, 2, 8, Lcap)
    mask = np.array([1, 0], np.uint8)
    a = _run_oracle_f64(q, k[:, :, :L], v[:, :, :L], np.array([L]), mask, 2, 5, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, L:] = np.nan
    v2[:, :, L:] = np.inf
    b = _run_oracle_f64(q, k2, v2, np.array([L]), mask, 2, 5, 0.5)
    assert np.array_equal(a, b)


def test_repeating_kv_heads_turns_gqa_into_mha():
    rng = np.random.default_rng(12)
    L, G = 40, 3
    q, k, v = _rand_case(rng, 2, 4, 6, 2, 8, L)
    mask = np.array([0, 1], np.uint8)
    lens = np.array([L, 33])
    gqa = _run_oracle_f64(q, k, v, lens, mask, 3, 9, 0.2)
    mha = _run_oracle_f64(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), lens,
                          np.repeat(mask, G), 3, 9, 0.2)
    np.testing.assert_allclose(gqa, mha, atol=0)


def test_dtype_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x7F80, 0x0001, 0x4049], np.uint16)
    got = ocache.to_f64(bits, 2)
    assert got[0] == 1.0 and got[1] == -1.0 and np.isinf(got[2])
    assert got[3] == 2.0 ** -133 and got[4] == 3.140625
    h = np.array([1.5, -0.25, 65504.0], np.float16).view(np.uint16)
    assert ocache.to_f64(h, 1).tolist() == [1.5, -0.25, 65504.0]


# ------------------------------------------------------------------------------------------------
# Row blocks (oracle.attend_rows): several rows of one head in one score matrix
# ------------------------------------------------------------------------------------------------
def _rows_by_blocks(q, k, v, lens, mask, sink, recent, scale, subset=False):
    """oracle.attend_rows over every (sequence, q head): all rows of a head at once. With subset,
    streaming heads get only the keys some row can see (the sinks and the union of the windows)."""
    B, q_len, Hq, D = q.shape
    G = Hq // k.shape[1]
    out = np.zeros(q.shape)
    for b in range(B):
        L = int(lens[b])
        p = L - q_len + np.arange(q_len)
        for hq in range(Hq):
            h = hq // G
            ret = bool(mask[h])
            keys = np.arange(L)
            if subset and not ret:
                keys = np.union1d(np.arange(min(sink, L)),
                                  np.arange(max(0, p[0] - recent + 1), L))
            out[b, :, hq] = oracle.attend_rows(q[b, :, hq], p, k[b, h, keys], v[b, h, keys], keys,
                                               retrieval=ret, sink=sink, recent=recent,
                                               scale=scale)
    return out


@pytest.mark.parametrize("L,q_len,sink,recent,Hq,Hkv,ret", SWEEP)
@pytest.mark.parametrize("subset", [False, True])
def test_row_blocks_match_brute_force(L, q_len, sink, recent, Hq, Hkv, ret, subset):
    rng = np.random.default_rng(L * 1000 + q_len + 17)
    B, D = 2, 8
    q, k, v = _rand_case(rng, B, q_len, Hq, Hkv, D, L + 5)
    lens = np.array([L, max(q_len, L - 2)])
    mask = np.zeros(Hkv, np.uint8)
    mask[list(ret)] = 1
    got = _rows_by_blocks(q, k, v, lens, mask, sink, recent, 0.3, subset)
    want = brute_force(q, k, v, lens, mask, sink, recent, 0.3)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,q_len,sink,recent,ret,sets", HAND)
def test_row_blocks_zero_query_average_exactly_the_visible_rows(L, q_len, sink, recent, ret, sets):
    D = 16
    v = np.zeros((L, D))
    v[np.arange(L), np.arange(L)] = 1.0
    k = np.random.default_rng(1).standard_normal((L, D))
    got = oracle.attend_rows(np.zeros((q_len, D)), L - q_len + np.arange(q_len), k, v,
                             np.arange(L), retrieval=ret, sink=sink, recent=recent, scale=0.5)
    for i, s in enumerate(sets):
        want = np.zeros(D)
        want[sorted(s)] = 1.0 / len(s)
        np.testing.assert_allclose(got[i], want, atol=1e-15)


def test_row_blocks_rows_before_the_start_are_zero():
    got = oracle.attend_rows(np.ones((3, 4)), np.array([-2, -1, 0]), np.ones((1, 4)),
                             np.full((1, 4), 2.0), np.array([0]), retrieval=True, sink=0, recent=1,
                             scale=1.0)
    assert (got[:2] == 0).all() and np.allclose(got[2], 2.0)


# ------------------------------------------------------------------------------------------------
# Planted mistakes: each must be caught by one of the pins above
# ------------------------------------------------------------------------------------------------
def _window_off_by_one(p, *, retrieval, sink, recent, block_size=None):
    j = np.arange(max(p, -1) + 1)
    return j if retrieval else j[(j < sink) | (p - j <= recent)]


def _sink_dropped(p, *, retrieval, sink, recent, block_size=None):
    j = np.arange(max(p, -1) + 1)
    return j if retrieval else j[p - j < recent]


def _future_leak(p, *, retrieval, sink, recent, block_size=None):
    j = np.arange(max(p, -1) + 2)
    return j if retrieval else j[(j < sink) | (p - j < recent)]


def _scale_inside_exp_missing(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    s = K @ q
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def _v_transposed_rows(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w[::-1] @ V) / w.sum()


@pytest.mark.parametrize("bug", [_window_off_by_one, _sink_dropped, _future_leak])
def test_planted_visible_set_bugs_are_caught(monkeypatch, bug):
    monkeypatch.setattr(oatt, "visible_positions", bug)
    caught = False
    for case in SWEEP:
        try:
            test_oracle_matches_brute_force(*case)
        except AssertionError:
            caught = True
            break
    assert caught


@pytest.mark.parametrize("bug", [_scale_inside_exp_missing, _v_transposed_rows])
def test_planted_softmax_bugs_are_caught(monkeypatch, bug):
    monkeypatch.setattr(oatt, "attend_row", bug)
    with pytest.raises(AssertionError):
        test_oracle_matches_brute_force(*SWEEP[3])


def _mask_window_off_by_one(p_rows, key_pos, *, retrieval, sink, recent, block_size=None):
    p, j = np.asarray(p_rows)[:, None], np.asarray(key_pos)[None, :]
    ok = (j >= 0) & (j <= p)
    return ok if retrieval else ok & ((j < sink) | (p - j <= recent))


def _mask_sink_dropped(p_rows, key_pos, *, retrieval, sink, recent, block_size=None):
    p, j = np.asarray(p_rows)[:, None], np.asarray(key_pos)[None, :]
    ok = (j >= 0) & (j <= p)
    return ok if retrieval else ok & (p - j < recent)


def _mask_future_leak(p_rows, key_pos, *, retrieval, sink, recent, block_size=None):
    p, j = np.asarray(p_rows)[:, None], np.asarray(key_pos)[None, :]
    ok = (j >= 0) & (j <= p + 1)
    return ok if retrieval else ok & ((j < sink) | (p - j < recent))


@pytest.mark.parametrize("bug", [_mask_window_off_by_one, _mask_sink_dropped, _mask_future_leak])
def test_planted_row_block_mask_bugs_are_caught(monkeypatch, bug):
    monkeypatch.setattr(oatt, "visible_mask", bug)
    caught = False
    for case in SWEEP:
        try:
            test_row_blocks_match_brute_force(*case, False)
        except AssertionError:
            caught = True
            break
    assert caught


def test_planted_ring_index_bug_is_caught(monkeypatch):
    def bad_slot(t, *, retrieval, sink, sink_slots, ring_slots):
        if retrieval or t < sink:
            return t
        return sink_slots + (t - sink + 1) % ring_slots
    monkeypatch.setattr(ocache, "slot_of", bad_slot)
    with pytest.raises(AssertionError):
        test_worked_ring_tables_match_page()
