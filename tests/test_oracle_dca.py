"""Pins for the Dual Chunk Attention oracle (oracle/dca.py), on the CPU.

* a separately written brute force in the PR's own form: three masked attentions (intra, succ,
  inter) merged by their log-sum-exp (tests/brute.py), swept over small shapes and chunk lengths;
* a library reduction: with q = q_succ = q_inter the method is plain causal attention with the
  softmax scale times mscale, which torch's CPU float64 scaled_dot_product_attention computes;
* a closed form that counts the keys each query vector meets: with every key equal to one unit
  vector, each query a multiple of it and one-hot V rows, the output is the weight vector itself,
  exp(score of the key's kind) / Z, where the counts come from the PR's statement that every chunk
  but the query's own is chunk_len long;
* invariants: a chunk covering the whole sequence leaves only the intra query (q_succ and q_inter
  have no effect, and the result is the ordinary attention of ``oracle.attend``); slots past the
  valid length have no effect;
* the row-block form (``attend_dca_rows``: the rows of one head against all keys in three matrix
  products) against the same brute force;
* planted mistakes in the oracle (wrong chunk of the succ query, succ and inter swapped, chunks
  counted from the query backwards, mscale dropped) must each fail a pin.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import dca as odca
from tests.brute import brute_force_dca

F32 = 0   # oracle dtype tag of float32 inputs


def _case(rng, B, q_len, Hq, Hkv, D, Lmax):
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return (f(B, q_len, Hq, D), f(B, q_len, Hq, D), f(B, q_len, Hq, D), f(B, Hkv, Lmax, D),
            f(B, Hkv, Lmax, D))


def _run(q, qs, qi, k, v, lens, ms, C, scale, rows=None):
    return odca.attend_dca(q, qs, qi, k, v, lens, ms, chunk_len=C, scale=scale, dtype=F32, rows=rows)


@pytest.mark.parametrize("B,q_len,Hq,Hkv,D,lens,C", [
    (1, 24, 2, 2, 8, [24], 8),        # whole sequence as queries, three chunks
    (2, 5, 4, 2, 16, [37, 21], 8),    # decode-like rows at the end, ragged last chunk
    (1, 40, 2, 1, 8, [40], 16),       # chunk boundary inside the rows, GQA
    (1, 7, 2, 2, 8, [50], 7),         # chunk length not a power of two
    (2, 3, 2, 2, 8, [3, 9], 64),      # one chunk only
    (1, 33, 1, 1, 4, [33], 1),        # one key per chunk
])
def test_matches_three_attentions_merged_by_lse(B, q_len, Hq, Hkv, D, lens, C):
    rng = np.random.default_rng(11 + C)
    q, qs, qi, k, v = _case(rng, B, q_len, Hq, Hkv, D, max(lens))
    ms = rng.uniform(0.5, 1.5, (B, q_len)).astype(np.float32)
    lens = np.array(lens)
    scale = 1 / np.sqrt(D)
    got = _run(q, qs, qi, k, v, lens, ms, C, scale)
    f = lambda a: a.astype(np.float64)
    want = brute_force_dca(f(q), f(qs), f(qi), f(k), f(v), lens, f(ms), C, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def _rows_form(q, qs, qi, k, v, lens, ms, C, scale):
    """attend_dca_rows over every (sequence, q head): all rows of a head at once."""
    B, q_len, Hq, D = q.shape
    G = Hq // k.shape[1]
    out = np.zeros(q.shape)
    f = lambda a: a.astype(np.float64)
    for b in range(B):
        p = int(lens[b]) - q_len + np.arange(q_len)
        for hq in range(Hq):
            h = hq // G
            out[b, :, hq] = odca.attend_dca_rows((f(q[b, :, hq]), f(qs[b, :, hq]), f(qi[b, :, hq])),
                                                 p, f(k[b, h]), f(v[b, h]), C, scale, ms[b])
    return out


@pytest.mark.parametrize("B,q_len,Hq,Hkv,D,lens,C", [
    (1, 24, 2, 2, 8, [24], 8),
    (2, 5, 4, 2, 16, [37, 21], 8),
    (1, 40, 2, 1, 8, [40], 16),
    (1, 7, 2, 2, 8, [50], 7),
    (2, 3, 2, 2, 8, [3, 9], 64),
    (1, 33, 1, 1, 4, [33], 1),
    (1, 6, 2, 2, 8, [4], 4),          # two rows before the sequence start
])
def test_row_blocks_match_three_attentions_merged_by_lse(B, q_len, Hq, Hkv, D, lens, C):
    rng = np.random.default_rng(23 + C)
    q, qs, qi, k, v = _case(rng, B, q_len, Hq, Hkv, D, max(lens))
    ms = rng.uniform(0.5, 1.5, (B, q_len)).astype(np.float32)
    lens = np.array(lens)
    scale = 1 / np.sqrt(D)
    got = _rows_form(q, qs, qi, k, v, lens, ms, C, scale)
    f = lambda a: a.astype(np.float64)
    want = brute_force_dca(f(q), f(qs), f(qi), f(k), f(v), lens, f(ms), C, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_equal_queries_reduce_to_causal_sdpa():
    rng = np.random.default_rng(3)
    B, L, H, D, C = 1, 48, 3, 16, 8
    q, _, _, k, v = _case(rng, B, L, H, H, D, L)
    ms = np.full((B, L), 1.25, dtype=np.float32)
    scale = 0.3
    got = _run(q, q, q, k, v, np.array([L]), ms, C, scale)
    tq = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)   # [B][H][L][D]
    tk = torch.from_numpy(k.astype(np.float64))
    tv = torch.from_numpy(v.astype(np.float64))
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                            scale=scale * 1.25)
    np.testing.assert_allclose(got, want.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


def _kind_counts(p, C):
    """Keys of each kind seen from position p, from the PR's statement on chunk lengths: the query's
    own chunk holds p mod C + 1 keys up to p, the chunk before it exactly C, the rest C each."""
    cq = p // C
    n_intra = p % C + 1
    n_succ = C if cq >= 1 else 0
    n_inter = (cq - 1) * C if cq >= 2 else 0
    return n_intra, n_succ, n_inter


@pytest.mark.parametrize("C", [1, 3, 8, 13, 64])
def test_closed_form_weights_count_each_kind(C):
    L, D = 40, 64                      # D >= L: one-hot V rows return the weights
    a, b, c = 1.5, -0.5, 0.75          # the three queries as multiples of the keys' unit vector
    e = np.zeros(D, dtype=np.float32)
    e[5] = 1.0
    q = np.broadcast_to(a * e, (1, L, 1, D)).astype(np.float32)
    qs = np.broadcast_to(b * e, (1, L, 1, D)).astype(np.float32)
    qi = np.broadcast_to(c * e, (1, L, 1, D)).astype(np.float32)
    k = np.broadcast_to(e, (1, 1, L, D)).astype(np.float32)
    v = np.eye(L, D, dtype=np.float32)[None, None]
    ms = np.full((1, L), 2.0, dtype=np.float32)
    scale = 0.5
    got = _run(q, qs, qi, k, v, np.array([L]), ms, C, scale)[0, :, 0, :L]
    for p in range(L):
        n0, n1, n2 = _kind_counts(p, C)
        assert n0 + n1 + n2 == p + 1
        w = [np.exp(scale * 2.0 * x) for x in (a, b, c)]
        Z = n0 * w[0] + n1 * w[1] + n2 * w[2]
        want = np.zeros(L)
        own = (p // C) * C
        want[own:p + 1] = w[0] / Z
        if n1:
            want[own - C:own] = w[1] / Z
        if n2:
            want[:own - C] = w[2] / Z
        np.testing.assert_allclose(got[p], want, rtol=0, atol=1e-14)


def test_one_chunk_is_ordinary_attention_and_ignores_other_queries():
    rng = np.random.default_rng(5)
    B, q_len, H, D, L = 2, 9, 2, 8, 30
    q, qs, qi, k, v = _case(rng, B, q_len, H, H, D, L)
    ms = np.full((B, q_len), 0.75, dtype=np.float32)
    lens = np.array([30, 17])
    got = _run(q, qs, qi, k, v, lens, ms, 32, 0.4)
    other = _run(q, qi * 3, qs - 1, k, v, lens, ms, 32, 0.4)
    np.testing.assert_array_equal(got, other)
    want = oracle.attend(q, k, v, lens, np.ones(H, dtype=np.uint8), sink=0, recent=1,
                         scale=0.4 * 0.75, dtype=F32)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_slots_past_the_valid_length_have_no_effect():
    rng = np.random.default_rng(9)
    q, qs, qi, k, v = _case(rng, 1, 6, 2, 2, 8, 64)
    lens = np.array([29])
    ms = np.ones((1, 6), dtype=np.float32)
    a = _run(q, qs, qi, k, v, lens, ms, 8, 0.35)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 29:] = np.nan
    v2[:, :, 29:] = np.inf
    b = _run(q, qs, qi, k2, v2, lens, ms, 8, 0.35)
    np.testing.assert_array_equal(a, b)


def _planted(monkeypatch, kind_fn=None, drop_mscale=False):
    if kind_fn is not None:
        monkeypatch.setattr(odca, "query_kind", kind_fn)
    if drop_mscale:
        orig = odca.attend_dca_row
        monkeypatch.setattr(odca, "attend_dca_row",
                            lambda qs, K, V, p, C, scale, ms: orig(qs, K, V, p, C, scale, 1.0))


def _kind_succ_two_back(p, j, C):
    cq, ck = p // C, np.asarray(j) // C
    return np.where(ck == cq, 0, np.where(ck == cq - 2, 1, 2))


def _kind_swapped(p, j, C):
    cq, ck = p // C, np.asarray(j) // C
    return np.where(ck == cq, 0, np.where(ck == cq - 1, 2, 1))


def _kind_from_query(p, j, C):
    d = (p - np.asarray(j)) // C
    return np.where(d == 0, 0, np.where(d == 1, 1, 2))


@pytest.mark.parametrize("mistake", ["succ_two_back", "swapped", "from_query", "no_mscale"])
def test_planted_mistakes_fail_a_pin(monkeypatch, mistake):
    fns = {"succ_two_back": _kind_succ_two_back, "swapped": _kind_swapped,
           "from_query": _kind_from_query}
    _planted(monkeypatch, kind_fn=fns.get(mistake), drop_mscale=mistake == "no_mscale")
    caught = 0
    with pytest.raises(AssertionError):
        test_closed_form_weights_count_each_kind(8)
    caught += 1
    with pytest.raises(AssertionError):
        test_matches_three_attentions_merged_by_lse(2, 5, 4, 2, 16, [37, 21], 8)
    caught += 1
    assert caught == 2


@pytest.mark.parametrize("mistake", ["succ_two_back", "swapped", "from_query"])
def test_planted_kind_mistakes_fail_the_row_block_pin(monkeypatch, mistake):
    fns = {"succ_two_back": _kind_succ_two_back, "swapped": _kind_swapped,
           "from_query": _kind_from_query}
    monkeypatch.setattr(odca, "query_kind", fns[mistake])
    with pytest.raises(AssertionError):
        test_row_blocks_match_three_attentions_merged_by_lse(2, 5, 4, 2, 16, [37, 21], 8)
