"""Oracle: mixed-head attention restricted to each head's visible positions, in float64.

Test infrastructure only (see the package docstring).

What a query at position p of sequence b, q head hq sees (h = hq // (q_heads / kv_heads) is its kv
head; a contiguous group of q heads shares one kv head, the usual grouped-query convention, which the
pages do not spell out -- parity unpinned by the pages for this mapping, pinned here only by the
"repeat kv heads" invariant):
  * every head: only positions j <= p of its own sequence (transformers PR "[WIP] Dynamic length in
    static cache", description: attend to the positions up to the current one, not the whole cache);
  * a retrieval head: all of them (DuoAttention README, abstract);
  * a streaming head: the attention sinks j < sink and the recent window p - j < recent, each
    position once (DuoAttention README, abstract and quick-start's sink_size / recent_size; vLLM issue
    "Could you support Attention Sink?", the sink tokens kept beside the streamed ones). The window
    counts the query's own position.
    A negative ``recent`` asks for the block-granular window instead (same vLLM issue, ChuanhongLi's
    comment: keep the sequence's first block as the sink, drop blocks in the middle and keep the
    recent blocks, with the number of blocks per sequence capped): positions are grouped into blocks
    of ``block_size`` (block n holds n*block_size .. (n+1)*block_size - 1), and the window is the
    -recent newest blocks up to the query's own, that block counting as one however few of its
    positions exist yet. The sink rule j < sink is unchanged.
Query row i of a call with q_len rows sits at position seq_len - q_len + i: the new tokens are in the
cache when they are attended (transformers PR, cache update then attention).

Scores are scale * (q . k) with the scale applied to the dot product (vLLM DualChunkAttention PR,
review thread on applying the softmax scale in fp32 rather than folding it into q). The output is
softmax-weighted V; an empty visible set (only possible for a row with p < 0) gives 0.
"""
from __future__ import annotations

import numpy as np

from .cache import to_f64, gather


def in_window(p, j, recent: int, block_size=None):
    """Is key position j inside the recent window of a query at position p (elementwise)?

    recent >= 0: the recent newest positions, p - j < recent. recent < 0: the -recent newest blocks of
    block_size positions, counted back from the block holding p: block(j) > block(p) + recent.
    """
    p = np.asarray(p, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    if recent >= 0:
        return p - j < recent
    if not block_size or block_size < 1:
        raise ValueError("a block-granular window (recent < 0) needs the block size")
    return j // block_size > p // block_size + recent


def visible_positions(p: int, *, retrieval: bool, sink: int, recent: int,
                      block_size=None) -> np.ndarray:
    """Sorted logical positions a query at position p may attend to."""
    if p < 0:
        return np.zeros(0, dtype=np.int64)
    j = np.arange(p + 1, dtype=np.int64)
    if retrieval:
        return j
    return j[(j < sink) | in_window(p, j, recent, block_size)]


def attend_row(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query over the given rows (all float64). Empty rows -> zeros."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1] if V.ndim == 2 else q.shape[0], dtype=np.float64)
    s = scale * (K @ q)
    m = s.max()
    w = np.exp(s - m)
    return (w @ V) / w.sum()


def visible_mask(p_rows, key_pos, *, retrieval: bool, sink: int, recent: int,
                 block_size=None) -> np.ndarray:
    """Boolean [R][N]: may a query at position p_rows[r] attend the key at position key_pos[n]?

    The rule of ``visible_positions``, applied to every (query, key) pair at once: the key is at or
    before the query, and for a streaming head it is a sink (j < sink) or in the recent window
    (``in_window``).
    """
    p = np.asarray(p_rows, dtype=np.int64)[:, None]
    j = np.asarray(key_pos, dtype=np.int64)[None, :]
    ok = (j >= 0) & (j <= p)
    if not retrieval:
        ok = ok & ((j < sink) | in_window(p, j, recent, block_size))
    return ok


def attend_rows(q_rows, p_rows, K, V, key_pos, *, retrieval: bool, sink: int, recent: int,
                scale: float, block_size=None) -> np.ndarray:
    """Several query rows of one (sequence, kv head) at once, float64: the same softmax attention
    as ``attend_row`` over ``visible_positions``, with the scores of all rows taken in one matrix
    product and the invisible ones set to -inf.

    q_rows [R][D] and p_rows [R] (positions); K, V [N][D] float64 rows held at the distinct key
    positions key_pos [N], which must include every key any of the rows can see (keys no row sees
    may be left out). Rows with nothing visible give zeros. Returns [R][D].
    """
    ok = visible_mask(p_rows, key_pos, retrieval=retrieval, sink=sink, recent=recent,
                      block_size=block_size)
    s = np.where(ok, scale * (np.asarray(q_rows, dtype=np.float64) @ K.T), -np.inf)
    seen = ok.any(axis=1)
    m = np.where(seen, s.max(axis=1), 0.0)
    w = np.where(ok, np.exp(s - m[:, None]), 0.0)
    den = w.sum(axis=1)
    out = (w @ V) / np.where(seen, den, 1.0)[:, None]
    out[~seen] = 0.0
    return out


def attend(q, k, v, seq_lens, retrieval_mask, *, sink, recent, scale, dtype, rows=None,
           block_size=None):
    """Reference output for every (or the selected) query rows, float64.

    q: [B][q_len][Hq][D] stored elements; k, v: logical caches [B][Hkv][>= max len][D] stored
    elements (position j of head h of sequence b at k[b, h, j]); seq_lens: [B] valid lengths
    including the query rows. rows: optional iterable of (b, i, hq); by default every row.
    block_size: the block length of a block-granular window (recent < 0).
    Returns out [B][q_len][Hq][D] float64 (unselected rows stay NaN).
    """
    B, q_len, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.full((B, q_len, Hq, D), np.nan, dtype=np.float64)
    if rows is None:
        rows = [(b, i, hq) for b in range(B) for i in range(q_len) for hq in range(Hq)]
    cache = {}
    for b, i, hq in rows:
        h = hq // G
        p = int(seq_lens[b]) - q_len + i
        J = visible_positions(p, retrieval=bool(retrieval_mask[h]), sink=sink, recent=recent,
                              block_size=block_size)
        key = (b, h)
        if key not in cache:
            cache = {key: (to_f64(k[b, h], dtype), to_f64(v[b, h], dtype))}
        Kf, Vf = cache[key]
        out[b, i, hq] = attend_row(to_f64(q[b, i, hq], dtype), Kf[J], Vf[J], scale)
    return out


def attend_paged(q, k_pool, v_pool, table, seq_lens, retrieval_mask, *, sink, recent, scale,
                 dtype, block_size, ring_blocks, rows=None):
    """Same as ``attend`` but reads K and V out of the paged pools through the oracle's own layout."""
    B, q_len, Hq, D = q.shape
    Hkv = table.shape[1]
    G = Hq // Hkv
    out = np.full((B, q_len, Hq, D), np.nan, dtype=np.float64)
    if rows is None:
        rows = [(b, i, hq) for b in range(B) for i in range(q_len) for hq in range(Hq)]
    for b, i, hq in rows:
        h = hq // G
        ret = bool(retrieval_mask[h])
        p = int(seq_lens[b]) - q_len + i
        J = visible_positions(p, retrieval=ret, sink=sink, recent=recent, block_size=block_size)
        Ks, Vs = gather(k_pool, v_pool, table, b, h, J, retrieval=ret, sink=sink,
                        block_size=block_size, ring_blocks=ring_blocks)
        out[b, i, hq] = attend_row(to_f64(q[b, i, hq], dtype), to_f64(Ks, dtype),
                                   to_f64(Vs, dtype), scale)
    return out
