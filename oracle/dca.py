"""Oracle: Dual Chunk Attention over a full causal cache, in float64.

Test infrastructure only (see the package docstring).

Source: vLLM PR "[Model] Implement DualChunkAttention for Qwen2 Models".
  * Description ("Overview", "Changes"): the sequence is cut into chunks, and the rotary layer hands
    the attention three query vectors per token, for keys in the same chunk (intra), in the chunk just
    before (succ) and in any earlier chunk (inter).
  * Review thread, on the brute-force varlen prefill: the only change from ordinary causal attention
    is which query meets a key; the query's own for a key of its chunk, q_succ for a key of the
    preceding chunk, q_inter for a key of any chunk before that.
  * Review thread, on the intra-chunk length: chunks have the fixed length chunk_len except the last
    (the query's own), which may be shorter. Chunks are therefore counted from position 0:
    chunk(t) = t // chunk_len.
  * Review thread, on the numerical issue: the weight is (query . key) * softmax_scale * mscale, with
    mscale a float32 value per query position, applied in float32 rather than folded into q.
  * Review thread, on the softmax LSE typo: the three partial attentions are merged by their
    log-sum-exp, which is the same as one softmax over the union of the three key sets; that union is
    every position j <= p, so this oracle takes the single softmax directly.

Readings taken where the page is silent (each listed with the other readings of the pages):
  * mscale is one float32 per query row, the same for its three query vectors;
  * every head is a full causal head (the page does not combine DCA with streaming heads), bounded by
    the sequence's valid length; query row i sits at position seq_len - q_len + i, as in ``attend``;
  * local_size and the YaRN settings shape the rotary positions baked into q, q_succ and q_inter, so
    they are not arguments here (positions and RoPE are outside the attention call).
"""
from __future__ import annotations

import numpy as np

from .cache import to_f64


def query_kind(p: int, j, chunk_len: int):
    """Which query vector a query at position p uses against key position(s) j (int or int array):
    0 intra (same chunk), 1 succ (the key's chunk directly precedes the query's), 2 inter."""
    cq, ck = p // chunk_len, np.asarray(j) // chunk_len
    return np.where(ck == cq, 0, np.where(ck == cq - 1, 1, 2))


def attend_dca_row(qs, K: np.ndarray, V: np.ndarray, p: int, chunk_len: int, scale: float,
                   mscale: float) -> np.ndarray:
    """One query row at position p over keys 0..p (K, V hold at least p + 1 rows, float64).

    qs = (q, q_succ, q_inter), each float64 [D]. Returns float64 [D]; zeros if p < 0.
    """
    D = V.shape[1]
    if p < 0:
        return np.zeros(D, dtype=np.float64)
    kind = query_kind(p, np.arange(p + 1), chunk_len)
    Kp = K[:p + 1]
    s = np.where(kind == 0, Kp @ qs[0], np.where(kind == 1, Kp @ qs[1], Kp @ qs[2]))
    s = s * (scale * mscale)
    m = s.max()
    w = np.exp(s - m)
    return (w @ V[:p + 1]) / w.sum()


def attend_dca(q, q_succ, q_inter, k, v, seq_lens, mscale, *, chunk_len, scale, dtype, rows=None):
    """Reference output of Dual Chunk Attention, float64.

    q, q_succ, q_inter: [B][q_len][Hq][D] stored elements; k, v: logical caches [B][Hkv][>= len][D];
    seq_lens: [B] valid lengths including the query rows; mscale: float32 [B][q_len] (upcast exactly).
    rows: optional iterable of (b, i, hq). Returns [B][q_len][Hq][D] float64 (unselected rows NaN).
    A q head hq reads kv head hq // (Hq / Hkv), as in ``attend``.
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
        key = (b, h)
        if key not in cache:
            cache = {key: (to_f64(k[b, h], dtype), to_f64(v[b, h], dtype))}
        Kf, Vf = cache[key]
        qs = tuple(to_f64(x[b, i, hq], dtype) for x in (q, q_succ, q_inter))
        out[b, i, hq] = attend_dca_row(qs, Kf, Vf, p, chunk_len, scale,
                                       float(np.float32(mscale[b, i])))
    return out


def attend_dca_rows(qs, p_rows, K: np.ndarray, V: np.ndarray, chunk_len: int, scale: float,
                    mscale_rows) -> np.ndarray:
    """Several query rows of one (sequence, kv head) at once, float64: ``attend_dca_row`` for each
    row, with the scores of the three query sets taken as three matrix products over keys
    0..max(p) and each (row, key) score taken from the set ``query_kind`` names for it.

    qs = (q, q_succ, q_inter), each float64 [R][D]; p_rows [R] positions; K, V float64 [>= max p + 1]
    rows; mscale_rows [R] (float32 values). Rows at p < 0 give zeros. Returns [R][D].
    """
    p = np.asarray(p_rows, dtype=np.int64)
    R, D = len(p), V.shape[1]
    out = np.zeros((R, D), dtype=np.float64)
    live = p >= 0
    if not live.any():
        return out
    n = int(p.max()) + 1
    j = np.arange(n, dtype=np.int64)
    kind = query_kind(p[:, None], j[None, :], chunk_len)
    Kp = K[:n]
    s = np.where(kind == 0, qs[0] @ Kp.T, np.where(kind == 1, qs[1] @ Kp.T, qs[2] @ Kp.T))
    s = s * (scale * np.asarray(mscale_rows, dtype=np.float64))[:, None]
    ok = j[None, :] <= p[:, None]
    s = np.where(ok, s, -np.inf)
    m = np.where(live, s.max(axis=1), 0.0)
    w = np.where(ok, np.exp(s - m[:, None]), 0.0)
    den = w.sum(axis=1)
    res = (w @ V[:n]) / np.where(live, den, 1.0)[:, None]
    out[live] = res[live]
    return out
