"""Dense brute-force masked softmax attention, written independently of the oracle.

Builds the whole [q_len x L] score matrix, writes -inf where the mask forbids, and takes a row
softmax. Used only to pin the oracle on tiny inputs.
"""
import numpy as np


def mask_matrix(L, q_len, retrieval, sink, recent):
    """allowed[i, j]: query row i (at position L - q_len + i) may look at key j (< L)."""
    rowpos = (L - q_len) + np.arange(q_len)[:, None]
    col = np.arange(L)[None, :]
    allowed = col <= rowpos
    if not retrieval:
        allowed = allowed & ((col < sink) | (col > rowpos - recent))
    return allowed


def brute_force(q, k, v, seq_lens, retrieval_mask, sink, recent, scale):
    """q [B][q_len][Hq][D]; k, v [B][Hkv][Lmax][D]; all float64."""
    B, q_len, Hq, D = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, q_len, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        for hq in range(Hq):
            h = hq * Hkv // Hq
            S = scale * (q[b, :, hq, :] @ k[b, h, :L].T)
            allowed = mask_matrix(L, q_len, bool(retrieval_mask[h]), sink, recent)
            S = np.where(allowed, S, -np.inf)
            top = S.max(axis=1, keepdims=True)
            top = np.where(np.isfinite(top), top, 0.0)
            E = np.exp(S - top)
            den = E.sum(axis=1, keepdims=True)
            O = E @ v[b, h, :L]
            out[b, :, hq, :] = np.where(den > 0, O / np.where(den > 0, den, 1.0), 0.0)
    return out


def brute_force_dca(q, q_succ, q_inter, k, v, seq_lens, mscale, chunk_len, scale):
    """Dual Chunk Attention as three separate masked attentions merged by their log-sum-exp.

    The split mirrors the brute-force form the DualChunkAttention PR describes (one attention per
    chunk relation, then a merge of the partial results through their LSE). All inputs float64;
    q* [B][q_len][Hq][D], k/v [B][Hkv][Lmax][D], mscale [B][q_len].
    """
    B, q_len, Hq, D = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, q_len, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        rowpos = (L - q_len) + np.arange(q_len)[:, None]
        col = np.arange(L)[None, :]
        causal = col <= rowpos
        qc = np.floor_divide(rowpos, chunk_len)
        kc = np.floor_divide(col, chunk_len)
        masks = [causal & (kc == qc), causal & (kc + 1 == qc), causal & (kc + 1 < qc)]
        for hq in range(Hq):
            h = hq * Hkv // Hq
            parts = []
            for qq, allowed in zip((q, q_succ, q_inter), masks):
                S = scale * mscale[b][:, None] * (qq[b, :, hq, :] @ k[b, h, :L].T)
                S = np.where(allowed, S, -np.inf)
                top = S.max(axis=1, keepdims=True)
                top = np.where(np.isfinite(top), top, 0.0)
                E = np.exp(S - top)
                den = E.sum(axis=1, keepdims=True)
                with np.errstate(divide="ignore"):
                    lse = np.where(den > 0, np.log(np.where(den > 0, den, 1.0)) + top, -np.inf)
                O = (E @ v[b, h, :L]) / np.where(den > 0, den, 1.0)
                parts.append((lse, O))
            big = np.maximum.reduce([lse for lse, _ in parts])
            big = np.where(np.isfinite(big), big, 0.0)
            wts = [np.exp(lse - big) for lse, _ in parts]
            tot = sum(wts)
            acc = sum(w * O for w, (_, O) in zip(wts, parts))
            out[b, :, hq, :] = np.where(tot > 0, acc / np.where(tot > 0, tot, 1.0), 0.0)
    return out
