"""Oracle: where a token of a (sequence, kv head) lives in the paged cache, and the append.

Test infrastructure only (see the package docstring).

Layout (the library documents the same layout in its header; this file implements it on its own):
  * each (sequence b, kv head h) owns one row of the block table, ``table[b][h][:]``;
  * a page holds ``block_size`` consecutive slots; the K page is token-major ``[block_size][D]``,
    the V page is channel-major ``[D][block_size]``;
  * slot s of the row lives in page ``table[b][h][s // block_size]`` at row ``s % block_size``.

Slot of logical position t (vLLM issue "Could you support Attention Sink?", sh1ng's comment: the
circular-buffer tables and option 3):
  * a retrieval head keeps every token: slot = t (DuoAttention README, abstract: full KV cache for
    retrieval heads);
  * a streaming head keeps sink tokens where they were written (slot = t for t < sink) and cycles the
    other tokens through a ring of ``ring_slots`` slots that starts at slot ``sink_slots``:
    slot = sink_slots + (t - sink) mod ring_slots.
    The page's second table keeps the sinks in place inside a 16-slot buffer; that is
    sink_slots = sink and ring_slots = 16 - sink. Option 3 (the layout of this cache) gives the sinks
    pages of their own: sink_slots = ceil(sink / block_size) * block_size and
    ring_slots = ring_blocks * block_size.
"""
from __future__ import annotations

import numpy as np

F32, F16, BF16 = 0, 1, 2


def to_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    """Exact conversion of stored elements to float64 (bf16/f16 arrive as uint16 bit patterns)."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == F16:
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == BF16:
        wide = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def slot_of(t: int, *, retrieval: bool, sink: int, sink_slots: int, ring_slots: int) -> int:
    """Slot of logical position t in its head's row (see the module docstring)."""
    if retrieval or t < sink:
        return t
    return sink_slots + (t - sink) % ring_slots


def ring_capacity(block_size: int, ring_blocks: int) -> int:
    return block_size * ring_blocks


def table_position(t: int, *, retrieval: bool, sink: int, block_size: int, ring_blocks: int):
    """(table column, row in page) of position t in this cache's layout (option 3)."""
    sink_slots = -(-sink // block_size) * block_size
    s = slot_of(t, retrieval=retrieval, sink=sink, sink_slots=sink_slots,
                ring_slots=ring_capacity(block_size, ring_blocks))
    return s // block_size, s % block_size


def pool_shapes(num_blocks: int, block_size: int, head_dim: int):
    """(K pool shape, V pool shape): K pages token-major, V pages channel-major."""
    return (num_blocks, block_size, head_dim), (num_blocks, head_dim, block_size)


def new_pools(num_blocks, block_size, head_dim, np_dtype, fill):
    ks, vs = pool_shapes(num_blocks, block_size, head_dim)
    return np.full(ks, fill, dtype=np_dtype), np.full(vs, fill, dtype=np_dtype)


def append(k_pool, v_pool, table, k_new, v_new, seq_lens_before, retrieval_mask, *, sink,
           block_size, ring_blocks, max_blocks_per_head):
    """Write new tokens into the pools in token order; returns the lengths after the call.

    k_new, v_new: [batch][t_new][kv_heads][D] stored elements; seq_lens_before: [batch].
    Token i of sequence b sits at position seq_lens_before[b] + i (transformers PR "[WIP] Dynamic
    length in static cache": the cache is updated at the new positions, then attended).
    Tokens are written in increasing position, so when two tokens of one call land in the same ring
    slot the later one is what remains (the vLLM issue's tables: a new token overwrites the oldest
    streamed token). A retrieval head has room for max_blocks_per_head * block_size positions;
    positions beyond that are not stored (the library documents the same).

    Plain loop over (sequence, head) and over runs of at most ring-capacity tokens: inside one run
    the destination slots are distinct, so each numpy assignment writes each slot once, and the runs
    are applied oldest first.
    """
    B, T, H, D = k_new.shape
    cap = max_blocks_per_head * block_size
    ring = ring_capacity(block_size, ring_blocks)
    for b in range(B):
        L0 = int(seq_lens_before[b])
        for h in range(H):
            ret = bool(retrieval_mask[h])
            step = T if ret else max(1, ring)
            for r0 in range(0, T, step):
                r1 = min(T, r0 + step)
                pos = np.arange(L0 + r0, L0 + r1)
                keep = pos < cap if ret else np.ones(pos.shape, dtype=bool)
                if not keep.any():
                    continue
                cols, rows = zip(*(table_position(int(t), retrieval=ret, sink=sink,
                                                  block_size=block_size, ring_blocks=ring_blocks)
                                   for t in pos[keep]))
                phys = table[b, h, np.asarray(cols)]
                rows = np.asarray(rows)
                src = np.arange(r0, r1)[keep]
                k_pool[phys, rows, :] = k_new[b, src, h, :]
                v_pool[phys, :, rows] = v_new[b, src, h, :]
    return np.asarray(seq_lens_before, dtype=np.int64) + T


def gather(k_pool, v_pool, table, b, h, positions, *, retrieval, sink, block_size, ring_blocks):
    """Read the stored K and V rows of the given logical positions of (sequence b, kv head h).

    Returns ([n][D], [n][D]) stored elements. Only positions still resident may be asked for (a
    streaming head keeps its sinks and the last ring-capacity positions).
    """
    positions = np.asarray(positions, dtype=np.int64)
    D = k_pool.shape[2]
    if positions.size == 0:
        return k_pool[:0, 0, :], np.empty((0, D), dtype=v_pool.dtype)
    cr = [table_position(int(t), retrieval=retrieval, sink=sink, block_size=block_size,
                         ring_blocks=ring_blocks) for t in positions]
    cols = np.asarray([c for c, _ in cr])
    rows = np.asarray([r for _, r in cr])
    phys = table[b, h, cols]
    return k_pool[phys, rows, :], v_pool[phys, :, rows]
