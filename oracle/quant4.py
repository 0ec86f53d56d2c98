"""Oracle: a 4-bit KV cache with one static scale per (kv head, channel), and attention over it.

Test infrastructure only (see the package docstring).

Source: the DuoAttention README pairs retrieval/streaming heads with a 4-bit KV cache. Its
installation section downloads "w8a8kv4-per-channel" demo models, and its efficiency section fits
3.3 million tokens of Llama-3-8B on one A100-80G with 8-bit weights and a 4-bit KV cache. The pages
give no scheme beyond "4-bit" and "per-channel". This cache takes the plainest reading that fits an
append-only paged cache, and states it as its definition:

  * symmetric 4-bit codes in [-7, 7]; K and V each have one fp32 scale per (kv head, channel),
    fixed by the caller (calibrated offline), so a new row is quantized without looking at any
    other row;
  * code = round-half-to-even(x / s) with x / s one correctly rounded fp32 division, clamped to
    [-7, 7]; a channel whose scale is 0 stores code 0; the value of a code is code * s;
  * storage: a code c is the 4-bit number u = c + 8 (1..15). A run of 8 codes e0..e7 along a row is
    one little-endian 32-bit word: the low 16 bits hold u(e0), u(e2), u(e4), u(e6) and the high 16
    bits u(e1), u(e3), u(e5), u(e7), each 4 bits with the first in the lowest bits. A K row (the
    head_dim codes of one token) is head_dim / 8 words in channel order; a V row (the block_size
    codes of one channel in one page) is block_size / 8 words in slot order.

Every step is fp32 arithmetic that IEEE 754 fixes bit for bit, so codes are exactly reproducible;
numpy performs each float32 operation in float32.

Pins (tests/test_oracle_int4.py): hand-worked rows (ties to even, saturation, zero scale), a
hand-packed word, pack/unpack round trips, codes of values on a power-of-two grid come back exactly,
attention over a cache whose values sit on the grid equals attention over the values themselves,
and planted mistakes in the quantizer and the packing.
"""
from __future__ import annotations

import numpy as np

from .cache import to_f64, append as append_rows
from .attention import visible_positions, attend_row

F32, F16, BF16 = 0, 1, 2


def quantize_rows4(x: np.ndarray, scales: np.ndarray, dtype: int) -> np.ndarray:
    """Codes int8 [..., D] of stored elements x [..., D] with per-channel scales [D] (float32)."""
    xf = to_f64(x, dtype).astype(np.float32)
    s = np.asarray(scales, dtype=np.float32)
    pos = s > 0
    safe = np.where(pos, s, np.float32(1.0)).astype(np.float32)
    q = (xf / safe).astype(np.float32)                  # one correctly rounded fp32 division
    codes = np.clip(np.rint(q), -7, 7)
    return np.where(pos, codes, 0).astype(np.int8)


def dequantize4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code * scale per channel (last axis), float64 (exact)."""
    return codes.astype(np.float64) * np.asarray(scales, dtype=np.float32).astype(np.float64)


def pack4(codes: np.ndarray) -> np.ndarray:
    """Codes [..., n] (n a multiple of 8) -> storage bytes uint8 [..., n / 2] in the word layout of
    the module docstring."""
    c = np.asarray(codes, dtype=np.int64)
    n = c.shape[-1]
    assert n % 8 == 0
    u = (c + 8).reshape(c.shape[:-1] + (n // 8, 8)).astype(np.uint32)
    word = np.zeros(u.shape[:-1], dtype=np.uint32)
    for i in range(4):
        word |= u[..., 2 * i] << np.uint32(4 * i)
        word |= u[..., 2 * i + 1] << np.uint32(16 + 4 * i)
    return np.ascontiguousarray(word.astype("<u4")).view(np.uint8).reshape(c.shape[:-1] + (n // 2,))


def unpack4(data: np.ndarray) -> np.ndarray:
    """Storage bytes [..., n / 2] -> codes int8 [..., n] (u - 8 of every 4-bit field)."""
    b = np.ascontiguousarray(data, dtype=np.uint8)
    m = b.shape[-1]
    assert m % 4 == 0
    word = b.reshape(b.shape[:-1] + (m // 4, 4)).view("<u4")[..., 0].astype(np.uint32)
    out = np.empty(word.shape + (8,), dtype=np.int64)
    for i in range(4):
        out[..., 2 * i] = (word >> np.uint32(4 * i)) & 15
        out[..., 2 * i + 1] = (word >> np.uint32(16 + 4 * i)) & 15
    return (out - 8).reshape(b.shape[:-1] + (2 * m,)).astype(np.int8)


def pool4_shapes(num_blocks: int, block_size: int, head_dim: int):
    """Byte pools: K [NB][bs][D / 2] (token-major rows), V [NB][D][bs / 2] (channel-major rows)."""
    return (num_blocks, block_size, head_dim // 2), (num_blocks, head_dim, block_size // 2)


def append_int4(k_pool, v_pool, k_scale, v_scale, table, k_new, v_new, seq_lens_before,
                retrieval_mask, dtype, *, sink, block_size, ring_blocks, max_blocks_per_head):
    """Quantize the new tokens' K and V rows with the per-(kv head, channel) scales and write their
    codes into the byte pools, in place (k_pool [NB][bs][D/2], v_pool [NB][D][bs/2] uint8;
    k_scale, v_scale [Hkv][D] float32; k_new, v_new [B][t_new][Hkv][D] stored elements). The slots
    are those of the unquantized cache (oracle.cache.append places the codes); codes of slots this
    call does not write keep their bits. Returns the lengths after the call."""
    Hkv = k_new.shape[2]
    kc = np.stack([quantize_rows4(k_new[:, :, h], k_scale[h], dtype) for h in range(Hkv)], axis=2)
    vc = np.stack([quantize_rows4(v_new[:, :, h], v_scale[h], dtype) for h in range(Hkv)], axis=2)
    k_codes = unpack4(k_pool)          # [NB][bs][D]
    v_codes = unpack4(v_pool)          # [NB][D][bs]
    after = append_rows(k_codes, v_codes, table, kc, vc, seq_lens_before, retrieval_mask,
                        sink=sink, block_size=block_size, ring_blocks=ring_blocks,
                        max_blocks_per_head=max_blocks_per_head)
    k_pool[...] = pack4(k_codes)
    v_pool[...] = pack4(v_codes)
    return after


def attend_int4(q, k_codes, v_codes, k_scale, v_scale, seq_lens, retrieval_mask, *, sink, recent,
                scale, dtype, rows=None, block_size=None):
    """Reference output over a logical 4-bit cache, float64.

    q: [B][q_len][Hq][D] stored elements of dtype; k_codes, v_codes: [B][Hkv][>= max len][D] int8
    codes; k_scale, v_scale: [Hkv][D] float32. Visible sets, query positions and the softmax are
    those of oracle.attention.attend (block_size as there), over the dequantized rows code * scale.
    """
    B, q_len, Hq, D = q.shape
    Hkv = k_codes.shape[1]
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
            cache = {key: (dequantize4(k_codes[b, h], k_scale[h]),
                           dequantize4(v_codes[b, h], v_scale[h]))}
        Kf, Vf = cache[key]
        out[b, i, hq] = attend_row(to_f64(q[b, i, hq], dtype), Kf[J], Vf[J], scale)
    return out
