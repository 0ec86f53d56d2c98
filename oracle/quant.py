"""Oracle: an int8 KV cache (one scale per token row of each kv head) and attention over it.

Test infrastructure only (see the package docstring).

Source: the DuoAttention README, installation-and-usage section (its QServe install step and its
demo), pairs retrieval/streaming heads with a 4-bit quantized KV cache (QServe), which is how its
demo fits a multi-million-token context on one GPU. The pages fix neither the bit width, nor the
grouping of scales, nor the rounding. This cache takes the plainest reading and states it as its
definition:

  * symmetric 8-bit codes in [-127, 127] with one fp32 scale per stored row: per (sequence, kv head,
    position) for K and, separately, for V, taken over that row's head_dim values;
  * amax = max |x| over the row (exact in fp32, since x is fp32, fp16 or bf16);
    inv = 127 / amax and scale = amax / 127, each one correctly rounded fp32 division;
    code = round-half-to-even(x * inv) with x * inv one correctly rounded fp32 product, clamped to
    [-127, 127]; an all-zero row gets codes 0 and scale 0;
  * the row's value is code * scale (dequantized exactly in float64 here).

Every step is fp32 arithmetic that IEEE 754 fixes bit for bit, so the codes and scales are exactly
reproducible; numpy performs each float32 operation in float32.

Pins (tests/test_oracle_quant.py): hand-worked rows, codes of values on a power-of-two grid come back
exactly, the largest magnitude always maps to +-127, the reconstruction error is at most half a step
(plus fp32 rounding), sign symmetry, zero rows; attention over a cache whose values sit on the grid
equals attention over the unquantized values.
"""
from __future__ import annotations

import numpy as np

from .cache import to_f64, append as append_rows
from .attention import visible_positions, attend_row

F32, F16, BF16 = 0, 1, 2


def to_f32(a: np.ndarray, dtype: int) -> np.ndarray:
    """Stored elements (bf16/f16 as uint16 bit patterns, or float32) as exact float32 values."""
    return to_f64(a, dtype).astype(np.float32)


def quantize_rows(x: np.ndarray, dtype: int):
    """Quantize the last axis of stored elements x [..., D]: (codes int8 [..., D], scales float32
    [...]) by the definition in the module docstring."""
    xf = to_f32(x, dtype)
    amax = np.max(np.abs(xf), axis=-1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(127.0) / safe).astype(np.float32)
    prod = (xf * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(prod), -127, 127)
    codes = np.where(nz[..., None], codes, 0).astype(np.int8)
    scales = np.where(nz, (amax / np.float32(127.0)).astype(np.float32), np.float32(0.0))
    return codes, scales.astype(np.float32)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code * scale per row, float64 (exact: an int8 times an fp32 fits a float64)."""
    return codes.astype(np.float64) * scales.astype(np.float64)[..., None]


def scale_pool_shape(num_blocks: int, block_size: int):
    """Scales sit beside the pages, one per slot: [num_blocks][block_size] float32."""
    return (num_blocks, block_size)


def append_int8(k_pool, v_pool, k_scale, v_scale, table, k_new, v_new, seq_lens_before,
                retrieval_mask, dtype, *, sink, block_size, ring_blocks, max_blocks_per_head):
    """Quantize the new tokens' K and V rows and write codes and scales to their slots.

    k_pool [NB][bs][D] int8 (token-major), v_pool [NB][D][bs] int8 (channel-major), k_scale and
    v_scale [NB][bs] float32; k_new, v_new [B][t_new][Hkv][D] stored elements of dtype. The slots
    are those of the unquantized cache (oracle.cache.append, which this reuses for the placement):
    the scale of slot s sits at [page][s % bs], so the scale pools are written as K-like pools of
    head_dim 1.
    """
    kc, ks = quantize_rows(k_new, dtype)
    vc, vs = quantize_rows(v_new, dtype)
    kw = dict(sink=sink, block_size=block_size, ring_blocks=ring_blocks,
              max_blocks_per_head=max_blocks_per_head)
    after = append_rows(k_pool, v_pool, table, kc, vc, seq_lens_before, retrieval_mask, **kw)
    ks_pool = k_scale.reshape(k_scale.shape[0], k_scale.shape[1], 1)
    vs_pool = v_scale.reshape(v_scale.shape[0], v_scale.shape[1], 1)
    # K-scale pool as a token-major K pool of head_dim 1; V-scale pool likewise (the same slot map)
    dummy_v = np.zeros((k_scale.shape[0], 1, k_scale.shape[1]), dtype=np.float32)
    append_rows(ks_pool, dummy_v, table, ks[..., None], ks[..., None], seq_lens_before,
                retrieval_mask, **kw)
    append_rows(vs_pool, dummy_v, table, vs[..., None], vs[..., None], seq_lens_before,
                retrieval_mask, **kw)
    return after


def attend_int8(q, k_codes, k_scales, v_codes, v_scales, seq_lens, retrieval_mask, *, sink, recent,
                scale, dtype, rows=None, block_size=None):
    """Reference output over a logical int8 cache, float64.

    q: [B][q_len][Hq][D] stored elements of dtype; k_codes, v_codes: [B][Hkv][>= max len][D] int8;
    k_scales, v_scales: [B][Hkv][>= max len] float32 (position j of head h of sequence b at
    [b, h, j]). Visible sets, query positions and the softmax are those of oracle.attention.attend
    (block_size as there), over the dequantized rows code * scale.
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
            cache = {key: (dequantize(k_codes[b, h], k_scales[b, h]),
                           dequantize(v_codes[b, h], v_scales[b, h]))}
        Kf, Vf = cache[key]
        out[b, i, hq] = attend_row(to_f64(q[b, i, hq], dtype), Kf[J], Vf[J], scale)
    return out
