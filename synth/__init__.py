"""Seeded synthetic inputs for the mixed-head KV-cache attention workloads.

This module is shared by the CPU oracle's tests, the GPU parity tests and the benchmark. It draws
random numbers, rounds them to the storage dtype, lays out block tables, and describes the shapes of
the workloads. It contains no step of the attention method and no cache-slot arithmetic: both the
oracle and the GPU path receive the same storage bits from here and do their own work on them.

Random streams are counter-based: every tensor piece is drawn from
``numpy.random.default_rng([seed, stream, *index])``, so any piece (one head, one chunk of tokens,
one decode step) can be regenerated on its own without drawing the whole tensor. That lets the
1M-token workload be produced, uploaded and re-derived for the oracle one slice at a time.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

# Storage dtype tags (same numbering as the C ABI's duo_dtype_t).
F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}

# Stream ids for the counter-based generator.
S_HEADS, S_LENS, S_K, S_V, S_Q, S_TABLE, S_GARBAGE, S_KSTEP, S_VSTEP, S_ROWSCALE, S_CHSCALE = range(11)


# ----------------------------------------------------------------------------------------------
# Rounding to storage bits (round to nearest, ties to even)
# ----------------------------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even; NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u.astype(np.uint64) + bias) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def f32_to_storage(x: np.ndarray, dtype: int) -> np.ndarray:
    """fp32 values -> the array whose bytes are what the device holds.

    F32 -> float32 array; F16 -> uint16 bit patterns (numpy's RNE cast); BF16 -> uint16 bit patterns.
    """
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype tag {dtype}")


def storage_np_dtype(dtype: int):
    return np.float32 if dtype == F32 else np.uint16


def normal(seed: int, stream: int, *index: int, shape) -> np.ndarray:
    """N(0,1) float32 draws for one addressable piece of a tensor."""
    rng = np.random.default_rng([seed, stream, *index])
    return rng.standard_normal(shape, dtype=np.float32)


def garbage_bits(seed: int, *index: int, shape, dtype: int) -> np.ndarray:
    """Arbitrary bit patterns (NaN and Inf encodings included) for cache slots nobody may read."""
    rng = np.random.default_rng([seed, S_GARBAGE, *index])
    if dtype == F32:
        return rng.integers(0, 2**32, size=shape, dtype=np.uint32).view(np.float32)
    return rng.integers(0, 2**16, size=shape, dtype=np.uint16)


# ----------------------------------------------------------------------------------------------
# Workload descriptions
# ----------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: int
    block_size: int
    sink: int
    recent: int
    retrieval: tuple            # kv-head ids with full attention (per-kv-head mask)
    context: int                # tokens the timed call attends over (see the per-workload notes)
    q_len: int                  # query rows per attention call (1 = decode)
    ring_blocks: int
    max_blocks_per_head: int
    seed: int
    steps: int = 1              # decode steps or prefill chunks
    note: str = ""
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def sink_blocks(self) -> int:
        return -(-self.sink // self.block_size)

    @property
    def retrieval_mask(self) -> np.ndarray:
        m = np.zeros(self.num_kv_heads, dtype=np.uint8)
        m[list(self.retrieval)] = 1
        return m

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]


def _ring_blocks_for(recent: int, q_len: int, block_size: int) -> int:
    # the ring must still hold the oldest key the first query of a chunk sees; a negative recent
    # is a window of -recent whole blocks
    span = recent if recent > 0 else -recent * block_size
    return -(-(span + q_len - 1) // block_size)


def _max_blocks(capacity_tokens: int, sink: int, ring_blocks: int, block_size: int) -> int:
    return max(-(-capacity_tokens // block_size), -(-sink // block_size) + ring_blocks)


def _pick_heads(seed: int, n: int, k: int) -> tuple:
    rng = np.random.default_rng([seed, S_HEADS])
    return tuple(sorted(int(h) for h in rng.permutation(n)[:k]))


def tiny() -> Workload:
    """fp32, 1 sequence, 4 q / 4 kv heads (0,1 retrieval), D 64, sink 4, recent 64; prefill 512 tokens
    then 16 decode steps."""
    bs, sink, recent, q_len = 16, 4, 64, 512
    rb = _ring_blocks_for(recent, q_len, bs)
    return Workload("tiny-f32-prefill512-decode16", 1, 4, 4, 64, F32, bs, sink, recent, (0, 1),
                    context=512, q_len=q_len, ring_blocks=rb,
                    max_blocks_per_head=_max_blocks(512 + 16, sink, rb, bs), seed=1, steps=16)


def llama3_8b_decode(batch: int = 8, context: int = 32768) -> Workload:
    """Llama-3-8B-shaped single-layer decode: 32 q / 8 kv heads (GQA 4:1), D 128, bf16, batch 8,
    32768 valid tokens at the timed decode (the decoded token included), 4 of 8 kv heads retrieval,
    sink 64, recent 256, pages of 16."""
    bs, sink, recent = 16, 64, 256
    rb = _ring_blocks_for(recent, 1, bs)
    return Workload(f"llama3-8b-gqa-decode-b{batch}-ctx{context}", batch, 32, 8, 128, BF16, bs, sink,
                    recent, _pick_heads(2, 8, 4), context=context, q_len=1, ring_blocks=rb,
                    max_blocks_per_head=_max_blocks(context, sink, rb, bs), seed=2)


def llama2_7b_chunked_prefill(chunk: int = 4096, chunks: int = 8) -> Workload:
    """Llama-2-7B-shaped MHA chunked prefill: 32 heads, D 128, bf16, batch 1, eight 4096-token chunks
    build a 32768-token context; 8 of 32 heads retrieval; sink 128, recent 1024."""
    bs, sink, recent = 16, 128, 1024
    rb = _ring_blocks_for(recent, chunk, bs)
    ctx = chunk * chunks
    return Workload(f"llama2-7b-mha-chunked-prefill-{chunks}x{chunk}", 1, 32, 32, 128, BF16, bs, sink,
                    recent, _pick_heads(3, 32, 8), context=ctx, q_len=chunk, ring_blocks=rb,
                    max_blocks_per_head=_max_blocks(ctx, sink, rb, bs), seed=3, steps=chunks)


def gemma_2b_static_decode(batch: int = 16, capacity: int = 8192) -> Workload:
    """Gemma-2b-shaped static-cache decode: 8 q heads over 1 kv head (MQA), D 256, fp16, capacity
    8192, batch 16, valid lengths uniform in [1024, 8192], every head retrieval, slots past each
    length hold arbitrary bits. Identity block table: the pool is the contiguous cache."""
    bs = 16
    return Workload(f"gemma-2b-mqa-static-decode-b{batch}-cap{capacity}", batch, 8, 1, 256, F16, bs,
                    0, 1, (0,), context=capacity, q_len=1, ring_blocks=1,
                    max_blocks_per_head=capacity // bs, seed=4)


def long_context_decode(context: int = 1 << 20, steps: int = 64) -> Workload:
    """Llama-3-8B GQA shape at batch 1 over a 1,048,576-token circular paged cache, 4 of 8 kv heads
    retrieval, sink 64, recent 256; then 64 steps of append + decode."""
    bs, sink, recent = 16, 64, 256
    rb = _ring_blocks_for(recent, 1, bs)
    return Workload(f"llama3-8b-gqa-decode-b1-ctx{context}", 1, 32, 8, 128, BF16, bs, sink, recent,
                    _pick_heads(5, 8, 4), context=context, q_len=1, ring_blocks=rb,
                    max_blocks_per_head=_max_blocks(context + steps, sink, rb, bs), seed=5,
                    steps=steps)


def qwen2_72b_dca_prefill(chunk: int = 32768, chunks: int = 4, chunk_len: int = 32768) -> Workload:
    """Qwen2-72B-shaped Dual Chunk Attention prefill, one GPU's share at tensor parallelism 4 (the
    DualChunkAttention PR's usage example: chunk_size 32768, chunked prefill of 32768 batched
    tokens, tensor_parallel_size 4): 64 / 4 = 16 q heads over 8 / 4 = 2 kv heads, D 128, bf16,
    batch 1; four 32768-token chunks build a 131072-token context, so the last chunk's queries meet
    intra-, succ- and inter-chunk keys. Every kv head is a full head."""
    bs = 16
    ctx = chunk * chunks
    return Workload(f"qwen2-72b-tp4-dca-prefill-{chunks}x{chunk}-c{chunk_len}", 1, 16, 2, 128, BF16,
                    bs, 0, 1, (0, 1), context=ctx, q_len=chunk, ring_blocks=1,
                    max_blocks_per_head=_max_blocks(ctx, 0, 1, bs), seed=6, steps=chunks,
                    extra={"chunk_len": chunk_len})


def continuous_batching_step(batch: int = 32, context: int = 32768, chunk: int = 4096) -> Workload:
    """A continuous-batching step on the Llama-3-8B GQA shape (32 q / 8 kv heads, D 128, bf16, 4 of
    8 kv heads retrieval, sink 64, recent 256, pages of 16): sequence 0 brings a 4096-row prompt
    chunk that ends its 32768-token context, the other 31 sequences one decode row each at 32768
    tokens. The ring holds a whole chunk's windows."""
    bs, sink, recent = 16, 64, 256
    rb = _ring_blocks_for(recent, chunk, bs)
    return Workload(f"llama3-8b-gqa-continuous-batching-b{batch}-ctx{context}-chunk{chunk}", batch,
                    32, 8, 128, BF16, bs, sink, recent, _pick_heads(2, 8, 4), context=context,
                    q_len=chunk, ring_blocks=rb, max_blocks_per_head=_max_blocks(context, sink, rb, bs),
                    seed=7, extra={"rows": [chunk] + [1] * (batch - 1)})


def small(name: str, *, batch=2, q_heads=4, kv_heads=2, head_dim=64, dtype=BF16, block_size=16,
          sink=4, recent=24, retrieval=(0,), context=100, q_len=1, seed=11, ring_blocks=None,
          capacity=None) -> Workload:
    """Small custom workloads for oracle pins and edge cases."""
    rb = ring_blocks if ring_blocks is not None else _ring_blocks_for(recent, q_len, block_size)
    cap = capacity if capacity is not None else context
    return Workload(name, batch, q_heads, kv_heads, head_dim, dtype, block_size, sink, recent,
                    tuple(retrieval), context=context, q_len=q_len, ring_blocks=rb,
                    max_blocks_per_head=_max_blocks(cap, sink, rb, block_size), seed=seed)


ALL = {
    "tiny": tiny,
    "llama3-8b-decode": llama3_8b_decode,
    "llama2-7b-chunked-prefill": llama2_7b_chunked_prefill,
    "gemma-2b-static-decode": gemma_2b_static_decode,
    "long-context-decode": long_context_decode,
    "qwen2-72b-dca-prefill": qwen2_72b_dca_prefill,
    "continuous-batching-step": continuous_batching_step,
}


# ----------------------------------------------------------------------------------------------
# Block tables
# ----------------------------------------------------------------------------------------------
def pages_needed(w: Workload, kv_head: int) -> int:
    """Table columns a (sequence, kv head) row uses: the whole row for a retrieval head, the sink
    pages plus the ring pages for a streaming head."""
    if kv_head in w.retrieval:
        return w.max_blocks_per_head
    return w.sink_blocks + w.ring_blocks


def block_table(w: Workload, *, shuffle: bool = True, identity: bool = False,
                share_sinks: bool = False):
    """Block table [batch][kv_heads][max_blocks_per_head] int32 and the pool size in pages.

    Every (sequence, kv head) gets its own pages. Physical page ids are a seeded permutation (or the
    identity when ``identity``); unused columns hold 0, a valid page id that no kernel may read.
    With ``share_sinks`` a streaming kv head's sink pages are allocated once and every sequence's
    row points at them (sequences whose first sink tokens are the same; the ring stays private).
    """
    sb = w.sink_blocks
    def own(b, h):
        if share_sinks and h not in w.retrieval and b > 0:
            return pages_needed(w, h) - sb
        return pages_needed(w, h)
    total = int(sum(own(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)))
    ids = np.arange(total, dtype=np.int64)
    if shuffle and not identity:
        ids = np.random.default_rng([w.seed, S_TABLE]).permutation(total)
    table = np.zeros((w.batch, w.num_kv_heads, w.max_blocks_per_head), dtype=np.int32)
    pos = 0
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            n = own(b, h)
            if n < pages_needed(w, h):       # shared sink pages: those of sequence 0
                table[b, h, :sb] = table[0, h, :sb]
                table[b, h, sb:sb + n] = ids[pos:pos + n]
            else:
                table[b, h, :n] = ids[pos:pos + n]
            pos += n
    return table, total


# ----------------------------------------------------------------------------------------------
# Token data
# ----------------------------------------------------------------------------------------------
KV_CHUNK = 4096  # tokens per addressable generator piece


def kv_tokens(w: Workload, which: int, b: int, h: int, start: int, stop: int) -> np.ndarray:
    """Context K (which=S_K) or V (which=S_V) for sequence b, kv head h, positions [start, stop):
    float32 [stop-start][D], drawn piecewise in KV_CHUNK-token pieces."""
    out = np.empty((stop - start, w.head_dim), dtype=np.float32)
    c0, c1 = start // KV_CHUNK, (stop - 1) // KV_CHUNK if stop > start else start // KV_CHUNK - 1
    for c in range(c0, c1 + 1):
        piece = normal(w.seed, which, b, h, c, shape=(KV_CHUNK, w.head_dim))
        lo, hi = max(start, c * KV_CHUNK), min(stop, (c + 1) * KV_CHUNK)
        out[lo - start:hi - start] = piece[lo - c * KV_CHUNK:hi - c * KV_CHUNK]
    return out


def kv_new(w: Workload, which: int, start: int, stop: int, batch_lens=None) -> np.ndarray:
    """New K or V rows in the append layout [batch][stop-start][kv_heads][D], float32."""
    T = stop - start
    out = np.empty((w.batch, T, w.num_kv_heads, w.head_dim), dtype=np.float32)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            out[b, :, h, :] = kv_tokens(w, which, b, h, start, stop)
    return out


def queries(w: Workload, step: int, q_len: int | None = None) -> np.ndarray:
    """Query rows for one attention call: float32 [batch][q_len][q_heads][D]."""
    q_len = w.q_len if q_len is None else q_len
    return normal(w.seed, S_Q, step, shape=(w.batch, q_len, w.num_q_heads, w.head_dim))


def row_scales(w: Workload, step: int, q_len: int, lo: float = 1.0, hi: float = 1.4) -> np.ndarray:
    """One positive float32 factor per query row, uniform in [lo, hi): float32 [batch][q_len] (the
    per-position scale factor Dual Chunk Attention takes; synthetic values, no method arithmetic)."""
    rng = np.random.default_rng([w.seed, S_ROWSCALE, step])
    return rng.uniform(lo, hi, size=(w.batch, q_len)).astype(np.float32)


def channel_scales(w: Workload, which: int, lo: float = 0.45, hi: float = 0.65) -> np.ndarray:
    """Per-(kv head, channel) scales float32 [Hkv][D] for a 4-bit cache of K (which = S_K) or V
    (S_V): seeded draws in [lo, hi), standing in for scales calibrated offline on N(0, 1) data
    (7 steps of 0.45-0.65 reach 3.2-4.6 standard deviations)."""
    rng = np.random.default_rng([w.seed, S_CHSCALE, which])
    return rng.uniform(lo, hi, (w.num_kv_heads, w.head_dim)).astype(np.float32)


def valid_lengths(w: Workload, lo: int, hi: int) -> np.ndarray:
    """Per-sequence valid lengths uniform in [lo, hi] (inclusive), int32."""
    rng = np.random.default_rng([w.seed, S_LENS])
    return rng.integers(lo, hi + 1, size=w.batch).astype(np.int32)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (used by tests to read device outputs)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def storage_to_f32(a: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.asarray(a, dtype=np.float32)
    if dtype == F16:
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float32)
    return bf16_bits_to_f32(a)


__all__ = [n for n in dir() if not n.startswith("_")]
