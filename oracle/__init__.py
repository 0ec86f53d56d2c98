"""CPU fp64 oracle for mixed-head attention over a block-paged, per-head circular KV cache.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The library (``kv_cache_sparsity_amd``) never imports it and
shares no code with it: no kernels, headers, helpers, tables or pre/post-processing. The oracle is
slow on purpose; every function follows the definition on the pages step by step.

Sources (the four web pages on KV-cache sparsity):
  * DuoAttention README ("DuoAttention: efficient long-context LLM inference with retrieval and
    streaming heads"), abstract and quick-start: retrieval heads keep full attention over all
    tokens; streaming heads keep only the attention sinks and the recent tokens.
  * vLLM issue "Could you support Attention Sink?": block-paged cache, the circular-buffer slot
    tables (with and without in-place sinks) and option 3 (sinks in their own block, a ring for the
    streamed tokens).
  * transformers PR "[WIP] Dynamic length in static cache", description: a new position only needs
    attention against the positions up to itself, not the whole static cache.
  * DuoAttention README, installation and efficiency sections: the method paired with a quantized
    KV cache (8-bit codes with a scale per stored row, ``quant``; 4-bit codes with a static scale
    per kv head and channel, ``quant4``, after the pages' "kv4-per-channel" demo models).
  * vLLM PR "[Model] Implement DualChunkAttention for Qwen2 Models", review thread: the softmax
    scale is applied in fp32 to the q.k product; Dual Chunk Attention itself (``dca``): three query
    vectors chosen by the chunk relation of query and key, a float32 mscale per query position.

Parity status of each function is stated in its docstring; every function here is pinned by tests
in ``tests/test_oracle_*.py`` (worked tables, brute force, a library cross-check, closed forms and
invariants). Two conventions inside ``attend`` are parity unpinned by the pages, which fix neither:
the grouping of q heads onto kv heads (contiguous, hq // (Hq / Hkv); pinned only internally by
"repeating each kv head turns GQA into MHA") and the value of the softmax scale (an argument).
"""
from .cache import (slot_of, table_position, append, gather, pool_shapes, to_f64,
                    new_pools, ring_capacity)
from .attention import (visible_positions, visible_mask, attend_row, attend_rows, attend,
                        attend_paged)
from .quant import quantize_rows, dequantize, scale_pool_shape, append_int8, attend_int8
from .dca import query_kind, attend_dca_row, attend_dca, attend_dca_rows
from .quant4 import (quantize_rows4, dequantize4, pack4, unpack4, pool4_shapes, append_int4,
                     attend_int4)

__all__ = ["slot_of", "table_position", "append", "gather", "pool_shapes", "to_f64", "new_pools",
           "ring_capacity", "visible_positions", "visible_mask", "attend_row", "attend_rows",
           "attend", "attend_paged",
           "quantize_rows", "dequantize", "scale_pool_shape", "append_int8", "attend_int8",
           "query_kind", "attend_dca_row", "attend_dca", "attend_dca_rows", "quantize_rows4",
           "dequantize4", "pack4", "unpack4", "pool4_shapes", "append_int4", "attend_int4"]
