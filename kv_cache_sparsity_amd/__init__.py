"""Python binding of libduoattn: mixed-head attention over a paged, per-head circular KV cache.

Argument marshalling only. Every step of the computation runs in the library's HIP kernels; this
module turns torch tensors into device pointers and sizes, calls the C ABI declared in
``include/duo_attn.h`` (same function names), and raises ``DuoAttnError`` on a non-zero status.
If ``libduoattn.so`` has not been built the calls fail loudly; there is no fallback.

Tensor layouts (all contiguous, on the GPU, one dtype per call: float32, float16 or bfloat16):
  k_pool [num_blocks][block_size][head_dim]   v_pool [num_blocks][head_dim][block_size]
  block_table int32 [batch][num_kv_heads][max_blocks_per_head]
  append:  k_new, v_new [batch][t_new][num_kv_heads][head_dim]
  decode:  q, out [batch][num_q_heads][head_dim]
  prefill: q, out [batch][q_len][num_q_heads][head_dim]
  dca:     q, q_succ, q_inter, out [batch][q_len][num_q_heads][head_dim], mscale float32 [batch][q_len]
           (decode: [batch][num_q_heads][head_dim] and mscale [batch])
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libduoattn.so")

DUO_F32, DUO_F16, DUO_BF16 = 0, 1, 2
STATUS = {0: "DUO_OK", 1: "DUO_ERR_INVALID_ARG", 2: "DUO_ERR_UNSUPPORTED", 3: "DUO_ERR_CAPACITY",
          4: "DUO_ERR_WORKSPACE", 5: "DUO_ERR_HIP"}
SYMBOLS = ("kv_append_circular", "duo_attn_decode_workspace_size", "duo_attn_decode",
           "duo_attn_prefill_workspace_size", "duo_attn_prefill", "duo_attn_prefill_varlen",
           "kv_append_circular_int8",
           "duo_attn_decode_int8", "dca_attn_prefill_workspace_size", "dca_attn_prefill",
           "dca_attn_decode", "duo_profile_next_launch",
           "duo_status_string", "duo_abi_version")


class DuoAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} "
                         f"({status_string(status)})")


_lib = None
_P, _I32, _SZ, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_sparsity_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        L.kv_append_circular.restype = _I32
        L.kv_append_circular.argtypes = [_P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _I32, _I32,
                                         _I32, _I32, _I32, _P, _I32, _I32, _I32, _P]
        L.duo_attn_decode_workspace_size.restype = _SZ
        L.duo_attn_decode_workspace_size.argtypes = [_I32] * 7
        L.duo_attn_decode.restype = _I32
        L.duo_attn_decode.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _P, _I32, _I32, _I32,
                                      _I32, _I32, _P, _I32, _I32, _I32, _F, _P, _P, _SZ, _I32, _P]
        L.duo_attn_prefill_workspace_size.restype = _SZ
        L.duo_attn_prefill_workspace_size.argtypes = [_I32] * 6 + [_P]
        L.duo_attn_prefill.restype = _I32
        L.duo_attn_prefill.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _P, _I32, _I32, _I32,
                                       _I32, _I32, _I32, _P, _I32, _I32, _I32, _F, _P, _P, _SZ,
                                       _P]
        L.duo_attn_prefill_varlen.restype = _I32
        L.duo_attn_prefill_varlen.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _I32, _I32,
                                              _I32, _I32, _I32, _I32, _I32, _P, _I32, _I32, _I32,
                                              _F, _P, _P, _SZ, _P]
        L.kv_append_circular_int8.restype = _I32
        L.kv_append_circular_int8.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P,
                                              _I32, _I32, _I32, _I32, _I32, _P, _I32, _I32, _I32,
                                              _P]
        L.duo_attn_decode_int8.restype = _I32
        L.duo_attn_decode_int8.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _I32, _I32,
                                           _I32, _I32, _I32, _P, _I32, _I32, _I32, _F, _P, _P, _SZ,
                                           _I32, _P]
        L.duo_status_string.restype = ctypes.c_char_p
        L.dca_attn_prefill_workspace_size.restype = _SZ
        L.dca_attn_prefill_workspace_size.argtypes = [_I32] * 6
        L.dca_attn_prefill.restype = _I32
        L.dca_attn_prefill.argtypes = [_P, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32, _I32, _P, _I32,
                                       _I32, _I32, _I32, _I32, _I32, _F, _P, _P, _SZ, _P]
        L.dca_attn_decode.restype = _I32
        L.dca_attn_decode.argtypes = [_P, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32, _I32, _P, _I32,
                                      _I32, _I32, _I32, _I32, _F, _P, _P, _SZ, _I32, _P]
        L.duo_profile_next_launch.restype = _I32
        L.duo_profile_next_launch.argtypes = [_P, _P]
        L.duo_status_string.argtypes = [_I32]
        L.duo_abi_version.restype = _I32
        L.duo_abi_version.argtypes = []
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().duo_status_string(status).decode()


def abi_version() -> int:
    return lib().duo_abi_version()


# ---- torch marshalling ---------------------------------------------------------------------------
def _dtype_tag(t) -> int:
    import torch
    tags = {torch.float32: DUO_F32, torch.float16: DUO_F16, torch.bfloat16: DUO_BF16}
    if t.dtype not in tags:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return tags[t.dtype]


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    return getattr(stream, "cuda_stream", stream) or None


class _HostMask:
    """head_is_retrieval as a host uint8 array kept alive for the call."""

    def __init__(self, mask):
        vals = [int(x) for x in (mask.tolist() if hasattr(mask, "tolist") else mask)]
        self.n = len(vals)
        self.buf = (ctypes.c_uint8 * max(1, self.n))(*vals)

    @property
    def ptr(self):
        return ctypes.cast(self.buf, ctypes.c_void_p)


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise DuoAttnError(fn, status)


def kv_append_circular(k_pool, v_pool, block_table, k_new, v_new, seq_lens_before, seq_lens_after,
                       head_is_retrieval, sink_size: int, recent_size: int, ring_blocks: int,
                       stream=None) -> None:
    num_blocks, block_size, head_dim = k_pool.shape
    batch, t_new, num_kv_heads, _ = k_new.shape
    mask = _HostMask(head_is_retrieval)
    st = lib().kv_append_circular(
        _ptr(k_pool), _ptr(v_pool), _ptr(block_table), num_blocks, block_size,
        block_table.shape[2], _ptr(k_new), _ptr(v_new), _ptr(seq_lens_before),
        _ptr(seq_lens_after), batch, t_new, num_kv_heads, head_dim, _dtype_tag(k_pool), mask.ptr,
        sink_size, recent_size, ring_blocks, _stream(stream))
    _check("kv_append_circular", st)


def duo_attn_decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                   max_blocks_per_head: int, block_size: int,
                                   split_tokens: int = 0) -> int:
    return lib().duo_attn_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                                max_blocks_per_head, block_size, split_tokens)


def decode_workspace(q, block_table, block_size: int, split_tokens: int = 0):
    """Allocate a zero-filled workspace for duo_attn_decode with these shapes."""
    import torch
    batch, num_q_heads, head_dim = q.shape
    n = duo_attn_decode_workspace_size(batch, num_q_heads, block_table.shape[1], head_dim,
                                       block_table.shape[2], block_size, split_tokens)
    if n == 0:
        raise ValueError("invalid sizes for the decode workspace")
    return torch.zeros(n, dtype=torch.uint8, device=q.device)


def duo_attn_decode(q, k_pool, v_pool, block_table, seq_lens, head_is_retrieval, sink_size: int,
                    recent_size: int, ring_blocks: int, softmax_scale: float, out, workspace,
                    split_tokens: int = 0, stream=None) -> None:
    num_blocks, block_size, head_dim = k_pool.shape
    batch, num_q_heads, _ = q.shape
    mask = _HostMask(head_is_retrieval)
    st = lib().duo_attn_decode(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), num_blocks, block_size,
        block_table.shape[2], _ptr(seq_lens), batch, num_q_heads, block_table.shape[1], head_dim,
        _dtype_tag(q), mask.ptr, sink_size, recent_size, ring_blocks, softmax_scale, _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), split_tokens,
        _stream(stream))
    _check("duo_attn_decode", st)


def duo_attn_prefill_workspace_size(batch: int, q_len: int, num_q_heads: int, num_kv_heads: int,
                                    head_dim: int, dtype: int, head_is_retrieval) -> int:
    mask = _HostMask(head_is_retrieval)
    return lib().duo_attn_prefill_workspace_size(batch, q_len, num_q_heads, num_kv_heads, head_dim,
                                                 dtype, mask.ptr)


def prefill_workspace(q, block_table, head_is_retrieval, head_dim: int | None = None):
    """Allocate a zero-filled workspace for duo_attn_prefill with these shapes."""
    import torch
    batch, q_len, num_q_heads, d = q.shape
    n = duo_attn_prefill_workspace_size(batch, q_len, num_q_heads, block_table.shape[1],
                                        head_dim or d, _dtype_tag(q), head_is_retrieval)
    if n == 0:
        raise ValueError("invalid sizes for the prefill workspace")
    return torch.zeros(n, dtype=torch.uint8, device=q.device)


def duo_attn_prefill(q, k_pool, v_pool, block_table, seq_lens, head_is_retrieval, sink_size: int,
                     recent_size: int, ring_blocks: int, softmax_scale: float, out, workspace,
                     stream=None) -> None:
    num_blocks, block_size, head_dim = k_pool.shape
    batch, q_len, num_q_heads, _ = q.shape
    mask = _HostMask(head_is_retrieval)
    st = lib().duo_attn_prefill(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), num_blocks, block_size,
        block_table.shape[2], _ptr(seq_lens), batch, q_len, num_q_heads, block_table.shape[1],
        head_dim, _dtype_tag(q), mask.ptr, sink_size, recent_size, ring_blocks, softmax_scale,
        _ptr(out), _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check("duo_attn_prefill", st)


def duo_attn_prefill_varlen(q, k_pool, v_pool, block_table, seq_lens, q_start, max_q_len: int,
                            head_is_retrieval, sink_size: int, recent_size: int, ring_blocks: int,
                            softmax_scale: float, out, workspace, stream=None) -> None:
    """Prefill of a packed batch: q, out [total_q][Hq][D]; q_start int32 [batch + 1] (device) gives
    each sequence's rows; max_q_len bounds any sequence's rows (the workspace is
    prefill_workspace for q_len = max_q_len)."""
    num_blocks, block_size, head_dim = k_pool.shape
    total_q, num_q_heads, _ = q.shape
    batch = q_start.shape[0] - 1
    mask = _HostMask(head_is_retrieval)
    st = lib().duo_attn_prefill_varlen(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), num_blocks, block_size,
        block_table.shape[2], _ptr(seq_lens), _ptr(q_start), batch, total_q, max_q_len,
        num_q_heads, block_table.shape[1], head_dim, _dtype_tag(q), mask.ptr, sink_size,
        recent_size, ring_blocks, softmax_scale, _ptr(out), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _check("duo_attn_prefill_varlen", st)


def prefill_varlen_workspace(q, block_table, head_is_retrieval, max_q_len: int, batch: int):
    """Zero-filled workspace for duo_attn_prefill_varlen (q: [total_q][Hq][D])."""
    import torch
    _, num_q_heads, d = q.shape
    n = duo_attn_prefill_workspace_size(batch, max_q_len, num_q_heads, block_table.shape[1], d,
                                        _dtype_tag(q), head_is_retrieval)
    if n == 0:
        raise ValueError("invalid sizes for the prefill workspace")
    return torch.zeros(n, dtype=torch.uint8, device=q.device)


def _int8_pools(k_pool, v_pool, k_scale, v_scale):
    import torch
    if k_pool.dtype != torch.int8 or v_pool.dtype != torch.int8:
        raise TypeError("int8 cache pools must be torch.int8")
    if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32:
        raise TypeError("int8 cache scales must be torch.float32")


def kv_append_circular_int8(k_pool, v_pool, k_scale, v_scale, block_table, k_new, v_new,
                            seq_lens_before, seq_lens_after, head_is_retrieval, sink_size: int,
                            recent_size: int, ring_blocks: int, stream=None) -> None:
    """Quantize and append new rows into the int8 cache: k_pool int8 [NB][bs][D], v_pool int8
    [NB][D][bs], k_scale / v_scale float32 [NB][bs]; k_new / v_new [B][t_new][Hkv][D]."""
    _int8_pools(k_pool, v_pool, k_scale, v_scale)
    num_blocks, block_size, head_dim = k_pool.shape
    batch, t_new, num_kv_heads, _ = k_new.shape
    mask = _HostMask(head_is_retrieval)
    st = lib().kv_append_circular_int8(
        _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table), num_blocks,
        block_size, block_table.shape[2], _ptr(k_new), _ptr(v_new), _ptr(seq_lens_before),
        _ptr(seq_lens_after), batch, t_new, num_kv_heads, head_dim, _dtype_tag(k_new), mask.ptr,
        sink_size, recent_size, ring_blocks, _stream(stream))
    _check("kv_append_circular_int8", st)


def duo_attn_decode_int8(q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens,
                         head_is_retrieval, sink_size: int, recent_size: int, ring_blocks: int,
                         softmax_scale: float, out, workspace, split_tokens: int = 0,
                         stream=None) -> None:
    """duo_attn_decode over the int8 cache (pools and scales as for kv_append_circular_int8)."""
    _int8_pools(k_pool, v_pool, k_scale, v_scale)
    num_blocks, block_size, head_dim = k_pool.shape
    batch, num_q_heads, _ = q.shape
    mask = _HostMask(head_is_retrieval)
    st = lib().duo_attn_decode_int8(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        num_blocks, block_size, block_table.shape[2], _ptr(seq_lens), batch, num_q_heads,
        block_table.shape[1], head_dim, _dtype_tag(q), mask.ptr, sink_size, recent_size,
        ring_blocks, softmax_scale, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), split_tokens, _stream(stream))
    _check("duo_attn_decode_int8", st)


def dca_attn_prefill_workspace_size(batch: int, q_len: int, num_q_heads: int, num_kv_heads: int,
                                    head_dim: int, dtype: int) -> int:
    return int(lib().dca_attn_prefill_workspace_size(batch, q_len, num_q_heads, num_kv_heads,
                                                     head_dim, dtype))


def dca_prefill_workspace(q, block_table):
    """Zero-filled workspace for dca_attn_prefill (q: [B][q_len][Hq][D])."""
    import torch
    batch, q_len, num_q_heads, d = q.shape
    n = dca_attn_prefill_workspace_size(batch, q_len, num_q_heads, block_table.shape[1], d,
                                        _dtype_tag(q))
    if n == 0:
        raise ValueError("invalid sizes for the Dual Chunk Attention workspace")
    return torch.zeros(n, dtype=torch.uint8, device=q.device)


def dca_attn_prefill(q, q_succ, q_inter, mscale, chunk_len: int, k_pool, v_pool, block_table,
                     seq_lens, softmax_scale: float, out, workspace, stream=None) -> None:
    """Dual Chunk Attention prefill: q, q_succ, q_inter, out [B][q_len][Hq][D] (float16 or
    bfloat16); mscale float32 [B][q_len]; the cache filled with every kv head a retrieval head."""
    import torch
    if mscale.dtype != torch.float32:
        raise TypeError("mscale must be torch.float32")
    num_blocks, block_size, head_dim = k_pool.shape
    batch, q_len, num_q_heads, _ = q.shape
    st = lib().dca_attn_prefill(
        _ptr(q), _ptr(q_succ), _ptr(q_inter), _ptr(mscale), chunk_len, _ptr(k_pool), _ptr(v_pool),
        _ptr(block_table), num_blocks, block_size, block_table.shape[2], _ptr(seq_lens), batch,
        q_len, num_q_heads, block_table.shape[1], head_dim, _dtype_tag(q), softmax_scale,
        _ptr(out), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dca_attn_prefill", st)


def dca_attn_decode(q, q_succ, q_inter, mscale, chunk_len: int, k_pool, v_pool, block_table,
                    seq_lens, softmax_scale: float, out, workspace, split_tokens: int = 0,
                    stream=None) -> None:
    """Dual Chunk Attention decode: q, q_succ, q_inter, out [B][Hq][D] (float16 or bfloat16);
    mscale float32 [B]; workspace as for duo_attn_decode (decode_workspace)."""
    import torch
    if mscale.dtype != torch.float32:
        raise TypeError("mscale must be torch.float32")
    num_blocks, block_size, head_dim = k_pool.shape
    batch, num_q_heads, _ = q.shape
    st = lib().dca_attn_decode(
        _ptr(q), _ptr(q_succ), _ptr(q_inter), _ptr(mscale), chunk_len, _ptr(k_pool), _ptr(v_pool),
        _ptr(block_table), num_blocks, block_size, block_table.shape[2], _ptr(seq_lens), batch,
        num_q_heads, block_table.shape[1], head_dim, _dtype_tag(q), softmax_scale, _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), split_tokens,
        _stream(stream))
    _check("dca_attn_decode", st)


def profile_next_launch(start_event=None, stop_event=None) -> None:
    """The next attention call on this thread records start_event / stop_event at its kernel's
    own start and end (torch.cuda.Event with timing, already recorded once so that it exists, or a
    raw hipEvent_t handle)."""
    def handle(e):
        if e is None:
            return None
        h = int(getattr(e, "cuda_event", e))
        if h == 0:
            raise ValueError("the event does not exist yet: record it once first")
        return h
    _check("duo_profile_next_launch",
           lib().duo_profile_next_launch(handle(start_event), handle(stop_event)))


__all__ = ["kv_append_circular", "duo_attn_decode", "duo_attn_prefill",
           "kv_append_circular_int8", "duo_attn_decode_int8", "duo_attn_prefill_varlen",
           "prefill_varlen_workspace", "dca_attn_prefill", "dca_attn_prefill_workspace_size", "dca_attn_decode",
           "profile_next_launch",
           "dca_prefill_workspace",
           "duo_attn_decode_workspace_size", "decode_workspace", "duo_attn_prefill_workspace_size",
           "prefill_workspace", "status_string", "abi_version",
           "DuoAttnError", "lib", "LIB_PATH", "SYMBOLS", "DUO_F32", "DUO_F16", "DUO_BF16"]
