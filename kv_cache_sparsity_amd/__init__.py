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
           "duo_attn_append_decode", "duo_attn_append_decode_int8", "duo_attn_append_decode_int4",
           "duo_attn_decode_noalloc",
           "duo_attn_prefill_workspace_size", "duo_attn_prefill", "duo_attn_prefill_varlen", "duo_attn_prefill_varlen_workspace_size",
           "kv_append_circular_int8", "kv_append_circular_int4", "duo_attn_decode_int4",
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
        L.duo_attn_append_decode.restype = _I32
        L.duo_attn_append_decode.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _I32,
                                             _I32, _I32, _I32, _I32, _P, _I32, _I32, _I32, _F, _P,
                                             _P, _SZ, _I32, _P]
        L.duo_attn_decode_noalloc.restype = _I32
        L.duo_attn_decode_noalloc.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _P, _I32, _I32,
                                              _I32, _I32, _I32, _P, _I32, _I32, _I32, _F, _P,
                                              _I32, _P]
        L.duo_attn_prefill_workspace_size.restype = _SZ
        L.duo_attn_prefill_workspace_size.argtypes = [_I32] * 6 + [_P]
        L.duo_attn_prefill.restype = _I32
        L.duo_attn_prefill.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _P, _I32, _I32, _I32,
                                       _I32, _I32, _I32, _P, _I32, _I32, _I32, _F, _P, _P, _SZ,
                                       _P]
        L.duo_attn_prefill_varlen_workspace_size.restype = _SZ
        L.duo_attn_prefill_varlen_workspace_size.argtypes = [_I32] * 9 + [_P]
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
        L.duo_attn_append_decode_int8.restype = _I32
        L.duo_attn_append_decode_int8.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                                  _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _I32,
                                                  _I32, _I32, _F, _P, _P, _SZ, _I32, _P]
        L.duo_attn_append_decode_int4.restype = _I32
        L.duo_attn_append_decode_int4.argtypes = L.duo_attn_append_decode_int8.argtypes
        L.kv_append_circular_int4.restype = _I32
        L.kv_append_circular_int4.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P,
                                              _I32, _I32, _I32, _I32, _I32, _P, _I32, _I32, _I32,
                                              _P]
        L.duo_attn_decode_int4.restype = _I32
        L.duo_attn_decode_int4.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _I32, _I32,
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


# Argument checks. The C ABI takes raw pointers, so a tensor of the wrong dtype, shape or device
# would be read or written past its end; every wrapper checks its tensors here first.
def _fail_type(msg: str):
    raise TypeError(msg)


def _fail(msg: str):
    raise ValueError(msg)


def _check_tensor(t, name: str, dtype=None, shape=None, ndim=None, like=None):
    """t has `dtype` (or like's dtype), `shape` (None entries free) / `ndim`, and like's device."""
    if t is None:
        _fail(f"{name} is required")
    want = like.dtype if like is not None and dtype is None else dtype
    if want is not None and t.dtype != want:
        _fail_type(f"{name} must be {want}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(g) != int(w)
                                        for g, w in zip(t.shape, shape)):
            _fail(f"{name} must have shape {tuple('*' if x is None else x for x in shape)}, "
                  f"got {tuple(t.shape)}")
    elif ndim is not None and t.dim() != ndim:
        _fail(f"{name} must have {ndim} dimensions, got {t.dim()}")
    if like is not None and t.device != like.device:
        _fail(f"{name} is on {t.device}, expected {like.device}")


def _check_gpu(t, name: str):
    if not t.is_cuda:
        _fail(f"{name} must be a GPU tensor (device pointers only)")


def _int32():
    import torch
    return torch.int32


class _HostMask:
    """head_is_retrieval as a host uint8 array kept alive for the call (num_kv_heads entries, each
    0 or 1)."""

    def __init__(self, mask, num_kv_heads: int | None = None):
        vals = [int(x) for x in (mask.tolist() if hasattr(mask, "tolist") else mask)]
        self.n = len(vals)
        if num_kv_heads is not None and self.n != num_kv_heads:
            _fail(f"head_is_retrieval has {self.n} entries, expected num_kv_heads = {num_kv_heads}")
        if any(v not in (0, 1) for v in vals):
            _fail("head_is_retrieval entries must be 0 or 1")
        self.buf = (ctypes.c_uint8 * max(1, self.n))(*vals)

    @property
    def ptr(self):
        return ctypes.cast(self.buf, ctypes.c_void_p)


def _check_tables(block_table, seq_lens, batch: int, num_kv_heads: int, like, lens_name="seq_lens"):
    _check_tensor(block_table, "block_table", dtype=_int32(), shape=(batch, num_kv_heads, None),
                  like=like)
    _check_tensor(seq_lens, lens_name, dtype=_int32(), shape=(batch,), like=like)


def _kv_heads(block_table) -> int:
    """num_kv_heads from an int32 block table [batch][num_kv_heads][max_blocks_per_head]."""
    _check_tensor(block_table, "block_table", dtype=_int32(), ndim=3)
    return int(block_table.shape[1])


def _check_workspace(workspace, like, required: bool = True):
    if workspace is None:
        if required:
            _fail("workspace is required")
        return
    if workspace.device != like.device:
        _fail(f"workspace is on {workspace.device}, expected {like.device}")
    if not workspace.is_contiguous():
        _fail("workspace must be contiguous")


def _check_cache16(q, k_pool, v_pool, head_dim_axis=-1):
    """16-bit / fp32 pools of q's dtype: k [NB][bs][D], v [NB][D][bs]."""
    _check_tensor(k_pool, "k_pool", ndim=3, like=q)
    nb, bs, d = k_pool.shape
    if int(q.shape[head_dim_axis]) != int(d):
        _fail(f"q has head_dim {q.shape[head_dim_axis]}, the pools {d}")
    _check_tensor(v_pool, "v_pool", shape=(nb, d, bs), like=q)


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise DuoAttnError(fn, status)


def kv_append_circular(k_pool, v_pool, block_table, k_new, v_new, seq_lens_before, seq_lens_after,
                       head_is_retrieval, sink_size: int, recent_size: int, ring_blocks: int,
                       stream=None) -> None:
    _check_tensor(k_pool, "k_pool", ndim=3)
    num_blocks, block_size, head_dim = k_pool.shape
    _check_tensor(v_pool, "v_pool", shape=(num_blocks, head_dim, block_size), like=k_pool)
    _check_tensor(k_new, "k_new", ndim=4, like=k_pool)
    batch, t_new, num_kv_heads, _ = k_new.shape
    _check_tensor(k_new, "k_new", shape=(batch, t_new, num_kv_heads, head_dim), like=k_pool)
    _check_tensor(v_new, "v_new", shape=tuple(k_new.shape), like=k_pool)
    _check_tables(block_table, seq_lens_before, batch, num_kv_heads, k_pool, "seq_lens_before")
    if seq_lens_after is not None:
        _check_tensor(seq_lens_after, "seq_lens_after", dtype=_int32(), shape=(batch,), like=k_pool)
    for t, n in ((k_pool, "k_pool"),):
        _check_gpu(t, n)
    mask = _HostMask(head_is_retrieval, num_kv_heads)
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
    _check_tensor(q, "q", ndim=3)
    _check_cache16(q, k_pool, v_pool)
    num_blocks, block_size, head_dim = k_pool.shape
    batch, num_q_heads, _ = q.shape
    _check_tables(block_table, seq_lens, batch, _kv_heads(block_table), q)
    _check_tensor(out, "out", shape=tuple(q.shape), like=q)
    _check_workspace(workspace, q)
    _check_gpu(q, "q")
    mask = _HostMask(head_is_retrieval, block_table.shape[1])
    st = lib().duo_attn_decode(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), num_blocks, block_size,
        block_table.shape[2], _ptr(seq_lens), batch, num_q_heads, block_table.shape[1], head_dim,
        _dtype_tag(q), mask.ptr, sink_size, recent_size, ring_blocks, softmax_scale, _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), split_tokens,
        _stream(stream))
    _check("duo_attn_decode", st)


def duo_attn_append_decode(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens_before,
                           seq_lens_after, head_is_retrieval, sink_size: int, recent_size: int,
                           ring_blocks: int, softmax_scale: float, out, workspace,
                           split_tokens: int = 0, stream=None) -> None:
    """kv_append_circular of one token per sequence (k_new, v_new [batch][1][kv heads][head_dim])
    and duo_attn_decode of its queries over seq_lens_before + 1 keys, in one launch."""
    _check_tensor(q, "q", ndim=3)
    _check_cache16(q, k_pool, v_pool)
    num_blocks, block_size, head_dim = k_pool.shape
    batch, num_q_heads, _ = q.shape
    num_kv_heads = _kv_heads(block_table)
    _check_tables(block_table, seq_lens_before, batch, num_kv_heads, q, "seq_lens_before")
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _check_tensor(t, n, shape=(batch, 1, num_kv_heads, head_dim), like=q)
    if seq_lens_after is not None:
        _check_tensor(seq_lens_after, "seq_lens_after", dtype=_int32(), shape=(batch,), like=q)
    _check_tensor(out, "out", shape=tuple(q.shape), like=q)
    _check_workspace(workspace, q)
    _check_gpu(q, "q")
    mask = _HostMask(head_is_retrieval, num_kv_heads)
    st = lib().duo_attn_append_decode(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
        num_blocks, block_size, block_table.shape[2], _ptr(seq_lens_before), _ptr(seq_lens_after),
        batch, num_q_heads, num_kv_heads, head_dim, _dtype_tag(q), mask.ptr, sink_size,
        recent_size, ring_blocks, softmax_scale, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), split_tokens, _stream(stream))
    _check("duo_attn_append_decode", st)


NOALLOC_SCRATCH_BYTES = 16 << 20   # DUO_NOALLOC_SCRATCH_BYTES


def duo_attn_decode_noalloc(q, k_pool, v_pool, block_table, seq_lens, head_is_retrieval,
                            sink_size: int, recent_size: int, ring_blocks: int,
                            softmax_scale: float, out, split_tokens: int = 0, stream=None) -> None:
    """duo_attn_decode without a workspace argument: the library's static per-GPU scratch serves
    instead, and the call allocates no device memory. Calls that overlap on one GPU race."""
    _check_tensor(q, "q", ndim=3)
    _check_cache16(q, k_pool, v_pool)
    num_blocks, block_size, head_dim = k_pool.shape
    batch, num_q_heads, _ = q.shape
    _check_tables(block_table, seq_lens, batch, _kv_heads(block_table), q)
    _check_tensor(out, "out", shape=tuple(q.shape), like=q)
    _check_gpu(q, "q")
    mask = _HostMask(head_is_retrieval, block_table.shape[1])
    st = lib().duo_attn_decode_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), num_blocks, block_size,
        block_table.shape[2], _ptr(seq_lens), batch, num_q_heads, block_table.shape[1], head_dim,
        _dtype_tag(q), mask.ptr, sink_size, recent_size, ring_blocks, softmax_scale, _ptr(out),
        split_tokens, _stream(stream))
    _check("duo_attn_decode_noalloc", st)


def duo_attn_prefill_workspace_size(batch: int, q_len: int, num_q_heads: int, num_kv_heads: int,
                                    head_dim: int, dtype: int, head_is_retrieval) -> int:
    mask = _HostMask(head_is_retrieval, num_kv_heads)
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
    _check_tensor(q, "q", ndim=4)
    _check_cache16(q, k_pool, v_pool)
    num_blocks, block_size, head_dim = k_pool.shape
    batch, q_len, num_q_heads, _ = q.shape
    _check_tables(block_table, seq_lens, batch, _kv_heads(block_table), q)
    _check_tensor(out, "out", shape=tuple(q.shape), like=q)
    _check_workspace(workspace, q, required=False)
    _check_gpu(q, "q")
    mask = _HostMask(head_is_retrieval, block_table.shape[1])
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
    _check_tensor(q, "q", ndim=3)
    _check_cache16(q, k_pool, v_pool)
    num_blocks, block_size, head_dim = k_pool.shape
    total_q, num_q_heads, _ = q.shape
    _check_tensor(q_start, "q_start", dtype=_int32(), ndim=1, like=q)
    batch = q_start.shape[0] - 1
    if batch < 1:
        _fail("q_start must hold batch + 1 >= 2 offsets")
    _check_tables(block_table, seq_lens, batch, _kv_heads(block_table), q)
    _check_tensor(out, "out", shape=tuple(q.shape), like=q)
    _check_workspace(workspace, q, required=False)
    _check_gpu(q, "q")
    mask = _HostMask(head_is_retrieval, block_table.shape[1])
    st = lib().duo_attn_prefill_varlen(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), num_blocks, block_size,
        block_table.shape[2], _ptr(seq_lens), _ptr(q_start), batch, total_q, max_q_len,
        num_q_heads, block_table.shape[1], head_dim, _dtype_tag(q), mask.ptr, sink_size,
        recent_size, ring_blocks, softmax_scale, _ptr(out), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _check("duo_attn_prefill_varlen", st)


def duo_attn_prefill_varlen_workspace_size(batch: int, total_q: int, max_q_len: int,
                                           num_q_heads: int, num_kv_heads: int, head_dim: int,
                                           dtype: int, max_blocks_per_head: int, block_size: int,
                                           head_is_retrieval) -> int:
    mask = _HostMask(head_is_retrieval, num_kv_heads)
    return int(lib().duo_attn_prefill_varlen_workspace_size(
        batch, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, dtype,
        max_blocks_per_head, block_size, mask.ptr))


def prefill_varlen_workspace(q, block_table, head_is_retrieval, max_q_len: int, batch: int,
                             block_size: int):
    """Zero-filled workspace for duo_attn_prefill_varlen (q: [total_q][Hq][D]; block_table
    [batch][Hkv][max_blocks_per_head]; block_size of the cache)."""
    import torch
    total_q, num_q_heads, d = q.shape
    n = duo_attn_prefill_varlen_workspace_size(batch, total_q, max_q_len, num_q_heads,
                                               block_table.shape[1], d, _dtype_tag(q),
                                               block_table.shape[2], block_size, head_is_retrieval)
    if n == 0:
        raise ValueError("invalid sizes for the varlen prefill workspace")
    return torch.zeros(n, dtype=torch.uint8, device=q.device)


def _int8_pools(k_pool, v_pool, k_scale, v_scale):
    """int8 codes k [NB][bs][D], v [NB][D][bs] and float32 scales [NB][bs], on one device."""
    import torch
    _check_tensor(k_pool, "k_pool", dtype=torch.int8, ndim=3)
    nb, bs, d = k_pool.shape
    _check_tensor(v_pool, "v_pool", dtype=torch.int8, shape=(nb, d, bs), like=k_pool)
    _check_tensor(k_scale, "k_scale", dtype=torch.float32, shape=(nb, bs), like=k_pool)
    _check_tensor(v_scale, "v_scale", dtype=torch.float32, shape=(nb, bs), like=k_pool)


def kv_append_circular_int8(k_pool, v_pool, k_scale, v_scale, block_table, k_new, v_new,
                            seq_lens_before, seq_lens_after, head_is_retrieval, sink_size: int,
                            recent_size: int, ring_blocks: int, stream=None) -> None:
    """Quantize and append new rows into the int8 cache: k_pool int8 [NB][bs][D], v_pool int8
    [NB][D][bs], k_scale / v_scale float32 [NB][bs]; k_new / v_new [B][t_new][Hkv][D]."""
    _int8_pools(k_pool, v_pool, k_scale, v_scale)
    num_blocks, block_size, head_dim = k_pool.shape
    _check_tensor(k_new, "k_new", ndim=4)
    batch, t_new, num_kv_heads, _ = k_new.shape
    _check_tensor(k_new, "k_new", shape=(batch, t_new, num_kv_heads, head_dim))
    _check_tensor(v_new, "v_new", shape=tuple(k_new.shape), like=k_new)
    if k_new.device != k_pool.device:
        _fail(f"k_new is on {k_new.device}, the pools on {k_pool.device}")
    _check_tables(block_table, seq_lens_before, batch, num_kv_heads, k_pool, "seq_lens_before")
    if seq_lens_after is not None:
        _check_tensor(seq_lens_after, "seq_lens_after", dtype=_int32(), shape=(batch,), like=k_pool)
    _check_gpu(k_pool, "k_pool")
    mask = _HostMask(head_is_retrieval, num_kv_heads)
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
    _check_tensor(q, "q", shape=(None, None, head_dim))
    if q.device != k_pool.device:
        _fail(f"q is on {q.device}, the pools on {k_pool.device}")
    batch, num_q_heads, _ = q.shape
    _check_tables(block_table, seq_lens, batch, _kv_heads(block_table), q)
    _check_tensor(out, "out", shape=tuple(q.shape), like=q)
    _check_workspace(workspace, q)
    _check_gpu(q, "q")
    mask = _HostMask(head_is_retrieval, block_table.shape[1])
    st = lib().duo_attn_decode_int8(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        num_blocks, block_size, block_table.shape[2], _ptr(seq_lens), batch, num_q_heads,
        block_table.shape[1], head_dim, _dtype_tag(q), mask.ptr, sink_size, recent_size,
        ring_blocks, softmax_scale, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), split_tokens, _stream(stream))
    _check("duo_attn_decode_int8", st)


def duo_attn_append_decode_int8(q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_table,
                                seq_lens_before, seq_lens_after, head_is_retrieval, sink_size: int,
                                recent_size: int, ring_blocks: int, softmax_scale: float, out,
                                workspace, split_tokens: int = 0, stream=None) -> None:
    """kv_append_circular_int8 of one token per sequence (k_new, v_new [batch][1][kv heads][D] in
    q's dtype) and duo_attn_decode_int8 of its queries over seq_lens_before + 1 keys, in one
    launch."""
    _int8_pools(k_pool, v_pool, k_scale, v_scale)
    num_blocks, block_size, head_dim = k_pool.shape
    _check_tensor(q, "q", shape=(None, None, head_dim))
    if q.device != k_pool.device:
        _fail(f"q is on {q.device}, the pools on {k_pool.device}")
    batch, num_q_heads, _ = q.shape
    num_kv_heads = _kv_heads(block_table)
    _check_tables(block_table, seq_lens_before, batch, num_kv_heads, q, "seq_lens_before")
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _check_tensor(t, n, shape=(batch, 1, num_kv_heads, head_dim), like=q)
    if seq_lens_after is not None:
        _check_tensor(seq_lens_after, "seq_lens_after", dtype=_int32(), shape=(batch,), like=q)
    _check_tensor(out, "out", shape=tuple(q.shape), like=q)
    _check_workspace(workspace, q)
    _check_gpu(q, "q")
    mask = _HostMask(head_is_retrieval, num_kv_heads)
    st = lib().duo_attn_append_decode_int8(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
        _ptr(v_scale), _ptr(block_table), num_blocks, block_size, block_table.shape[2],
        _ptr(seq_lens_before), _ptr(seq_lens_after), batch, num_q_heads, num_kv_heads, head_dim,
        _dtype_tag(q), mask.ptr, sink_size, recent_size, ring_blocks, softmax_scale, _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), split_tokens,
        _stream(stream))
    _check("duo_attn_append_decode_int8", st)


def _int4_pools(k_pool, v_pool, k_scale, v_scale):
    """4-bit codes k uint8 [NB][bs][D/2], v uint8 [NB][D][bs/2]; float32 scales [Hkv][D]. Returns
    (num_blocks, block_size, head_dim)."""
    import torch
    _check_tensor(k_pool, "k_pool", dtype=torch.uint8, ndim=3)
    nb, bs, half_d = k_pool.shape
    d = 2 * int(half_d)
    _check_tensor(v_pool, "v_pool", dtype=torch.uint8, shape=(nb, d, bs // 2), like=k_pool)
    _check_tensor(k_scale, "k_scale", dtype=torch.float32, shape=(None, d), like=k_pool)
    _check_tensor(v_scale, "v_scale", dtype=torch.float32, shape=tuple(k_scale.shape), like=k_pool)
    return int(nb), int(bs), d


def kv_append_circular_int4(k_pool, v_pool, k_scale, v_scale, block_table, k_new, v_new,
                            seq_lens_before, seq_lens_after, head_is_retrieval, sink_size: int,
                            recent_size: int, ring_blocks: int, stream=None) -> None:
    """Quantize and append new rows into the 4-bit cache: k_pool uint8 [NB][bs][D/2], v_pool uint8
    [NB][D][bs/2], k_scale / v_scale float32 [Hkv][D] (per kv head and channel, read);
    k_new / v_new [B][t_new][Hkv][D] float16 or bfloat16."""
    num_blocks, block_size, head_dim = _int4_pools(k_pool, v_pool, k_scale, v_scale)
    _check_tensor(k_new, "k_new", ndim=4)
    batch, t_new, num_kv_heads, _ = k_new.shape
    _check_tensor(k_new, "k_new", shape=(batch, t_new, num_kv_heads, head_dim))
    _check_tensor(v_new, "v_new", shape=tuple(k_new.shape), like=k_new)
    if k_new.device != k_pool.device:
        _fail(f"k_new is on {k_new.device}, the pools on {k_pool.device}")
    if int(k_scale.shape[0]) != num_kv_heads:
        _fail(f"k_scale has {k_scale.shape[0]} kv heads, k_new {num_kv_heads}")
    _check_tables(block_table, seq_lens_before, batch, num_kv_heads, k_pool, "seq_lens_before")
    if seq_lens_after is not None:
        _check_tensor(seq_lens_after, "seq_lens_after", dtype=_int32(), shape=(batch,), like=k_pool)
    _check_gpu(k_pool, "k_pool")
    mask = _HostMask(head_is_retrieval, num_kv_heads)
    st = lib().kv_append_circular_int4(
        _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table), num_blocks,
        block_size, block_table.shape[2], _ptr(k_new), _ptr(v_new), _ptr(seq_lens_before),
        _ptr(seq_lens_after), batch, t_new, num_kv_heads, head_dim, _dtype_tag(k_new), mask.ptr,
        sink_size, recent_size, ring_blocks, _stream(stream))
    _check("kv_append_circular_int4", st)


def duo_attn_append_decode_int4(q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_table,
                                seq_lens_before, seq_lens_after, head_is_retrieval, sink_size: int,
                                recent_size: int, ring_blocks: int, softmax_scale: float, out,
                                workspace, split_tokens: int = 0, stream=None) -> None:
    """kv_append_circular_int4 of one token per sequence (k_new, v_new [batch][1][kv heads][D] in
    q's dtype) and duo_attn_decode_int4 of its queries over seq_lens_before + 1 keys, in one
    launch."""
    num_blocks, block_size, head_dim = _int4_pools(k_pool, v_pool, k_scale, v_scale)
    _check_tensor(q, "q", shape=(None, None, head_dim))
    if q.device != k_pool.device:
        _fail(f"q is on {q.device}, the pools on {k_pool.device}")
    batch, num_q_heads, _ = q.shape
    hkv = _kv_heads(block_table)
    if int(k_scale.shape[0]) != hkv:
        _fail(f"k_scale has {k_scale.shape[0]} kv heads, the block table {hkv}")
    _check_tables(block_table, seq_lens_before, batch, hkv, q, "seq_lens_before")
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _check_tensor(t, n, shape=(batch, 1, hkv, head_dim), like=q)
    if seq_lens_after is not None:
        _check_tensor(seq_lens_after, "seq_lens_after", dtype=_int32(), shape=(batch,), like=q)
    _check_tensor(out, "out", shape=tuple(q.shape), like=q)
    _check_workspace(workspace, q)
    _check_gpu(q, "q")
    mask = _HostMask(head_is_retrieval, hkv)
    st = lib().duo_attn_append_decode_int4(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
        _ptr(v_scale), _ptr(block_table), num_blocks, block_size, block_table.shape[2],
        _ptr(seq_lens_before), _ptr(seq_lens_after), batch, num_q_heads, hkv, head_dim,
        _dtype_tag(q), mask.ptr, sink_size, recent_size, ring_blocks, softmax_scale, _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), split_tokens,
        _stream(stream))
    _check("duo_attn_append_decode_int4", st)


def duo_attn_decode_int4(q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens,
                         head_is_retrieval, sink_size: int, recent_size: int, ring_blocks: int,
                         softmax_scale: float, out, workspace, split_tokens: int = 0,
                         stream=None) -> None:
    """duo_attn_decode over the 4-bit cache (pools and scales as for kv_append_circular_int4)."""
    num_blocks, block_size, head_dim = _int4_pools(k_pool, v_pool, k_scale, v_scale)
    _check_tensor(q, "q", shape=(None, None, head_dim))
    if q.device != k_pool.device:
        _fail(f"q is on {q.device}, the pools on {k_pool.device}")
    batch, num_q_heads, _ = q.shape
    hkv = _kv_heads(block_table)
    if int(k_scale.shape[0]) != hkv:
        _fail(f"k_scale has {k_scale.shape[0]} kv heads, the block table {hkv}")
    _check_tables(block_table, seq_lens, batch, hkv, q)
    _check_tensor(out, "out", shape=tuple(q.shape), like=q)
    _check_workspace(workspace, q)
    _check_gpu(q, "q")
    mask = _HostMask(head_is_retrieval, hkv)
    st = lib().duo_attn_decode_int4(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        num_blocks, block_size, block_table.shape[2], _ptr(seq_lens), batch, num_q_heads, hkv,
        head_dim, _dtype_tag(q), mask.ptr, sink_size, recent_size, ring_blocks, softmax_scale,
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), split_tokens,
        _stream(stream))
    _check("duo_attn_decode_int4", st)


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
    _check_tensor(q, "q", ndim=4)
    _check_cache16(q, k_pool, v_pool)
    num_blocks, block_size, head_dim = k_pool.shape
    batch, q_len, num_q_heads, _ = q.shape
    _check_tensor(q_succ, "q_succ", shape=tuple(q.shape), like=q)
    _check_tensor(q_inter, "q_inter", shape=tuple(q.shape), like=q)
    _check_tensor(mscale, "mscale", dtype=torch.float32, shape=(batch, q_len), like=q)
    _check_tables(block_table, seq_lens, batch, _kv_heads(block_table), q)
    _check_tensor(out, "out", shape=tuple(q.shape), like=q)
    _check_workspace(workspace, q, required=False)
    _check_gpu(q, "q")
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
    _check_tensor(q, "q", ndim=3)
    _check_cache16(q, k_pool, v_pool)
    num_blocks, block_size, head_dim = k_pool.shape
    batch, num_q_heads, _ = q.shape
    _check_tensor(q_succ, "q_succ", shape=tuple(q.shape), like=q)
    _check_tensor(q_inter, "q_inter", shape=tuple(q.shape), like=q)
    _check_tensor(mscale, "mscale", dtype=torch.float32, shape=(batch,), like=q)
    _check_tables(block_table, seq_lens, batch, _kv_heads(block_table), q)
    _check_tensor(out, "out", shape=tuple(q.shape), like=q)
    _check_workspace(workspace, q)
    _check_gpu(q, "q")
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


__all__ = ["kv_append_circular", "duo_attn_decode", "duo_attn_append_decode",
           "duo_attn_append_decode_int8", "duo_attn_append_decode_int4", "duo_attn_prefill",
           "duo_attn_decode_noalloc",
           "NOALLOC_SCRATCH_BYTES",
           "kv_append_circular_int8", "duo_attn_decode_int8", "duo_attn_prefill_varlen",
           "kv_append_circular_int4", "duo_attn_decode_int4", "prefill_varlen_workspace",
           "duo_attn_prefill_varlen_workspace_size", "dca_attn_prefill", "dca_attn_prefill_workspace_size", "dca_attn_decode",
           "profile_next_launch",
           "dca_prefill_workspace",
           "duo_attn_decode_workspace_size", "decode_workspace", "duo_attn_prefill_workspace_size",
           "prefill_workspace", "status_string", "abi_version",
           "DuoAttnError", "lib", "LIB_PATH", "SYMBOLS", "DUO_F32", "DUO_F16", "DUO_BF16"]
