"""Helpers for the GPU parity tests: move seeded storage bits to and from the device, drive the
library through its C ABI (via the binding), and compute the oracle on the same bits."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import kv_cache_sparsity_amd as duo
import oracle
import synth

TOL = {synth.F32: 1e-4, synth.F16: 2e-2, synth.BF16: 2e-2}
TORCH_DT = {synth.F32: torch.float32, synth.F16: torch.float16, synth.BF16: torch.bfloat16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, dtype: int, device="cuda") -> torch.Tensor:
    """Storage bits (float32, or uint16 bit patterns) -> device tensor of the dtype."""
    if dtype == synth.F32:
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16))
    return t.to(device).view(TORCH_DT[dtype])


def to_host_bits(t: torch.Tensor, dtype: int) -> np.ndarray:
    if dtype == synth.F32:
        return t.detach().cpu().numpy()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_host_f64(t: torch.Tensor, dtype: int) -> np.ndarray:
    return oracle.to_f64(to_host_bits(t, dtype), dtype)


def fill_bits(dtype: int, kind: str):
    """A fill value for pools: 'nan' (quiet NaN bits) or 'sentinel' (a distinctive finite value)."""
    if dtype == synth.F32:
        return np.float32(np.nan) if kind == "nan" else np.float32(-12345.0)
    if kind == "nan":
        return np.uint16(0x7FC0 if dtype == synth.BF16 else 0x7E00)
    return np.uint16(0xC640 if dtype == synth.BF16 else 0xF208)


def logical_kv(w: synth.Workload, L: int, which: int) -> np.ndarray:
    """Context K or V as storage bits, logical layout [B][Hkv][L][D]."""
    out = np.empty((w.batch, w.num_kv_heads, L, w.head_dim), dtype=synth.storage_np_dtype(w.dtype))
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            out[b, h] = synth.f32_to_storage(synth.kv_tokens(w, which, b, h, 0, L), w.dtype)
    return out


class Cache:
    """Device pools + block table + lengths for one workload, filled through kv_append_circular."""

    def __init__(self, w: synth.Workload, fill: str = "nan", identity: bool = False,
                 mask=None, share_sinks: bool = False):
        self.w = w
        self.mask = np.asarray(mask if mask is not None else w.retrieval_mask, dtype=np.uint8)
        self.table_h, self.num_blocks = synth.block_table(w, identity=identity,
                                                          share_sinks=share_sinks)
        self.table = torch.from_numpy(self.table_h).cuda()
        ks, vs = oracle.pool_shapes(self.num_blocks, w.block_size, w.head_dim)
        fv = fill_bits(w.dtype, fill)
        self.k_pool = to_dev(np.full(ks, fv), w.dtype)
        self.v_pool = to_dev(np.full(vs, fv), w.dtype)
        self.fill_value = fv
        self.lens = torch.zeros(w.batch, dtype=torch.int32, device="cuda")

    def append(self, k_new_bits: np.ndarray, v_new_bits: np.ndarray, lens_before=None):
        """k_new_bits, v_new_bits: storage [B][T][Hkv][D]."""
        w = self.w
        before = self.lens if lens_before is None else torch.as_tensor(
            np.asarray(lens_before, np.int32)).cuda()
        after = torch.empty_like(before)
        duo.kv_append_circular(self.k_pool, self.v_pool, self.table, to_dev(k_new_bits, w.dtype),
                               to_dev(v_new_bits, w.dtype), before, after, self.mask, w.sink,
                               w.recent, w.ring_blocks)
        self.lens = after

    def append_logical(self, K: np.ndarray, V: np.ndarray, start: int, stop: int, chunk=65536):
        """Append positions [start, stop) of logical storage arrays [B][Hkv][L][D], chunked."""
        for s in range(start, stop, chunk):
            e = min(stop, s + chunk)
            kn = np.ascontiguousarray(K[:, :, s:e].transpose(0, 2, 1, 3))
            vn = np.ascontiguousarray(V[:, :, s:e].transpose(0, 2, 1, 3))
            self.append(kn, vn)

    def set_lens(self, lens):
        self.lens = torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda()

    def decode(self, q_bits: np.ndarray, split_tokens: int = 0, workspace=None):
        w = self.w
        q = to_dev(q_bits, w.dtype)
        out = torch.empty_like(q)
        ws = workspace if workspace is not None else duo.decode_workspace(
            q, self.table, w.block_size, split_tokens)
        duo.duo_attn_decode(q, self.k_pool, self.v_pool, self.table, self.lens, self.mask, w.sink,
                            w.recent, w.ring_blocks, w.scale, out, ws, split_tokens)
        return out

    def prefill(self, q_bits: np.ndarray, workspace=None):
        w = self.w
        q = to_dev(q_bits, w.dtype)
        out = torch.empty_like(q)
        ws = workspace if workspace is not None else duo.prefill_workspace(q, self.table, self.mask)
        duo.duo_attn_prefill(q, self.k_pool, self.v_pool, self.table, self.lens, self.mask, w.sink,
                             w.recent, w.ring_blocks, w.scale, out, ws)
        return out


def check_close(got_f64: np.ndarray, want_f64: np.ndarray, dtype: int, what: str):
    assert got_f64.shape == want_f64.shape, (got_f64.shape, want_f64.shape)
    assert np.isfinite(got_f64).all(), f"{what}: non-finite output"
    err = float(np.max(np.abs(got_f64 - want_f64))) if got_f64.size else 0.0
    say(f"  {what}: max |gpu - oracle| = {err:.3e} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype], f"{what}: max abs err {err} > {TOL[dtype]}"
    return err


def q_decode(w: synth.Workload, step: int) -> np.ndarray:
    """Decode queries [B][Hq][D] as storage bits."""
    return synth.f32_to_storage(synth.queries(w, step, q_len=1)[:, 0], w.dtype)


def q_prefill(w: synth.Workload, step: int, q_len: int) -> np.ndarray:
    return synth.f32_to_storage(synth.queries(w, step, q_len=q_len), w.dtype)


def oracle_decode(w, q_bits, K, V, lens, mask, rows=None):
    """Oracle for decode queries [B][Hq][D] over logical storage K, V."""
    q4 = q_bits[:, None]
    o = oracle.attend(q4, K, V, lens, mask, sink=w.sink, recent=w.recent, scale=w.scale,
                      dtype=w.dtype, rows=None if rows is None else [(b, 0, hq) for b, hq in rows],
                      block_size=w.block_size)
    return o[:, 0]
