"""GPU parity of the block-granular streaming window (recent_size < 0) against the oracle.

A streaming head then keeps its sink and the -recent_size newest blocks up to the query's own (vLLM
issue "Could you support Attention Sink?", ChuanhongLi's comment: keep the first block, drop middle
blocks, keep the recent blocks). The lengths below put queries on, just before and just after block
boundaries, where the window jumps by a block; rings are sized to the window's span exactly, so
the oldest kept block shares its slots with the newest positions.

Bars as in the other parity tests: max abs error 1e-4 (fp32) or 2e-2 (bf16/fp16) against the fp64
oracle; pools start filled with NaN.
"""
import os

import numpy as np
import pytest
import torch

import kv_cache_sparsity_amd as duo
import oracle
import synth
from tests.gpu_harness import (Cache, check_close, logical_kv, q_decode, q_prefill, say, to_dev,
                               to_host_f64)
from tests.test_gpu_int4 import Int4Cache
from tests.test_gpu_int8 import Int8Cache, _logical_codes
from tests.test_gpu_parity import _append_per_sequence

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(duo.LIB_PATH):
        pytest.fail("libduoattn.so is not built; the GPU tests need the HIP library")


def _workload(case, context, q_len, seed):
    return synth.small(case["name"], batch=case.get("batch", len(case.get("lens", [0, 0]))),
                       q_heads=case["kv"] * case["group"], kv_heads=case["kv"],
                       head_dim=case["head_dim"], dtype=case["dtype"],
                       block_size=case["block_size"], sink=case["sink"], recent=-case["blocks"],
                       retrieval=case["ret"], context=context, q_len=q_len, seed=seed)


DECODE_CASES = [
    dict(name="bf16-d128-bs16-sink16-k2", dtype=synth.BF16, head_dim=128, group=4, kv=2, ret=(0,),
         block_size=16, sink=16, blocks=2, lens=[1, 16, 17, 32, 33, 48, 49, 700]),
    dict(name="f16-d256-bs16-sink16-k3-streaming", dtype=synth.F16, head_dim=256, group=8, kv=1,
         ret=(), block_size=16, sink=16, blocks=3, lens=[47, 48, 49, 1000]),
    dict(name="f32-d64-bs32-sink0-k1", dtype=synth.F32, head_dim=64, group=2, kv=2, ret=(1,),
         block_size=32, sink=0, blocks=1, lens=[31, 32, 33, 64, 65, 999]),
    dict(name="bf16-d128-bs256-sink256-k2", dtype=synth.BF16, head_dim=128, group=2, kv=2,
         ret=(1,), block_size=256, sink=256, blocks=2, lens=[255, 256, 257, 512, 513, 3000]),
    dict(name="bf16-d128-g20-bs16-sink5-k4", dtype=synth.BF16, head_dim=128, group=20, kv=2,
         ret=(1,), block_size=16, sink=5, blocks=4, lens=[0, 60, 63, 64, 65, 900]),
]


def _oracle_decode(w, q, K, V, lens, mask):
    return oracle.attend(q[:, None], K, V, lens, mask, sink=w.sink, recent=w.recent, scale=w.scale,
                         dtype=w.dtype, block_size=w.block_size)[:, 0]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c["name"] for c in DECODE_CASES])
def test_decode_block_window(case):
    say(f"decode block window {case['name']}")
    lens = np.asarray(case["lens"])
    Lmax = int(lens.max())
    w = _workload(case, Lmax, 1, 61)
    assert w.ring_blocks == case["blocks"]      # the ring holds exactly the window's span
    cache = Cache(w, fill="nan")
    K = logical_kv(w, Lmax, synth.S_K)
    V = logical_kv(w, Lmax, synth.S_V)
    _append_per_sequence(cache, K, V, lens)
    q = q_decode(w, 0)
    want = _oracle_decode(w, q, K, V, lens, cache.mask)
    for split in ((0, 128) if case["ret"] else (0,)):
        got = to_host_f64(cache.decode(q, split_tokens=split), w.dtype)
        check_close(got, want, w.dtype, f"{case['name']} split {split}")
        for b in np.flatnonzero(lens == 0):
            assert (got[b] == 0).all()


QUANT_CASE = dict(name="bf16-d128-bs16-sink16-k2-quant", dtype=synth.BF16, head_dim=128, group=4,
                  kv=2, ret=(1,), block_size=16, sink=16, blocks=2, lens=[33, 48, 49, 700])


def test_decode_int8_block_window():
    say("decode int8 block window")
    lens = np.asarray(QUANT_CASE["lens"])
    Lmax = int(lens.max())
    w = _workload(QUANT_CASE, Lmax, 1, 62)
    cache = Int8Cache(w)
    K = logical_kv(w, Lmax, synth.S_K)
    V = logical_kv(w, Lmax, synth.S_V)
    cache.fill_per_sequence(K, V, lens)
    kc, ks, vc, vs = _logical_codes(K, V, w.dtype)
    q = q_decode(w, 0)
    want = oracle.attend_int8(q[:, None], kc, ks, vc, vs, lens, cache.mask, sink=w.sink,
                              recent=w.recent, scale=w.scale, dtype=w.dtype,
                              block_size=w.block_size)[:, 0]
    got = to_host_f64(cache.decode(q), w.dtype)
    check_close(got, want, w.dtype, "int8 block window")


def test_decode_int4_block_window():
    say("decode int4 block window")
    lens = np.asarray(QUANT_CASE["lens"])
    Lmax = int(lens.max())
    w = _workload(QUANT_CASE, Lmax, 1, 63)
    cache = Int4Cache(w)
    K = logical_kv(w, Lmax, synth.S_K)
    V = logical_kv(w, Lmax, synth.S_V)
    cache.fill_per_sequence(K, V, lens)
    kc, vc = cache.logical_codes(K, V)
    q = q_decode(w, 0)
    want = oracle.attend_int4(q[:, None], kc, vc, cache.ks_h, cache.vs_h, lens, cache.mask,
                              sink=w.sink, recent=w.recent, scale=w.scale, dtype=w.dtype,
                              block_size=w.block_size)[:, 0]
    got = to_host_f64(cache.decode(q), w.dtype)
    check_close(got, want, w.dtype, "int4 block window")


PREFILL_CASES = [
    dict(name="bf16-d128-bs16-sink16-k3", dtype=synth.BF16, head_dim=128, group=1, kv=2, ret=(1,),
         block_size=16, sink=16, blocks=3, chunks=[100, 37, 300]),
    dict(name="f16-d256-bs16-sink16-k2", dtype=synth.F16, head_dim=256, group=2, kv=1, ret=(),
         block_size=16, sink=16, blocks=2, chunks=[64, 64, 130]),
    dict(name="f32-d64-bs32-sink0-k1", dtype=synth.F32, head_dim=64, group=1, kv=2, ret=(0,),
         block_size=32, sink=0, blocks=1, chunks=[33, 1, 128]),
    dict(name="bf16-d64-bs64-sink64-k2", dtype=synth.BF16, head_dim=64, group=2, kv=2, ret=(0,),
         block_size=64, sink=64, blocks=2, chunks=[333, 333]),
    dict(name="bf16-d128-bs256-sink0-k2", dtype=synth.BF16, head_dim=128, group=1, kv=2, ret=(1,),
         block_size=256, sink=0, blocks=2, chunks=[700]),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c["name"] for c in PREFILL_CASES])
def test_prefill_block_window(case):
    say(f"prefill block window {case['name']}")
    chunks = case["chunks"]
    total = sum(chunks)
    w = _workload(dict(case, batch=2), total, max(chunks), 64)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, total, synth.S_K)
    V = logical_kv(w, total, synth.S_V)
    pos = 0
    for ci, n in enumerate(chunks):
        cache.append_logical(K, V, pos, pos + n)
        pos += n
        q = q_prefill(w, ci, n)
        got = to_host_f64(cache.prefill(q), w.dtype)
        want = oracle.attend(q, K, V, np.full(w.batch, pos), cache.mask, sink=w.sink,
                             recent=w.recent, scale=w.scale, dtype=w.dtype,
                             block_size=w.block_size)
        check_close(got, want, w.dtype, f"{case['name']} chunk {ci}")


def test_prefill_varlen_block_window_with_single_rows():
    """A packed batch whose single rows run as split-K decode items in the same launch."""
    case = dict(name="bf16-d128-gqa2-bs16-k2-varlen", dtype=synth.BF16, head_dim=128, group=2,
                kv=2, ret=(0,), block_size=16, sink=16, blocks=2, batch=4)
    rows, lens = [300, 1, 0, 37], np.asarray([700, 513, 100, 37])
    B, max_q = len(rows), max(rows)
    say(f"prefill varlen block window {case['name']}")
    w = _workload(case, int(lens.max()), max_q, 65)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, int(lens.max()), synth.S_K)
    V = logical_kv(w, int(lens.max()), synth.S_V)
    _append_per_sequence(cache, K, V, lens)
    qs = [q_prefill(w, b, n)[b:b + 1] for b, n in enumerate(rows)]
    packed = np.concatenate([q[0] for q in qs], axis=0)
    q_start = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    qd = to_dev(packed, w.dtype)
    out = torch.full_like(qd, float("nan"))
    ws = duo.prefill_varlen_workspace(qd, cache.table, cache.mask, max_q, B, w.block_size)
    duo.duo_attn_prefill_varlen(qd, cache.k_pool, cache.v_pool, cache.table, cache.lens,
                                torch.from_numpy(q_start).cuda(), max_q, cache.mask, w.sink,
                                w.recent, w.ring_blocks, w.scale, out, ws)
    got = to_host_f64(out, w.dtype)
    for b, n in enumerate(rows):
        if n == 0:
            continue
        want = oracle.attend(qs[b], K[b:b + 1], V[b:b + 1], lens[b:b + 1], cache.mask,
                             sink=w.sink, recent=w.recent, scale=w.scale, dtype=w.dtype,
                             block_size=w.block_size)[0]
        check_close(got[q_start[b]:q_start[b + 1]], want, w.dtype, f"varlen sequence {b}")


def test_block_window_differs_from_the_token_window():
    """The same cache read with k blocks and with k * block_size tokens: queries in the middle of a
    block see fewer keys under the block window, so the outputs must differ there (the library
    really applies the block rule, not a token window of the same span)."""
    case = DECODE_CASES[0]
    # queries at 50 and 51, inside block 3: the two blocks 2, 3 start at 32, the 32-token window
    # at 19 and 20 (sink 16 in both)
    lens = np.asarray([51, 52])
    w = _workload(dict(case, lens=list(lens)), 52, 1, 66)
    cache = Cache(w, fill="nan", mask=np.zeros(w.num_kv_heads, np.uint8))
    K = logical_kv(w, 52, synth.S_K)
    V = logical_kv(w, 52, synth.S_V)
    _append_per_sequence(cache, K, V, lens)
    q = to_dev(q_decode(w, 0), w.dtype)
    outs = []
    for recent in (w.recent, -w.recent * w.block_size):
        out = torch.empty_like(q)
        ws = duo.decode_workspace(q, cache.table, w.block_size, 0)
        duo.duo_attn_decode(q, cache.k_pool, cache.v_pool, cache.table, cache.lens, cache.mask,
                            w.sink, recent, w.ring_blocks, w.scale, out, ws, 0)
        outs.append(to_host_f64(out, w.dtype))
    assert np.abs(outs[0] - outs[1]).max() > 1e-2
