"""duo_attn_append_decode and its int8 and 4-bit forms, through the C ABI: the fused append of one
token per sequence and the decode of its queries, against the two calls each stands for
(kv_append_circular[_int8|_int4], then duo_attn_decode[_int8|_int4] over seq_lens + 1) on twin
caches, and against the oracle.

Bars: pools bit-exact against the two calls (the token lands in the same slot with the same bits,
and nothing else changes); lengths after the call exact; outputs within the usual bound of the
fp64 oracle (1e-4 fp32, 2e-2 bf16/fp16) and of the two-call output. Pools start filled with NaN.
"""
import os

import numpy as np
import pytest
import torch

import kv_cache_sparsity_amd as duo
import oracle
import synth
from tests.gpu_harness import (Cache, check_close, logical_kv, oracle_decode, q_decode, say, to_dev,
                               to_host_bits, to_host_f64, TOL)
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


CASES = [
    # ring of 48 slots behind 4 sinks; the first token of a sequence (length 0) and ring wraps
    dict(name="bf16-d128-g4-mixed", dtype=synth.BF16, head_dim=128, group=4, kv=4, ret=(0, 2),
         block_size=16, sink=4, recent=40, ring_blocks=3, lens=[0, 15, 16, 47, 48, 300, 1000]),
    dict(name="f16-d256-g8-all-streaming", dtype=synth.F16, head_dim=256, group=8, kv=1, ret=(),
         block_size=16, sink=16, recent=100, ring_blocks=8, lens=[99, 700]),
    dict(name="f32-d64-g2-bs32", dtype=synth.F32, head_dim=64, group=2, kv=2, ret=(1,),
         block_size=32, sink=0, recent=33, ring_blocks=2, lens=[31, 32, 64, 65]),
    # a group of 20 q heads: two chunks of one kv head each write the token
    dict(name="bf16-d128-g20-chunks", dtype=synth.BF16, head_dim=128, group=20, kv=2, ret=(1,),
         block_size=16, sink=5, recent=64, ring_blocks=5, lens=[500, 63]),
    # block-granular window of two 16-position blocks
    dict(name="bf16-d128-block-window", dtype=synth.BF16, head_dim=128, group=4, kv=2, ret=(0,),
         block_size=16, sink=16, recent=-2, ring_blocks=2, lens=[16, 31, 32, 47, 100]),
]
STEPS = 3


def _setup(case, seed):
    lens = np.asarray(case["lens"])
    Lmax = int(lens.max()) + STEPS
    w = synth.small(case["name"], batch=len(lens), q_heads=case["kv"] * case["group"],
                    kv_heads=case["kv"], head_dim=case["head_dim"], dtype=case["dtype"],
                    block_size=case["block_size"], sink=case["sink"], recent=case["recent"],
                    retrieval=case["ret"], context=Lmax, ring_blocks=case["ring_blocks"],
                    seed=seed)
    K = logical_kv(w, Lmax, synth.S_K)
    V = logical_kv(w, Lmax, synth.S_V)
    fused, split = Cache(w, fill="nan"), Cache(w, fill="nan")
    _append_per_sequence(fused, K, V, lens)
    _append_per_sequence(split, K, V, lens)
    return w, K, V, lens, fused, split


def _same_bits(a, b, dtype):
    """Pools equal bit for bit (fp32 pools come back as floats: compare their bit patterns, so
    that the NaN of unwritten slots matches itself)."""
    x, y = to_host_bits(a, dtype), to_host_bits(b, dtype)
    if dtype == synth.F32:
        x, y = x.view(np.uint32), y.view(np.uint32)
    return np.array_equal(x, y)


def _token(w, X, lens):
    """[batch][1][kv heads][D] storage bits of position lens[b] of each sequence."""
    t = np.stack([X[b, :, int(lens[b])] for b in range(w.batch)])   # [B][Hkv][D]
    return to_dev(np.ascontiguousarray(t[:, None]), w.dtype)


@pytest.mark.parametrize("split_tokens", [0, 128])
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_append_decode_equals_append_then_decode(case, split_tokens):
    say(f"append+decode {case['name']} split {split_tokens}")
    w, K, V, lens, fused, split = _setup(case, 71)
    for step in range(STEPS):
        q = to_dev(q_decode(w, step), w.dtype)
        k_new, v_new = _token(w, K, lens), _token(w, V, lens)
        before = torch.from_numpy(lens.astype(np.int32)).cuda()
        # the fused call
        after_f = torch.full_like(before, -1)
        out_f = torch.empty_like(q)
        ws_f = duo.decode_workspace(q, fused.table, w.block_size, split_tokens)
        duo.duo_attn_append_decode(q, k_new, v_new, fused.k_pool, fused.v_pool, fused.table, before,
                                   after_f, fused.mask, w.sink, w.recent, w.ring_blocks, w.scale,
                                   out_f, ws_f, split_tokens)
        # the two calls
        after_s = torch.full_like(before, -1)
        out_s = torch.empty_like(q)
        duo.kv_append_circular(split.k_pool, split.v_pool, split.table, k_new, v_new, before,
                               after_s, split.mask, w.sink, w.recent, w.ring_blocks)
        ws_s = duo.decode_workspace(q, split.table, w.block_size, split_tokens)
        duo.duo_attn_decode(q, split.k_pool, split.v_pool, split.table, after_s, split.mask,
                            w.sink, w.recent, w.ring_blocks, w.scale, out_s, ws_s, split_tokens)
        torch.cuda.synchronize()
        lens = lens + 1
        assert (after_f.cpu().numpy() == lens).all(), after_f
        assert _same_bits(fused.k_pool, split.k_pool, w.dtype)
        assert _same_bits(fused.v_pool, split.v_pool, w.dtype)
        got = to_host_f64(out_f, w.dtype)
        want = oracle_decode(w, to_host_bits(q, w.dtype), K, V, lens, fused.mask)
        check_close(got, want, w.dtype, f"{case['name']} step {step}")
        assert float(np.abs(got - to_host_f64(out_s, w.dtype)).max()) <= TOL[w.dtype]


def test_append_decode_at_the_retrieval_capacity():
    """A retrieval row already full: the token is not written (as kv_append_circular), the decode
    attends over the row's capacity, and the new length still counts the token."""
    case = dict(name="bf16-capacity", dtype=synth.BF16, head_dim=128, group=4, kv=2, ret=(0,),
                block_size=16, sink=4, recent=40, ring_blocks=3, lens=[64, 63])
    say("append+decode at capacity")
    lens = np.asarray(case["lens"])
    w = synth.small(case["name"], batch=2, q_heads=8, kv_heads=2, head_dim=128, dtype=synth.BF16,
                    block_size=16, sink=4, recent=40, retrieval=(0,), context=64, ring_blocks=3,
                    capacity=64, seed=72)
    K = logical_kv(w, 65, synth.S_K)
    V = logical_kv(w, 65, synth.S_V)
    fused, split = Cache(w, fill="nan"), Cache(w, fill="nan")
    _append_per_sequence(fused, K, V, lens)
    _append_per_sequence(split, K, V, lens)
    q = to_dev(q_decode(w, 0), w.dtype)
    k_new, v_new = _token(w, K, lens), _token(w, V, lens)
    before = torch.from_numpy(lens.astype(np.int32)).cuda()
    after_f, after_s = torch.full_like(before, -1), torch.full_like(before, -1)
    out_f, out_s = torch.empty_like(q), torch.empty_like(q)
    duo.duo_attn_append_decode(q, k_new, v_new, fused.k_pool, fused.v_pool, fused.table, before,
                               after_f, fused.mask, w.sink, w.recent, w.ring_blocks, w.scale,
                               out_f, duo.decode_workspace(q, fused.table, w.block_size))
    duo.kv_append_circular(split.k_pool, split.v_pool, split.table, k_new, v_new, before, after_s,
                           split.mask, w.sink, w.recent, w.ring_blocks)
    duo.duo_attn_decode(q, split.k_pool, split.v_pool, split.table, after_s, split.mask, w.sink,
                        w.recent, w.ring_blocks, w.scale, out_s,
                        duo.decode_workspace(q, split.table, w.block_size))
    torch.cuda.synchronize()
    assert (after_f.cpu().numpy() == lens + 1).all()
    assert _same_bits(fused.k_pool, split.k_pool, w.dtype)
    assert _same_bits(fused.v_pool, split.v_pool, w.dtype)
    got, ref = to_host_f64(out_f, w.dtype), to_host_f64(out_s, w.dtype)
    assert np.isfinite(got).all()
    assert float(np.abs(got - ref).max()) <= TOL[w.dtype]


INT8_CASES = [
    dict(name="int8-bf16-d128-g4-mixed", dtype=synth.BF16, head_dim=128, group=4, kv=4, ret=(0, 2),
         block_size=16, sink=4, recent=40, ring_blocks=3, lens=[0, 15, 47, 300, 1000]),
    dict(name="int8-f16-d256-g8", dtype=synth.F16, head_dim=256, group=8, kv=1, ret=(0,),
         block_size=16, sink=16, recent=100, ring_blocks=8, lens=[99, 700]),
    dict(name="int8-f32-d64-bs32", dtype=synth.F32, head_dim=64, group=2, kv=2, ret=(1,),
         block_size=32, sink=0, recent=33, ring_blocks=2, lens=[31, 64, 65]),
]


@pytest.mark.parametrize("split_tokens", [0, 128])
@pytest.mark.parametrize("case", INT8_CASES, ids=[c["name"] for c in INT8_CASES])
def test_append_decode_int8_equals_append_then_decode(case, split_tokens):
    say(f"append+decode int8 {case['name']} split {split_tokens}")
    lens = np.asarray(case["lens"])
    Lmax = int(lens.max()) + STEPS
    w = synth.small(case["name"], batch=len(lens), q_heads=case["kv"] * case["group"],
                    kv_heads=case["kv"], head_dim=case["head_dim"], dtype=case["dtype"],
                    block_size=case["block_size"], sink=case["sink"], recent=case["recent"],
                    retrieval=case["ret"], context=Lmax, ring_blocks=case["ring_blocks"], seed=73)
    K = logical_kv(w, Lmax, synth.S_K)
    V = logical_kv(w, Lmax, synth.S_V)
    kc, ks, vc, vs = _logical_codes(K, V, w.dtype)
    fused, split = Int8Cache(w), Int8Cache(w)
    fused.fill_per_sequence(K, V, lens)
    split.fill_per_sequence(K, V, lens)
    for step in range(STEPS):
        q_bits = q_decode(w, step)
        q = to_dev(q_bits, w.dtype)
        k_new, v_new = _token(w, K, lens), _token(w, V, lens)
        before = torch.from_numpy(lens.astype(np.int32)).cuda()
        after_f, after_s = torch.full_like(before, -1), torch.full_like(before, -1)
        out_f, out_s = torch.empty_like(q), torch.empty_like(q)
        duo.duo_attn_append_decode_int8(
            q, k_new, v_new, fused.k_pool, fused.v_pool, fused.k_scale, fused.v_scale, fused.table,
            before, after_f, fused.mask, w.sink, w.recent, w.ring_blocks, w.scale, out_f,
            duo.decode_workspace(q, fused.table, w.block_size, split_tokens), split_tokens)
        duo.kv_append_circular_int8(split.k_pool, split.v_pool, split.k_scale, split.v_scale,
                                    split.table, k_new, v_new, before, after_s, split.mask, w.sink,
                                    w.recent, w.ring_blocks)
        duo.duo_attn_decode_int8(q, split.k_pool, split.v_pool, split.k_scale, split.v_scale,
                                 split.table, after_s, split.mask, w.sink, w.recent, w.ring_blocks,
                                 w.scale, out_s,
                                 duo.decode_workspace(q, split.table, w.block_size, split_tokens),
                                 split_tokens)
        torch.cuda.synchronize()
        lens = lens + 1
        assert (after_f.cpu().numpy() == lens).all(), after_f
        assert torch.equal(fused.k_pool, split.k_pool) and torch.equal(fused.v_pool, split.v_pool)
        for a, b in ((fused.k_scale, split.k_scale), (fused.v_scale, split.v_scale)):
            assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))
        got = to_host_f64(out_f, w.dtype)
        want = oracle.attend_int8(q_bits[:, None], kc, ks, vc, vs, lens, fused.mask, sink=w.sink,
                                  recent=w.recent, scale=w.scale, dtype=w.dtype,
                                  block_size=w.block_size)[:, 0]
        check_close(got, want, w.dtype, f"{case['name']} step {step}")
        assert float(np.abs(got - to_host_f64(out_s, w.dtype)).max()) <= TOL[w.dtype]


INT4_CASES = [
    dict(name="int4-bf16-d128-g4-mixed", dtype=synth.BF16, head_dim=128, group=4, kv=4, ret=(0, 2),
         block_size=16, sink=4, recent=40, ring_blocks=3, lens=[0, 15, 47, 300, 1000]),
    dict(name="int4-f16-d256-g8", dtype=synth.F16, head_dim=256, group=8, kv=1, ret=(0,),
         block_size=16, sink=16, recent=100, ring_blocks=8, lens=[99, 700]),
    dict(name="int4-bf16-d64-bs64", dtype=synth.BF16, head_dim=64, group=2, kv=2, ret=(1,),
         block_size=64, sink=9, recent=70, ring_blocks=2, lens=[8, 63, 64, 65, 500]),
]


@pytest.mark.parametrize("split_tokens", [0, 128])
@pytest.mark.parametrize("case", INT4_CASES, ids=[c["name"] for c in INT4_CASES])
def test_append_decode_int4_equals_append_then_decode(case, split_tokens):
    say(f"append+decode 4-bit {case['name']} split {split_tokens}")
    lens = np.asarray(case["lens"])
    Lmax = int(lens.max()) + STEPS
    w = synth.small(case["name"], batch=len(lens), q_heads=case["kv"] * case["group"],
                    kv_heads=case["kv"], head_dim=case["head_dim"], dtype=case["dtype"],
                    block_size=case["block_size"], sink=case["sink"], recent=case["recent"],
                    retrieval=case["ret"], context=Lmax, ring_blocks=case["ring_blocks"], seed=74)
    K = logical_kv(w, Lmax, synth.S_K)
    V = logical_kv(w, Lmax, synth.S_V)
    fused, split = Int4Cache(w), Int4Cache(w)
    kc, vc = fused.logical_codes(K, V)
    fused.fill_per_sequence(K, V, lens)
    split.fill_per_sequence(K, V, lens)
    for step in range(STEPS):
        q_bits = q_decode(w, step)
        q = to_dev(q_bits, w.dtype)
        k_new, v_new = _token(w, K, lens), _token(w, V, lens)
        before = torch.from_numpy(lens.astype(np.int32)).cuda()
        after_f, after_s = torch.full_like(before, -1), torch.full_like(before, -1)
        out_f, out_s = torch.empty_like(q), torch.empty_like(q)
        duo.duo_attn_append_decode_int4(
            q, k_new, v_new, fused.k_pool, fused.v_pool, fused.k_scale, fused.v_scale, fused.table,
            before, after_f, fused.mask, w.sink, w.recent, w.ring_blocks, w.scale, out_f,
            duo.decode_workspace(q, fused.table, w.block_size, split_tokens), split_tokens)
        duo.kv_append_circular_int4(split.k_pool, split.v_pool, split.k_scale, split.v_scale,
                                    split.table, k_new, v_new, before, after_s, split.mask, w.sink,
                                    w.recent, w.ring_blocks)
        duo.duo_attn_decode_int4(q, split.k_pool, split.v_pool, split.k_scale, split.v_scale,
                                 split.table, after_s, split.mask, w.sink, w.recent, w.ring_blocks,
                                 w.scale, out_s,
                                 duo.decode_workspace(q, split.table, w.block_size, split_tokens),
                                 split_tokens)
        torch.cuda.synchronize()
        lens = lens + 1
        assert (after_f.cpu().numpy() == lens).all(), after_f
        assert torch.equal(fused.k_pool, split.k_pool) and torch.equal(fused.v_pool, split.v_pool)
        got = to_host_f64(out_f, w.dtype)
        want = oracle.attend_int4(q_bits[:, None], kc, vc, fused.ks_h, fused.vs_h, lens, fused.mask,
                                  sink=w.sink, recent=w.recent, scale=w.scale, dtype=w.dtype,
                                  block_size=w.block_size)[:, 0]
        check_close(got, want, w.dtype, f"{case['name']} step {step}")
        assert float(np.abs(got - to_host_f64(out_s, w.dtype)).max()) <= TOL[w.dtype]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("bits", [16, 8, 4])
def test_llama3_8b_append_decode_batch8_ctx32768(bits):
    """The fused call at the full Llama-3-8B decode shape (batch 8, 32768 tokens, 32 q heads over 8
    kv heads, half of them retrieval), in the launch configuration the benchmark times: the cache
    holds 32767 tokens, the call appends the 32768th and attends over all of them. Pools against
    the standalone append on a copy of the same pools, bit for bit; outputs against the oracle."""
    w = synth.llama3_8b_decode()
    say(f"workload {w.name}, append+decode, {bits}-bit cache" if bits < 16
        else f"workload {w.name}, append+decode")
    L = w.context
    K = logical_kv(w, L, synth.S_K)
    V = logical_kv(w, L, synth.S_V)
    lens = np.full(w.batch, L - 1)
    if bits == 16:
        cache = Cache(w, fill="nan")
        cache.append_logical(K, V, 0, L - 1, chunk=8192)
    else:
        cache = Int8Cache(w) if bits == 8 else Int4Cache(w)
        cache.fill_per_sequence(K, V, lens)
    scales = [] if bits == 16 else [cache.k_scale, cache.v_scale]
    twin = [t.clone() for t in [cache.k_pool, cache.v_pool] + scales]
    q_bits = q_decode(w, 0)
    q = to_dev(q_bits, w.dtype)
    k_new, v_new = _token(w, K, lens), _token(w, V, lens)
    before = torch.from_numpy(lens.astype(np.int32)).cuda()
    after_f, after_s = torch.full_like(before, -1), torch.full_like(before, -1)
    out_f, out_s = torch.empty_like(q), torch.empty_like(q)
    ws = duo.decode_workspace(q, cache.table, w.block_size)
    common = (w.sink, w.recent, w.ring_blocks)
    if bits == 16:
        duo.duo_attn_append_decode(q, k_new, v_new, cache.k_pool, cache.v_pool, cache.table, before,
                                   after_f, cache.mask, *common, w.scale, out_f, ws)
        duo.kv_append_circular(*twin, cache.table, k_new, v_new, before, after_s, cache.mask,
                               *common)
        torch.cuda.synchronize()
        duo.duo_attn_decode(q, *twin, cache.table, after_s, cache.mask, *common, w.scale, out_s, ws)
    else:
        fused = duo.duo_attn_append_decode_int8 if bits == 8 else duo.duo_attn_append_decode_int4
        append = duo.kv_append_circular_int8 if bits == 8 else duo.kv_append_circular_int4
        decode = duo.duo_attn_decode_int8 if bits == 8 else duo.duo_attn_decode_int4
        fused(q, k_new, v_new, cache.k_pool, cache.v_pool, cache.k_scale, cache.v_scale,
              cache.table, before, after_f, cache.mask, *common, w.scale, out_f, ws)
        append(*twin, cache.table, k_new, v_new, before, after_s, cache.mask, *common)
        torch.cuda.synchronize()
        decode(q, *twin, cache.table, after_s, cache.mask, *common, w.scale, out_s, ws)
    torch.cuda.synchronize()
    assert (after_f.cpu().numpy() == L).all() and (after_s.cpu().numpy() == L).all()
    for a, b in zip([cache.k_pool, cache.v_pool] + scales, twin):
        if a.dtype == torch.float32:
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        else:
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    got = to_host_f64(out_f, w.dtype)
    full = np.full(w.batch, L)
    if bits == 16:
        want = oracle_decode(w, q_bits, K, V, full, cache.mask)
    elif bits == 8:
        kc, ks, vc, vs = _logical_codes(K, V, w.dtype)
        want = oracle.attend_int8(q_bits[:, None], kc, ks, vc, vs, full, cache.mask, sink=w.sink,
                                  recent=w.recent, scale=w.scale, dtype=w.dtype)[:, 0]
    else:
        kc, vc = cache.logical_codes(K, V)
        want = oracle.attend_int4(q_bits[:, None], kc, vc, cache.ks_h, cache.vs_h, full,
                                  cache.mask, sink=w.sink, recent=w.recent, scale=w.scale,
                                  dtype=w.dtype)[:, 0]
    check_close(got, want, w.dtype, f"{w.name} append+decode {bits}-bit")
    assert float(np.abs(got - to_host_f64(out_s, w.dtype)).max()) <= TOL[w.dtype]


LONG_CASE = dict(name="bf16-d128-g4-long-splits", dtype=synth.BF16, head_dim=128, group=4, kv=2,
                 ret=(0,), block_size=16, sink=4, recent=40, ring_blocks=3,
                 lens=[9000, 20000, 8191, 8192, 16383])


@pytest.mark.parametrize("bits", [16, 4])
def test_append_decode_with_splits_past_one_run_segment(bits):
    """Splits of 16384 keys: a token more than 512 runs (8192 keys) into its split takes its page
    from the block table after the length, the others from the entries the split read before it
    (both kinds here, and tokens at the first and last run of a segment)."""
    if bits == 16:
        test_append_decode_equals_append_then_decode(LONG_CASE, 16384)
    else:
        test_append_decode_int4_equals_append_then_decode(dict(LONG_CASE, name="int4-long-splits"),
                                                          16384)
