"""GPU parity on seeded random shapes: decode (GQA groups up to 64), prefill, the int8 and 4-bit
decodes and Dual Chunk Attention against the CPU oracle.

Each case draws a dtype, head dim, kv-head count, GQA group, page size, sink and recent sizes, a
retrieval mask, per-sequence lengths and (for prefill) a chunk length, all within the documented
limits of the calls, fills the cache one sequence at a time through kv_append_circular and compares
every output row with the oracle. Bars as everywhere: 1e-4 (fp32), 2e-2 (fp16 / bf16).
"""
import os

import numpy as np
import pytest
import torch

import kv_cache_sparsity_amd as duo
import oracle
import synth
from tests.gpu_harness import (Cache, check_close, logical_kv, oracle_decode, q_decode, q_prefill,
                               say, to_dev, to_host_f64)

N_CASES = 96


@pytest.fixture(scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(duo.LIB_PATH):
        pytest.fail("libduoattn.so is not built; the GPU tests need the HIP library")


def draw_case(i: int) -> dict:
    """The i-th seeded case (host-only; also usable without a GPU)."""
    rng = np.random.default_rng([2024, i])
    dtype = (synth.F32, synth.F16, synth.BF16)[rng.integers(3)]
    D = (64, 128, 256)[rng.integers(3)]
    if dtype == synth.F32 and D == 256:
        D = 128                                  # fp32 prefill is limited to D <= 128
    kv = int(rng.integers(1, 4))
    return dict(dtype=dtype, D=D, kv=kv, G=(1, 2, 4, 8)[rng.integers(4)],
                bs=(16, 32, 64)[rng.integers(3)], sink=int(rng.integers(0, 40)),
                recent=int(rng.integers(1, 200)),
                ret=tuple(h for h in range(kv) if rng.random() < 0.5),
                lens=[int(x) for x in rng.integers(1, 1500, int(rng.integers(1, 4)))],
                mode="decode" if rng.random() < 0.5 else "prefill", rng=rng)


def test_cases_are_valid_calls():
    """Host check: every drawn case fits the cache it builds (ring and row capacity)."""
    for i in range(N_CASES):
        c = draw_case(i)
        q_len = 1 if c["mode"] == "decode" else int(c["rng"].integers(1, min(min(c["lens"]), 400) + 1))
        w = synth.small("x", batch=len(c["lens"]), q_heads=c["kv"] * c["G"], kv_heads=c["kv"],
                        head_dim=c["D"], dtype=c["dtype"], block_size=c["bs"], sink=c["sink"],
                        recent=c["recent"], retrieval=c["ret"], context=max(c["lens"]),
                        q_len=q_len)
        assert w.ring_blocks * c["bs"] >= c["recent"] + q_len - 1
        assert w.max_blocks_per_head * c["bs"] >= max(c["lens"])


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_parity(i, _need_gpu):
    c = draw_case(i)
    lens = np.asarray(c["lens"])
    q_len = 1 if c["mode"] == "decode" else int(c["rng"].integers(1, min(lens.min(), 400) + 1))
    name = (f"{i}: {c['mode']} dtype {c['dtype']} D {c['D']} kv {c['kv']} G {c['G']} bs {c['bs']} "
            f"sink {c['sink']} recent {c['recent']} ret {c['ret']} lens {c['lens']} q_len {q_len}")
    say(name)
    B, dtype = len(lens), c["dtype"]
    w = synth.small(f"rand{i}", batch=B, q_heads=c["kv"] * c["G"], kv_heads=c["kv"],
                    head_dim=c["D"], dtype=dtype, block_size=c["bs"], sink=c["sink"],
                    recent=c["recent"], retrieval=c["ret"], context=int(lens.max()), q_len=q_len,
                    seed=100 + i)
    cache = Cache(w, fill="nan")
    Lm = int(lens.max())
    K = logical_kv(w, Lm, synth.S_K)
    V = logical_kv(w, Lm, synth.S_V)
    final = torch.zeros(B, dtype=torch.int32, device="cuda")
    for b in range(B):
        L = int(lens[b])
        kn = np.ascontiguousarray(K[b:b + 1, :, :L].transpose(0, 2, 1, 3))
        vn = np.ascontiguousarray(V[b:b + 1, :, :L].transpose(0, 2, 1, 3))
        before = torch.zeros(1, dtype=torch.int32, device="cuda")
        after = torch.zeros(1, dtype=torch.int32, device="cuda")
        duo.kv_append_circular(cache.k_pool, cache.v_pool, cache.table[b:b + 1],
                               to_dev(kn, dtype), to_dev(vn, dtype), before, after, cache.mask,
                               w.sink, w.recent, w.ring_blocks)
        final[b] = after[0]
    cache.lens = final
    if c["mode"] == "decode":
        q = q_decode(w, 0)
        got = to_host_f64(cache.decode(q), dtype)
        want = oracle_decode(w, q, K, V, lens, cache.mask)
    else:
        q = q_prefill(w, 0, q_len)
        got = to_host_f64(cache.prefill(q), dtype)
        want = oracle.attend(q, K, V, lens, cache.mask, sink=w.sink, recent=w.recent,
                             scale=w.scale, dtype=dtype)
    check_close(got, want, dtype, name)


# ------------------------------------------------------------------------------------------------
# the int8 cache and Dual Chunk Attention on seeded random shapes
# ------------------------------------------------------------------------------------------------
N_INT8 = 30
N_DCA = 24


def _fill(cache_append, K, V, lens, table):
    """Fill sequence b with positions [0, lens[b]) through batch-1 appends on table row slices."""
    final = torch.zeros(len(lens), dtype=torch.int32, device="cuda")
    for b, L in enumerate(lens):
        kn = np.ascontiguousarray(K[b:b + 1, :, :L].transpose(0, 2, 1, 3))
        vn = np.ascontiguousarray(V[b:b + 1, :, :L].transpose(0, 2, 1, 3))
        before = torch.zeros(1, dtype=torch.int32, device="cuda")
        final[b] = cache_append(kn, vn, table[b:b + 1], before)[0]
    return final


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_INT8))
def test_random_shape_int8_decode_parity(i, _need_gpu):
    from tests.test_gpu_int8 import Int8Cache, _logical_codes
    rng = np.random.default_rng([2025, i])
    dtype = (synth.F32, synth.F16, synth.BF16)[rng.integers(3)]
    D = (64, 128, 256)[rng.integers(3)]
    kv = int(rng.integers(1, 4))
    G = (1, 2, 4, 8)[rng.integers(4)]
    bs = (16, 32, 64)[rng.integers(3)]
    sink, recent = int(rng.integers(0, 40)), int(rng.integers(1, 200))
    ret = tuple(h for h in range(kv) if rng.random() < 0.5)
    lens = [int(x) for x in rng.integers(1, 1500, int(rng.integers(1, 4)))]
    split = (0, 128, 256)[rng.integers(3)]
    name = (f"int8 {i}: dtype {dtype} D {D} kv {kv} G {G} bs {bs} sink {sink} recent {recent} "
            f"ret {ret} lens {lens} split {split}")
    say(name)
    w = synth.small(f"rand8-{i}", batch=len(lens), q_heads=kv * G, kv_heads=kv, head_dim=D,
                    dtype=dtype, block_size=bs, sink=sink, recent=recent, retrieval=ret,
                    context=max(lens), q_len=1, seed=300 + i)
    cache = Int8Cache(w)
    K = logical_kv(w, max(lens), synth.S_K)
    V = logical_kv(w, max(lens), synth.S_V)
    cache.lens = _fill(lambda kn, vn, t, bf: cache.append(kn, vn, table=t, before=bf), K, V, lens,
                       cache.table)
    kc, ks, vc, vs = _logical_codes(K, V, dtype)
    q = q_decode(w, 0)
    want = oracle.attend_int8(q[:, None], kc, ks, vc, vs, np.asarray(lens), cache.mask,
                              sink=sink, recent=recent, scale=w.scale, dtype=dtype)[:, 0]
    got = to_host_f64(cache.decode(q, split_tokens=split), dtype)
    check_close(got, want, dtype, name)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_DCA))
def test_random_shape_dca_parity(i, _need_gpu):
    rng = np.random.default_rng([2026, i])
    dtype = (synth.F16, synth.BF16)[rng.integers(2)]
    D = (64, 128)[rng.integers(2)]
    kv = int(rng.integers(1, 4))
    G = (1, 2, 4, 8)[rng.integers(4)]
    bs = (16, 32, 64)[rng.integers(3)]
    chunk_len = (64, 128, 192, 256, 512)[rng.integers(5)]
    lens = [int(x) for x in rng.integers(1, 1500, int(rng.integers(1, 4)))]
    decode = rng.random() < 0.4
    q_len = 1 if decode else int(rng.integers(1, min(lens) + 1))
    name = (f"dca {i}: {'decode' if decode else 'prefill'} dtype {dtype} D {D} kv {kv} G {G} "
            f"bs {bs} chunk {chunk_len} lens {lens} q_len {q_len}")
    say(name)
    w = synth.small(f"randdca-{i}", batch=len(lens), q_heads=kv * G, kv_heads=kv, head_dim=D,
                    dtype=dtype, block_size=bs, sink=0, recent=1, retrieval=tuple(range(kv)),
                    context=max(lens), q_len=q_len, seed=400 + i)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, max(lens), synth.S_K)
    V = logical_kv(w, max(lens), synth.S_V)

    def app(kn, vn, t, before):
        after = torch.zeros(1, dtype=torch.int32, device="cuda")
        duo.kv_append_circular(cache.k_pool, cache.v_pool, t, to_dev(kn, dtype), to_dev(vn, dtype),
                               before, after, cache.mask, w.sink, w.recent, w.ring_blocks)
        return after
    cache.lens = _fill(app, K, V, lens, cache.table)
    qs = [synth.f32_to_storage(synth.queries(w, k, q_len=q_len), dtype) for k in range(3)]
    ms = synth.row_scales(w, 0, q_len)
    want = oracle.attend_dca(*qs, K, V, np.asarray(lens), ms, chunk_len=chunk_len, scale=w.scale,
                             dtype=dtype)
    qd = [to_dev(x, dtype) for x in qs]
    if decode:
        qd = [x[:, 0].contiguous() for x in qd]
        out = torch.empty_like(qd[0])
        ws = duo.decode_workspace(qd[0], cache.table, bs)
        duo.dca_attn_decode(*qd, torch.from_numpy(ms[:, 0].copy()).cuda(), chunk_len, cache.k_pool,
                            cache.v_pool, cache.table, cache.lens, w.scale, out, ws)
        got = to_host_f64(out, dtype)
        want = want[:, 0]
    else:
        out = torch.empty_like(qd[0])
        ws = duo.dca_prefill_workspace(qd[0], cache.table)
        duo.dca_attn_prefill(*qd, torch.from_numpy(ms).cuda(), chunk_len, cache.k_pool,
                             cache.v_pool, cache.table, cache.lens, w.scale, out, ws)
        got = to_host_f64(out, dtype)
    check_close(got, want, dtype, name)


N_VARLEN = 20


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_VARLEN))
def test_random_shape_varlen_prefill_parity(i, _need_gpu):
    """Packed batches: every sequence brings 0..len rows (a chunk, a single decode row or none)."""
    rng = np.random.default_rng([2027, i])
    dtype = (synth.F32, synth.F16, synth.BF16)[rng.integers(3)]
    D = (64, 128)[rng.integers(2)] if dtype == synth.F32 else (64, 128, 256)[rng.integers(3)]
    kv = int(rng.integers(1, 4))
    G = (1, 2, 4)[rng.integers(3)]
    bs = (16, 32, 64)[rng.integers(3)]
    sink, recent = int(rng.integers(0, 30)), int(rng.integers(1, 150))
    ret = tuple(h for h in range(kv) if rng.random() < 0.5)
    B = int(rng.integers(2, 5))
    lens = [int(x) for x in rng.integers(1, 1200, B)]
    rows = [int(rng.choice([0, 1, int(rng.integers(1, min(L, 300) + 1))])) for L in lens]
    rows = [min(r, L) for r, L in zip(rows, lens)]
    if sum(rows) == 0:
        rows[0] = 1
    max_q = max(rows)
    name = (f"varlen {i}: dtype {dtype} D {D} kv {kv} G {G} bs {bs} sink {sink} recent {recent} "
            f"ret {ret} lens {lens} rows {rows}")
    say(name)
    w = synth.small(f"randvl-{i}", batch=B, q_heads=kv * G, kv_heads=kv, head_dim=D, dtype=dtype,
                    block_size=bs, sink=sink, recent=recent, retrieval=ret, context=max(lens),
                    q_len=max_q, seed=500 + i)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, max(lens), synth.S_K)
    V = logical_kv(w, max(lens), synth.S_V)

    def app(kn, vn, t, before):
        after = torch.zeros(1, dtype=torch.int32, device="cuda")
        duo.kv_append_circular(cache.k_pool, cache.v_pool, t, to_dev(kn, dtype), to_dev(vn, dtype),
                               before, after, cache.mask, w.sink, w.recent, w.ring_blocks)
        return after
    cache.lens = _fill(app, K, V, lens, cache.table)
    qs = [q_prefill(w, b, n)[b:b + 1] for b, n in enumerate(rows)]
    packed = np.concatenate([q[0] for q in qs], axis=0)
    q_start = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    qd = to_dev(packed, dtype)
    out = torch.full_like(qd, float("nan"))
    ws = duo.prefill_varlen_workspace(qd, cache.table, cache.mask, max_q, B, w.block_size)
    duo.duo_attn_prefill_varlen(qd, cache.k_pool, cache.v_pool, cache.table, cache.lens,
                                torch.from_numpy(q_start).cuda(), max_q, cache.mask, w.sink,
                                w.recent, w.ring_blocks, w.scale, out, ws)
    got = to_host_f64(out, dtype)
    for b, n in enumerate(rows):
        if n == 0:
            continue
        want = oracle.attend(qs[b], K[b:b + 1], V[b:b + 1], np.asarray(lens[b:b + 1]), cache.mask,
                             sink=w.sink, recent=w.recent, scale=w.scale, dtype=dtype)[0]
        check_close(got[q_start[b]:q_start[b + 1]], want, dtype, f"{name} sequence {b}")


# ------------------------------------------------------------------------------------------------
# the 4-bit cache, and decode with GQA groups of more than 16 q heads, on seeded random shapes
# ------------------------------------------------------------------------------------------------
N_INT4 = 36
N_GROUPS = 30


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_INT4))
def test_random_shape_int4_decode_parity(i, _need_gpu):
    from tests.test_gpu_int4 import Int4Cache
    rng = np.random.default_rng([2028, i])
    dtype = (synth.F16, synth.BF16)[rng.integers(2)]
    D = (64, 128, 256)[rng.integers(3)]
    kv = int(rng.integers(1, 4))
    G = (1, 2, 4, 8, 16, 24, 33)[rng.integers(7)]
    bs = (16, 32, 64)[rng.integers(3)]
    sink, recent = int(rng.integers(0, 40)), int(rng.integers(1, 200))
    ret = tuple(h for h in range(kv) if rng.random() < 0.5)
    lens = [int(x) for x in rng.integers(1, 1500, int(rng.integers(1, 4)))]
    split = (0, 128, 256, 1024)[rng.integers(4)]
    name = (f"int4 {i}: dtype {dtype} D {D} kv {kv} G {G} bs {bs} sink {sink} recent {recent} "
            f"ret {ret} lens {lens} split {split}")
    say(name)
    w = synth.small(f"rand4-{i}", batch=len(lens), q_heads=kv * G, kv_heads=kv, head_dim=D,
                    dtype=dtype, block_size=bs, sink=sink, recent=recent, retrieval=ret,
                    context=max(lens), q_len=1, seed=500 + i)
    cache = Int4Cache(w)
    K = logical_kv(w, max(lens), synth.S_K)
    V = logical_kv(w, max(lens), synth.S_V)
    cache.fill_per_sequence(K, V, np.asarray(lens))
    kc, vc = cache.logical_codes(K, V)
    q = q_decode(w, 0)
    want = oracle.attend_int4(q[:, None], kc, vc, cache.ks_h, cache.vs_h, np.asarray(lens),
                              cache.mask, sink=sink, recent=recent, scale=w.scale,
                              dtype=dtype)[:, 0]
    got = to_host_f64(cache.decode(q, split_tokens=split), dtype)
    check_close(got, want, dtype, name)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_GROUPS))
def test_random_shape_large_group_decode_parity(i, _need_gpu):
    """Groups of 17 to 64 q heads per kv head: the decode takes them in chunks of 16 (the last one
    short), each chunk its own row of items, tickets and merge records."""
    rng = np.random.default_rng([2029, i])
    dtype = (synth.F32, synth.F16, synth.BF16)[rng.integers(3)]
    D = (64, 128, 256)[rng.integers(3)]
    kv = int(rng.integers(1, 3))
    G = (17, 20, 31, 32, 40, 48, 64)[rng.integers(7)]
    bs = (16, 32)[rng.integers(2)]
    sink, recent = int(rng.integers(0, 40)), int(rng.integers(1, 200))
    ret = tuple(h for h in range(kv) if rng.random() < 0.6)
    lens = [int(x) for x in rng.integers(0, 2500, int(rng.integers(1, 4)))]
    split = (0, 128, 512)[rng.integers(3)]
    name = (f"group {i}: dtype {dtype} D {D} kv {kv} G {G} bs {bs} sink {sink} recent {recent} "
            f"ret {ret} lens {lens} split {split}")
    say(name)
    Lm = max(max(lens), 1)
    w = synth.small(f"randg-{i}", batch=len(lens), q_heads=kv * G, kv_heads=kv, head_dim=D,
                    dtype=dtype, block_size=bs, sink=sink, recent=recent, retrieval=ret,
                    context=Lm, q_len=1, seed=700 + i)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, Lm, synth.S_K)
    V = logical_kv(w, Lm, synth.S_V)

    def app(kn, vn, t, before):
        if kn.shape[1] == 0:    # an empty sequence: nothing to append
            return before
        after = torch.zeros(1, dtype=torch.int32, device="cuda")
        duo.kv_append_circular(cache.k_pool, cache.v_pool, t, to_dev(kn, dtype),
                               to_dev(vn, dtype), before, after, cache.mask, w.sink, w.recent,
                               w.ring_blocks)
        return after
    cache.lens = _fill(app, K, V, lens, cache.table)
    q = q_decode(w, 0)
    got = to_host_f64(cache.decode(q, split_tokens=split), dtype)
    want = oracle_decode(w, q, K, V, np.asarray(lens), cache.mask)
    check_close(got, want, dtype, name)
    for b, L in enumerate(lens):
        if L == 0:
            assert (got[b] == 0).all()
