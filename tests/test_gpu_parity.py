"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded bits.

Bars: KV slot placement bit-exact (whole pools compared); attention outputs within max abs error
1e-4 (fp32) or 2e-2 (bf16/fp16) of the fp64 oracle. Pools start filled with NaN, so every slot the
kernels must not read is poisoned.
"""
import os

import numpy as np
import pytest
import torch

import kv_cache_sparsity_amd as duo
import oracle
import synth
from tests.gpu_harness import (Cache, check_close, logical_kv, q_decode, q_prefill, say, to_dev,
                               to_host_bits, to_host_f64, fill_bits, oracle_decode, TOL)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(duo.LIB_PATH):
        pytest.fail("libduoattn.so is not built; the GPU tests need the HIP library")


def _mask(hkv, ret):
    m = np.zeros(hkv, np.uint8)
    m[list(ret)] = 1
    return m


def _append_per_sequence(cache, K, V, lens):
    """Fill each sequence b with positions [0, lens[b]) (batch-1 calls on row slices)."""
    w = cache.w
    final = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    for b in range(w.batch):
        L = int(lens[b])
        if L == 0:
            continue
        kn = np.ascontiguousarray(K[b:b + 1, :, :L].transpose(0, 2, 1, 3))
        vn = np.ascontiguousarray(V[b:b + 1, :, :L].transpose(0, 2, 1, 3))
        before = torch.zeros(1, dtype=torch.int32, device="cuda")
        after = torch.zeros(1, dtype=torch.int32, device="cuda")
        duo.kv_append_circular(cache.k_pool, cache.v_pool, cache.table[b:b + 1],
                               to_dev(kn, w.dtype), to_dev(vn, w.dtype), before, after,
                               cache.mask, w.sink, w.recent, w.ring_blocks)
        final[b] = after[0]
    cache.lens = final


# ------------------------------------------------------------------------------------------------
# kv_append_circular: bit-exact pools
# ------------------------------------------------------------------------------------------------
APPEND_CASES = [
    dict(name="bf16-d128-bs16-sink4-ring2", dtype=synth.BF16, head_dim=128, block_size=16, sink=4,
         recent=24, ring_blocks=2, kv=3, ret=(0,), calls=[5, 40, 1, 1, 70]),
    dict(name="f32-d64-bs32-sink0-ring1", dtype=synth.F32, head_dim=64, block_size=32, sink=0,
         recent=20, ring_blocks=1, kv=2, ret=(1,), calls=[33, 2, 64, 7]),
    dict(name="f16-d256-bs16-sink20-ring3", dtype=synth.F16, head_dim=256, block_size=16, sink=20,
         recent=40, ring_blocks=3, kv=2, ret=(), calls=[1, 19, 3, 100, 16]),
    dict(name="bf16-d64-bs4-sink2-ring3", dtype=synth.BF16, head_dim=64, block_size=4, sink=2,
         recent=10, ring_blocks=3, kv=2, ret=(0,), calls=[17, 3, 30]),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[c["name"] for c in APPEND_CASES])
def test_append_bit_exact(case):
    say(f"append {case['name']}")
    total = sum(case["calls"])
    w = synth.small(case["name"], batch=2, q_heads=case["kv"], kv_heads=case["kv"],
                    head_dim=case["head_dim"], dtype=case["dtype"], block_size=case["block_size"],
                    sink=case["sink"], recent=case["recent"], retrieval=case["ret"],
                    context=total, ring_blocks=case["ring_blocks"], seed=21)
    cache = Cache(w, fill="sentinel")
    K = logical_kv(w, total, synth.S_K)
    V = logical_kv(w, total, synth.S_V)
    kp = to_host_bits(cache.k_pool, w.dtype).copy()
    vp = to_host_bits(cache.v_pool, w.dtype).copy()
    pos = 0
    for n in case["calls"]:
        kn = np.ascontiguousarray(K[:, :, pos:pos + n].transpose(0, 2, 1, 3))
        vn = np.ascontiguousarray(V[:, :, pos:pos + n].transpose(0, 2, 1, 3))
        before = cache.lens.cpu().numpy()
        cache.append(kn, vn)
        oracle.append(kp, vp, cache.table_h, kn, vn, before, cache.mask, sink=w.sink,
                      block_size=w.block_size, ring_blocks=w.ring_blocks,
                      max_blocks_per_head=w.max_blocks_per_head)
        pos += n
        assert cache.lens.cpu().tolist() == [pos] * w.batch
        gk = to_host_bits(cache.k_pool, w.dtype)
        gv = to_host_bits(cache.v_pool, w.dtype)
        assert gk.tobytes() == kp.tobytes(), f"K pool differs after {pos} tokens"
        assert gv.tobytes() == vp.tobytes(), f"V pool differs after {pos} tokens"


def test_append_reproduces_the_pages_circular_buffer_table():
    """vLLM issue 'Could you support Attention Sink?': the no-sink table (4 blocks of 4 slots)."""
    import tests.test_oracle_pins as pins
    table = pins._load_tables()["no_sink"]["states"]
    w = synth.small("page-table", batch=1, q_heads=1, kv_heads=1, head_dim=64, dtype=synth.F32,
                    block_size=4, sink=0, recent=16, retrieval=(), context=18, ring_blocks=4,
                    seed=1)
    cache = Cache(w, fill="sentinel", identity=True)
    for t in range(18):
        tok = np.full((1, 1, 1, 64), float(t), dtype=np.float32)
        cache.append(tok, tok)
        if t in table:
            k = to_host_bits(cache.k_pool, w.dtype)[:, :, 0]     # [4 pages][4 rows]
            got = [[None if x == cache.fill_value else int(x) for x in page] for page in k]
            assert got == table[t], (t, got)


# ------------------------------------------------------------------------------------------------
# decode
# ------------------------------------------------------------------------------------------------
DECODE_CASES = [
    dict(name="bf16-d128-g4-mixed", dtype=synth.BF16, head_dim=128, group=4, kv=2, ret=(0,),
         block_size=16, sink=4, recent=24, ring_blocks=2, lens=[1, 37, 300]),
    dict(name="f16-d256-g8-mqa", dtype=synth.F16, head_dim=256, group=8, kv=1, ret=(0,),
         block_size=16, sink=0, recent=1, ring_blocks=1, lens=[100, 1000, 4097]),
    dict(name="f32-d64-g1-mha", dtype=synth.F32, head_dim=64, group=1, kv=4, ret=(0, 2),
         block_size=16, sink=4, recent=64, ring_blocks=4, lens=[0, 3, 513]),
    dict(name="bf16-d64-g16-bs32-ringwrap", dtype=synth.BF16, head_dim=64, group=16, kv=2,
         ret=(1,), block_size=32, sink=0, recent=7, ring_blocks=1, lens=[50, 2000]),
    dict(name="bf16-d128-g2-bs64-sink70", dtype=synth.BF16, head_dim=128, group=2, kv=2, ret=(1,),
         block_size=64, sink=70, recent=100, ring_blocks=2, lens=[69, 70, 71, 170, 171, 5000]),
    dict(name="f16-d128-g4-all-streaming", dtype=synth.F16, head_dim=128, group=4, kv=3, ret=(),
         block_size=16, sink=16, recent=32, ring_blocks=2, lens=[16, 48, 49, 777]),
    dict(name="bf16-d128-g4-bs256", dtype=synth.BF16, head_dim=128, group=4, kv=2, ret=(0,),
         block_size=256, sink=3, recent=300, ring_blocks=2, lens=[255, 256, 257, 3000]),
    # groups of more than 16 q heads: taken in chunks of 16 (the last one short)
    dict(name="bf16-d128-g20-mixed", dtype=synth.BF16, head_dim=128, group=20, kv=2, ret=(1,),
         block_size=16, sink=4, recent=40, ring_blocks=3, lens=[0, 17, 900]),
    dict(name="f16-d64-g48-mqa", dtype=synth.F16, head_dim=64, group=48, kv=1, ret=(0,),
         block_size=32, sink=0, recent=1, ring_blocks=1, lens=[2049, 3]),
    dict(name="f16-d256-g40-streaming", dtype=synth.F16, head_dim=256, group=40, kv=2, ret=(),
         block_size=16, sink=16, recent=100, ring_blocks=8, lens=[700, 15]),
]


def _decode_case(case, split_tokens=0):
    lens = case["lens"]
    Lmax = max(lens)
    w = synth.small(case["name"], batch=len(lens), q_heads=case["kv"] * case["group"],
                    kv_heads=case["kv"], head_dim=case["head_dim"], dtype=case["dtype"],
                    block_size=case["block_size"], sink=case["sink"], recent=case["recent"],
                    retrieval=case["ret"], context=Lmax, ring_blocks=case["ring_blocks"], seed=31)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, Lmax, synth.S_K)
    V = logical_kv(w, Lmax, synth.S_V)
    _append_per_sequence(cache, K, V, lens)
    q = q_decode(w, 0)
    return w, cache, K, V, q


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c["name"] for c in DECODE_CASES])
def test_decode_parity(case):
    say(f"decode {case['name']}")
    w, cache, K, V, q = _decode_case(case)
    got = to_host_f64(cache.decode(q), w.dtype)
    want = oracle_decode(w, q, K, V, np.asarray(case["lens"]), cache.mask)
    check_close(got, want, w.dtype, case["name"])
    zero_rows = [b for b, L in enumerate(case["lens"]) if L == 0]
    for b in zero_rows:
        assert (got[b] == 0).all()


@pytest.mark.parametrize("split", [128, 1024])
def test_decode_large_group_explicit_splits(split):
    """A group of 20 q heads (chunks of 16 and 4) with explicit splits: records of the short chunk
    and merges across splits."""
    case = next(c for c in DECODE_CASES if c["name"] == "bf16-d128-g20-mixed")
    say(f"decode group 20, split {split}")
    w, cache, K, V, q = _decode_case(case)
    got = to_host_f64(cache.decode(q, split_tokens=split), w.dtype)
    want = oracle_decode(w, q, K, V, np.asarray(case["lens"]), cache.mask)
    check_close(got, want, w.dtype, f"group 20 split={split}")
    assert (got[0] == 0).all()


@pytest.mark.parametrize("split", [128, 256, 1024, 0])
def test_decode_split_count_invariance(split):
    case = DECODE_CASES[1]
    say(f"decode split {split}")
    w, cache, K, V, q = _decode_case(case)
    got = to_host_f64(cache.decode(q, split_tokens=split), w.dtype)
    want = oracle_decode(w, q, K, V, np.asarray(case["lens"]), cache.mask)
    check_close(got, want, w.dtype, f"split={split}")


@pytest.mark.parametrize("L", [32768, 32769, 40000])
def test_decode_merge_at_and_past_256_splits(L):
    """128-key splits: 256 live splits take the two-phase merge (weights in LDS), 257 and more the
    one-pass online merge."""
    say(f"decode 128-key splits, L={L}")
    w = synth.small(f"many-splits-{L}", batch=1, q_heads=8, kv_heads=2, head_dim=128,
                    dtype=synth.BF16, block_size=16, sink=4, recent=64, retrieval=(1,), context=L,
                    seed=33)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, L, synth.S_K)
    V = logical_kv(w, L, synth.S_V)
    cache.append_logical(K, V, 0, L)
    q = q_decode(w, 0)
    got = to_host_f64(cache.decode(q, split_tokens=128), w.dtype)
    want = oracle_decode(w, q, K, V, np.array([L]), cache.mask)
    check_close(got, want, w.dtype, f"L={L} split=128")


TWO_LEVEL_CASE = dict(name="bf16-d128-g4-two-level-merge", dtype=synth.BF16, head_dim=128, group=4,
                      kv=2, ret=(0, 1), block_size=16, sink=4, recent=24, ring_blocks=2,
                      lens=[0, 1, 2047, 2048, 2049, 5120])


def test_decode_two_level_merge_ragged_rows_and_workspace_reuse():
    """More than 16 splits per row merge in two levels (groups of 16 splits, then the groups). With
    128-key splits over 5120 keys of capacity a row has 40 splits in 3 groups; the ragged lengths
    leave whole groups empty (length 1, 2047, 2048) or cut one inside (2049), and length 0 leaves
    every group empty. One workspace serves 128-, 256- and automatic splits in turn, twice, so every
    ticket must be back at zero after each call."""
    case = TWO_LEVEL_CASE
    say(f"decode {case['name']}")
    w, cache, K, V, q = _decode_case(case)
    want = oracle_decode(w, q, K, V, np.asarray(case["lens"]), cache.mask)
    qd = to_dev(q, w.dtype)
    ws = duo.decode_workspace(qd, cache.table, w.block_size, 128)
    for rep in range(2):
        for split in (128, 256, 0):
            got = to_host_f64(cache.decode(q, split_tokens=split, workspace=ws), w.dtype)
            check_close(got, want, w.dtype, f"{case['name']} split {split} pass {rep}")
            assert (got[0] == 0).all()


def test_profile_hook_times_one_kernel_then_clears():
    """duo_profile_next_launch: the next call's kernel records the events on its dispatch; the call
    after it leaves them alone."""
    case = DECODE_CASES[0]
    w, cache, K, V, q = _decode_case(case)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    duo.profile_next_launch(a, b)
    got = to_host_f64(cache.decode(q), w.dtype)
    torch.cuda.synchronize()
    t1 = a.elapsed_time(b)
    assert 0.0 < t1 < 100.0, t1
    cache.decode(q)
    torch.cuda.synchronize()
    assert a.elapsed_time(b) == t1
    want = oracle_decode(w, q, K, V, np.asarray(case["lens"]), cache.mask)
    check_close(got, want, w.dtype, "decode with launch events")


def test_decode_repeated_calls_and_workspace_reuse():
    """Repeated calls on one workspace, with 1024-key splits, so that each work item has more 32-key
    steps than its workgroup has waves and the waves claim the later steps at run time. Which wave
    takes which step depends on timing, so the rounding of the sums may differ from call to call
    (the decode is not bitwise reproducible); every call must stay within the tolerance of the
    oracle, and every merge ticket must be back at zero after each call."""
    case = dict(name="bf16-d128-g4-claimed-steps", dtype=synth.BF16, head_dim=128, group=4, kv=2,
                ret=(0, 1), block_size=16, sink=4, recent=24, ring_blocks=2,
                lens=[1, 1023, 1024, 1025, 4000, 8192])
    w, cache, K, V, q = _decode_case(case)
    want = oracle_decode(w, q, K, V, np.asarray(case["lens"]), cache.mask)
    qd = to_dev(q, w.dtype)
    ws = duo.decode_workspace(qd, cache.table, w.block_size, 1024)
    outs = []
    for rep in range(4):
        got = cache.decode(q, split_tokens=1024, workspace=ws)
        outs.append(to_host_bits(got, w.dtype))
        check_close(to_host_f64(got, w.dtype), want, w.dtype, f"call {rep}")
        torch.cuda.synchronize()
        nctr = w.batch * w.num_kv_heads
        assert int(ws[:4 * nctr].view(torch.int32).abs().sum().item()) == 0
    same = sum(o.tobytes() == outs[0].tobytes() for o in outs[1:])
    say(f"  {same} of 3 repeated calls bitwise equal to the first")


_rng_ret = np.random.default_rng(97)
ALL_RETRIEVAL_CASES = [
    # 64 sequences: empty, one-token and full rows among random ones
    dict(name="bf16-d128-g4-b64", dtype=synth.BF16, head_dim=128, group=4, kv=2, ret=(0, 1),
         block_size=16, sink=0, recent=1, ring_blocks=1,
         lens=[0, 1, 4096, 4095] + [int(x) for x in _rng_ret.integers(0, 4097, 60)]),
    # a Gemma-like static cache: lengths around split boundaries
    dict(name="f16-d256-g8-mqa", dtype=synth.F16, head_dim=256, group=8, kv=1, ret=(0,),
         block_size=16, sink=0, recent=1, ring_blocks=1,
         lens=[0, 1, 5, 383, 384, 385, 2000, 8192]),
    # q heads in chunks of 16 (two rows per sequence and kv head)
    dict(name="bf16-d64-g20", dtype=synth.BF16, head_dim=64, group=20, kv=1, ret=(0,),
         block_size=32, sink=0, recent=1, ring_blocks=1, lens=[1, 700, 3000]),
    # short rows: one live split each, the rest of the row's items past its length
    dict(name="f16-d128-short", dtype=synth.F16, head_dim=128, group=2, kv=3, ret=(0, 1, 2),
         block_size=16, sink=0, recent=1, ring_blocks=1, lens=[1, 2, 15, 16, 17, 40]),
]


@pytest.mark.parametrize("case", ALL_RETRIEVAL_CASES, ids=[c["name"] for c in ALL_RETRIEVAL_CASES])
def test_decode_all_retrieval_mixed_lengths(case):
    """No streaming heads, the library's split, lengths from 0 to the capacity (many items past
    their row's length). Two calls on one workspace, each within the oracle's tolerance, every merge
    ticket back at zero after each."""
    say(f"decode, all retrieval heads: {case['name']}")
    w, cache, K, V, q = _decode_case(case)
    want = oracle_decode(w, q, K, V, np.asarray(case["lens"]), cache.mask)
    qd = to_dev(q, w.dtype)
    ws = duo.decode_workspace(qd, cache.table, w.block_size, 0)
    gch = -(-case["group"] // 16)
    for rep in range(2):
        got = to_host_f64(cache.decode(q, workspace=ws), w.dtype)
        check_close(got, want, w.dtype, f"{case['name']} call {rep}")
        for b, L in enumerate(case["lens"]):
            if L == 0:
                assert (got[b] == 0).all()
        torch.cuda.synchronize()
        nctr = w.batch * w.num_kv_heads * gch
        assert int(ws[:4 * nctr].view(torch.int32).abs().sum().item()) == 0


# ------------------------------------------------------------------------------------------------
# prefill
# ------------------------------------------------------------------------------------------------
PREFILL_CASES = [
    dict(name="bf16-d128-mha-ragged300", dtype=synth.BF16, head_dim=128, group=1, kv=4,
         ret=(0, 3), block_size=16, sink=8, recent=40, chunks=[300]),
    dict(name="bf16-d128-chunked3x200", dtype=synth.BF16, head_dim=128, group=1, kv=2, ret=(1,),
         block_size=16, sink=8, recent=40, chunks=[200, 200, 200]),
    dict(name="f16-d64-gqa4-q129", dtype=synth.F16, head_dim=64, group=4, kv=2, ret=(0,),
         block_size=16, sink=3, recent=20, chunks=[129]),
    dict(name="f32-d64-q512", dtype=synth.F32, head_dim=64, group=1, kv=4, ret=(0, 1),
         block_size=16, sink=4, recent=64, chunks=[512]),
    dict(name="f16-d256-q64x2", dtype=synth.F16, head_dim=256, group=2, kv=1, ret=(), block_size=16,
         sink=16, recent=16, chunks=[64, 64]),
    dict(name="bf16-d128-bs32-sink5", dtype=synth.BF16, head_dim=128, group=1, kv=2, ret=(0,),
         block_size=32, sink=5, recent=77, chunks=[150, 260]),
    dict(name="f32-d128-g2-chunks", dtype=synth.F32, head_dim=128, group=2, kv=2, ret=(1,),
         block_size=16, sink=1, recent=1, chunks=[33, 1, 128]),
    dict(name="bf16-d128-bs64-q333x2", dtype=synth.BF16, head_dim=128, group=1, kv=2, ret=(0,),
         block_size=64, sink=20, recent=200, chunks=[333, 333]),
    dict(name="bf16-d64-g2-bs256-q700", dtype=synth.BF16, head_dim=64, group=2, kv=2, ret=(1,),
         block_size=256, sink=0, recent=128, chunks=[700]),
]


def _rows_all(B, q_len, Hq):
    return [(b, i, hq) for b in range(B) for hq in range(Hq) for i in range(q_len)]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c["name"] for c in PREFILL_CASES])
def test_prefill_parity(case):
    say(f"prefill {case['name']}")
    chunks = case["chunks"]
    total = sum(chunks)
    w = synth.small(case["name"], batch=2, q_heads=case["kv"] * case["group"], kv_heads=case["kv"],
                    head_dim=case["head_dim"], dtype=case["dtype"], block_size=case["block_size"],
                    sink=case["sink"], recent=case["recent"], retrieval=case["ret"], context=total,
                    q_len=max(chunks), seed=41)
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
                             rows=_rows_all(w.batch, n, w.num_q_heads))
        check_close(got, want, w.dtype, f"{case['name']} chunk {ci}")


def test_shared_sink_pages_across_sequences():
    """Streaming heads of every sequence point at one set of sink pages (option 3 of the vLLM
    attention-sink issue: sinks in blocks of their own, reusable by every request that starts with
    the same sink tokens). Every sequence appends its own positions, so the shared pages receive the
    same bits from each; decode and prefill read them through the table."""
    say("shared sink pages")
    w = synth.small("shared-sinks", batch=4, q_heads=8, kv_heads=4, head_dim=128,
                    dtype=synth.BF16, block_size=16, sink=20, recent=64, retrieval=(0, 2),
                    context=600, q_len=64, seed=47)
    cache = Cache(w, fill="nan", share_sinks=True)
    t = cache.table_h
    for h in (1, 3):                       # streaming heads share their two sink pages
        assert (t[:, h, :w.sink_blocks] == t[0, h, :w.sink_blocks]).all()
    K = logical_kv(w, 600, synth.S_K)
    V = logical_kv(w, 600, synth.S_V)
    K[:, :, :w.sink] = K[0:1, :, :w.sink]  # the same first sink tokens in every sequence
    V[:, :, :w.sink] = V[0:1, :, :w.sink]
    cache.append_logical(K, V, 0, 536)
    cache.append_logical(K, V, 536, 600)
    torch.cuda.synchronize()
    kp = to_host_bits(cache.k_pool, w.dtype)
    for h in (1, 3):
        for s in range(w.sink):
            assert np.array_equal(kp[t[0, h, s // 16], s % 16], K[0, h, s])
    lens = np.full(w.batch, 600)
    q = q_prefill(w, 0, 64)
    got = to_host_f64(cache.prefill(q), w.dtype)
    want = oracle.attend(q, K, V, lens, cache.mask, sink=w.sink, recent=w.recent, scale=w.scale,
                         dtype=w.dtype)
    check_close(got, want, w.dtype, "shared sinks prefill")
    qd = q_decode(w, 1)
    got = to_host_f64(cache.decode(qd), w.dtype)
    check_close(got, oracle_decode(w, qd, K, V, lens, cache.mask), w.dtype, "shared sinks decode")


VARLEN_CASES = [
    dict(name="bf16-d128-gqa2", dtype=synth.BF16, head_dim=128, group=2, kv=2, ret=(0,),
         block_size=16, sink=4, recent=64, rows=[300, 1, 0, 37], lens=[700, 512, 100, 37]),
    dict(name="f16-d64-mha-bs64", dtype=synth.F16, head_dim=64, group=1, kv=3, ret=(1, 2),
         block_size=64, sink=0, recent=40, rows=[5, 129, 64], lens=[5, 900, 64]),
    dict(name="f32-d64-all-streaming", dtype=synth.F32, head_dim=64, group=2, kv=1, ret=(),
         block_size=16, sink=7, recent=30, rows=[33, 2], lens=[400, 40]),
    # a group of 24: the single rows' decode items take the q heads in chunks of 16 and 8
    dict(name="bf16-d128-gqa24", dtype=synth.BF16, head_dim=128, group=24, kv=2, ret=(1,),
         block_size=16, sink=4, recent=64, rows=[1, 70, 1, 1], lens=[900, 300, 1, 2000]),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[c["name"] for c in VARLEN_CASES])
def test_prefill_varlen_parity(case):
    """A packed batch: each sequence brings its own rows (a chunk, a single decode row, none)."""
    say(f"prefill varlen {case['name']}")
    rows, lens = case["rows"], np.asarray(case["lens"])
    B, max_q = len(rows), max(rows)
    w = synth.small(case["name"], batch=B, q_heads=case["kv"] * case["group"], kv_heads=case["kv"],
                    head_dim=case["head_dim"], dtype=case["dtype"], block_size=case["block_size"],
                    sink=case["sink"], recent=case["recent"], retrieval=case["ret"],
                    context=int(lens.max()), q_len=max_q, seed=46)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, int(lens.max()), synth.S_K)
    V = logical_kv(w, int(lens.max()), synth.S_V)
    _append_per_sequence(cache, K, V, lens)
    qs = [q_prefill(w, b, n)[b:b + 1] for b, n in enumerate(rows)]   # [1][n][Hq][D] per sequence
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
                             sink=w.sink, recent=w.recent, scale=w.scale, dtype=w.dtype)[0]
        check_close(got[q_start[b]:q_start[b + 1]], want, w.dtype, f"{case['name']} sequence {b}")


def test_prefill_rows_before_the_sequence_start_are_zero():
    """seq_len < q_len: rows at negative positions see nothing (zero output)."""
    w = synth.small("neg-rows", batch=1, q_heads=2, kv_heads=2, head_dim=64, dtype=synth.BF16,
                    block_size=16, sink=2, recent=8, retrieval=(0,), context=20, q_len=25, seed=43)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, 20, synth.S_K)
    V = logical_kv(w, 20, synth.S_V)
    cache.append_logical(K, V, 0, 20)
    q = q_prefill(w, 0, 25)
    got = to_host_f64(cache.prefill(q), w.dtype)
    want = oracle.attend(q, K, V, np.array([20]), cache.mask, sink=w.sink, recent=w.recent,
                         scale=w.scale, dtype=w.dtype)
    assert (got[0, :5] == 0).all()
    check_close(got, want, w.dtype, "negative rows")


def test_prefill_is_deterministic():
    case = PREFILL_CASES[0]
    w = synth.small("det", batch=1, q_heads=4, kv_heads=4, head_dim=128, dtype=synth.BF16,
                    block_size=16, sink=8, recent=40, retrieval=(0, 3), context=300, q_len=300,
                    seed=44)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, 300, synth.S_K)
    V = logical_kv(w, 300, synth.S_V)
    cache.append_logical(K, V, 0, 300)
    q = q_prefill(w, 0, 300)
    a = to_host_bits(cache.prefill(q), w.dtype)
    b = to_host_bits(cache.prefill(q), w.dtype)
    assert a.tobytes() == b.tobytes()


@pytest.mark.parametrize("context", [16250, 16384, 20000])
def test_prefill_long_retrieval_rows(context):
    """A short chunk at the end of a long context: a retrieval item's keys are split between
    workgroups, and the split point and the edges of the kernel's staged page lists (512 runs)
    fall one tile apart (16250), together (16384) or apart (20000)."""
    q_len = 40
    w = synth.small(f"long-ret-{context}", batch=1, q_heads=4, kv_heads=2, head_dim=64,
                    dtype=synth.BF16, block_size=16, sink=4, recent=64, retrieval=(0,),
                    context=context, q_len=q_len, seed=45)
    say(f"prefill long retrieval rows, context {context}")
    cache = Cache(w, fill="nan")
    K = logical_kv(w, context, synth.S_K)
    V = logical_kv(w, context, synth.S_V)
    cache.append_logical(K, V, 0, context)
    q = q_prefill(w, 0, q_len)
    got = to_host_f64(cache.prefill(q), w.dtype)
    want = oracle.attend(q, K, V, np.full(w.batch, context), cache.mask, sink=w.sink,
                         recent=w.recent, scale=w.scale, dtype=w.dtype,
                         rows=_rows_all(w.batch, q_len, w.num_q_heads))
    check_close(got, want, w.dtype, f"context {context}")


# ------------------------------------------------------------------------------------------------
# The five workloads at their real shapes
# ------------------------------------------------------------------------------------------------
def test_tiny_f32_prefill_then_16_decode_steps():
    w = synth.tiny()
    say(f"workload {w.name}")
    total = w.context + w.steps
    cache = Cache(w, fill="nan")
    K = logical_kv(w, total, synth.S_K)
    V = logical_kv(w, total, synth.S_V)
    cache.append_logical(K, V, 0, w.context)
    q = q_prefill(w, 0, w.q_len)
    got = to_host_f64(cache.prefill(q), w.dtype)
    want = oracle.attend(q, K, V, np.array([w.context]), cache.mask, sink=w.sink, recent=w.recent,
                         scale=w.scale, dtype=w.dtype)
    check_close(got, want, w.dtype, "tiny prefill 512")
    for step in range(1, w.steps + 1):
        L = w.context + step
        cache.append_logical(K, V, L - 1, L)
        q1 = q_decode(w, step)
        got = to_host_f64(cache.decode(q1), w.dtype)
        want = oracle_decode(w, q1, K, V, np.array([L]), cache.mask)
        check_close(got, want, w.dtype, f"tiny decode step {step}")


def test_llama3_8b_gqa_decode_batch8_ctx32768():
    w = synth.llama3_8b_decode()
    say(f"workload {w.name}")
    L = w.context
    cache = Cache(w, fill="nan")
    K = logical_kv(w, L, synth.S_K)
    V = logical_kv(w, L, synth.S_V)
    cache.append_logical(K, V, 0, L - 1, chunk=8192)
    cache.append_logical(K, V, L - 1, L)          # the decoded token
    q = q_decode(w, 0)
    got = to_host_f64(cache.decode(q), w.dtype)
    want = oracle_decode(w, q, K, V, np.full(w.batch, L), cache.mask)
    check_close(got, want, w.dtype, w.name)
    # spot-check slot placement on the big pools: pages of sequence 0 against the oracle's gather
    kp = to_host_bits(cache.k_pool, w.dtype)
    vp = to_host_bits(cache.v_pool, w.dtype)
    for h in range(w.num_kv_heads):
        ret = bool(cache.mask[h])
        pos = np.arange(L) if ret else np.r_[np.arange(w.sink), np.arange(L - 256, L)]
        kg, vg = oracle.gather(kp, vp, cache.table_h, 0, h, pos, retrieval=ret, sink=w.sink,
                               block_size=w.block_size, ring_blocks=w.ring_blocks)
        assert kg.tobytes() == K[0, h, pos].tobytes()
        assert vg.tobytes() == V[0, h, pos].tobytes()


def _tile_rows(q_len, tile, per_tile, rng):
    """per_tile rows of every tile of `tile` rows: its first two, the rows at a quarter, half and
    its last one, and random others."""
    rows = []
    for t0 in range(0, q_len, tile):
        t1 = min(q_len, t0 + tile)
        fixed = {t0, t0 + 1, t0 + 31, t0 + 32, t0 + tile // 2 - 1, t0 + tile // 2, t1 - 1}
        fixed = {r for r in fixed if t0 <= r < t1}
        rest = np.setdiff1d(np.arange(t0, t1), sorted(fixed))
        extra = rng.choice(rest, size=min(len(rest), per_tile - len(fixed)), replace=False)
        rows.extend(sorted(fixed | set(int(x) for x in extra)))
    return np.array(rows, dtype=np.int64)


@pytest.mark.timeout(600)
def test_llama2_7b_mha_chunked_prefill_row_tiles():
    """Eight 4096-row chunks building a 32768-token context (32 heads, 8 retrieval). Every row of
    chunk 0 and 512 rows of each later chunk (32 in every 256-row tile, tile edges included) are
    compared on all 32 heads. The oracle takes all sampled rows of a head in one score matrix
    (oracle.attend_rows); a streaming head's keys are its sinks and the union of the rows' windows."""
    w = synth.llama2_7b_chunked_prefill()
    say(f"workload {w.name}")
    cache = Cache(w, fill="nan")
    K = logical_kv(w, w.context, synth.S_K)
    V = logical_kv(w, w.context, synth.S_V)
    rng = np.random.default_rng(99)
    for c in range(w.steps):
        lo = c * w.q_len
        Lc = lo + w.q_len
        cache.append_logical(K, V, lo, Lc, chunk=w.q_len)
        q = q_prefill(w, c, w.q_len)
        got = to_host_f64(cache.prefill(q), w.dtype)
        assert np.isfinite(got).all()
        rows = np.arange(w.q_len) if c == 0 else _tile_rows(w.q_len, 256, 32, rng)
        p = lo + rows
        errs = []
        for hq in range(w.num_q_heads):
            h = hq // w.group
            ret = bool(cache.mask[h])
            # a retrieval head's rows in one block over all keys; a streaming head's rows tile by
            # tile, each over its sinks and the union of its rows' windows
            blocks = [np.arange(len(rows))] if ret else np.array_split(
                np.arange(len(rows)), max(1, len(rows) // 256))
            for blk in blocks:
                pb = p[blk]
                keys = (np.arange(Lc) if ret else np.union1d(
                    np.arange(w.sink), np.arange(max(0, int(pb.min()) - w.recent + 1), int(pb.max()) + 1)))
                want = oracle.attend_rows(oracle.to_f64(q[0, rows[blk], hq], w.dtype), pb,
                                          oracle.to_f64(K[0, h, keys], w.dtype),
                                          oracle.to_f64(V[0, h, keys], w.dtype), keys,
                                          retrieval=ret, sink=w.sink, recent=w.recent,
                                          scale=w.scale)
                errs.append(np.abs(got[0, rows[blk], hq] - want).max())
        err = float(max(errs))
        say(f"  chunk {c}: {len(rows)} rows x {w.num_q_heads} heads, max |gpu - oracle| = "
            f"{err:.3e} (tol {TOL[w.dtype]:.0e})")
        assert err <= TOL[w.dtype], (c, err)


@pytest.mark.timeout(900)
def test_continuous_batching_step_one_chunk_and_31_decode_rows():
    """One packed call on the Llama-3-8B GQA shape at 32768 tokens: sequence 0 brings a 4096-row
    chunk, sequences 1..31 one decode row each (run as split-K decode items in the same launch).
    Every q head of every decode row is compared, and 512 rows of the chunk (32 in every 256-row
    tile) on every q head. The oracle runs sequence by sequence while the cache is filled, so each
    sequence's keys and values are drawn once."""
    w = synth.continuous_batching_step()
    rows_n = w.extra["rows"]
    L = w.context
    say(f"workload {w.name}")
    cache = Cache(w, fill="nan")
    B, Hq, G = w.batch, w.num_q_heads, w.group
    q_start = np.concatenate([[0], np.cumsum(rows_n)]).astype(np.int32)
    qs = [q_prefill(w, b, n)[b:b + 1] for b, n in enumerate(rows_n)]   # [1][n][Hq][D] each
    packed = np.concatenate([q[0] for q in qs], axis=0)
    rng = np.random.default_rng(17)
    chunk_rows = _tile_rows(rows_n[0], 256, 32, rng)
    want = {}
    for b in range(B):
        Kb = np.stack([synth.f32_to_storage(synth.kv_tokens(w, synth.S_K, b, h, 0, L), w.dtype)
                       for h in range(w.num_kv_heads)])[None]
        Vb = np.stack([synth.f32_to_storage(synth.kv_tokens(w, synth.S_V, b, h, 0, L), w.dtype)
                       for h in range(w.num_kv_heads)])[None]
        z = torch.zeros(1, dtype=torch.int32, device="cuda")
        duo.kv_append_circular(cache.k_pool, cache.v_pool, cache.table[b:b + 1],
                               to_dev(np.ascontiguousarray(Kb.transpose(0, 2, 1, 3)), w.dtype),
                               to_dev(np.ascontiguousarray(Vb.transpose(0, 2, 1, 3)), w.dtype),
                               z, torch.empty_like(z), cache.mask, w.sink, w.recent, w.ring_blocks)
        n = rows_n[b]
        rows = chunk_rows if n > 1 else np.arange(1)
        p = L - n + rows
        for h in range(w.num_kv_heads):
            ret = bool(cache.mask[h])
            keys = (np.arange(L) if ret else
                    np.union1d(np.arange(w.sink), np.arange(max(0, int(p.min()) - w.recent + 1), L)))
            Kf = oracle.to_f64(Kb[0, h, keys], w.dtype)
            Vf = oracle.to_f64(Vb[0, h, keys], w.dtype)
            for hq in range(h * G, (h + 1) * G):
                if ret or n == 1:
                    want[(b, hq)] = oracle.attend_rows(oracle.to_f64(qs[b][0, rows, hq], w.dtype), p,
                                                       Kf, Vf, keys, retrieval=ret, sink=w.sink,
                                                       recent=w.recent, scale=w.scale)
                else:   # a streaming head's chunk rows, tile by tile over their own windows
                    out_rows = []
                    for blk in np.array_split(np.arange(len(rows)), len(rows) // 32):
                        pb = p[blk]
                        kk = np.union1d(np.arange(w.sink),
                                        np.arange(max(0, int(pb.min()) - w.recent + 1), int(pb.max()) + 1))
                        sel = np.searchsorted(keys, kk)
                        out_rows.append(oracle.attend_rows(
                            oracle.to_f64(qs[b][0, rows[blk], hq], w.dtype), pb, Kf[sel], Vf[sel],
                            kk, retrieval=False, sink=w.sink, recent=w.recent, scale=w.scale))
                    want[(b, hq)] = np.concatenate(out_rows)
    cache.set_lens(np.full(B, L))
    say("  filled; oracle done")
    qd = to_dev(packed, w.dtype)
    out = torch.full_like(qd, float("nan"))
    ws = duo.prefill_varlen_workspace(qd, cache.table, cache.mask, rows_n[0], B, w.block_size)
    duo.duo_attn_prefill_varlen(qd, cache.k_pool, cache.v_pool, cache.table, cache.lens,
                                torch.from_numpy(q_start).cuda(), rows_n[0], cache.mask, w.sink,
                                w.recent, w.ring_blocks, w.scale, out, ws)
    got = to_host_f64(out, w.dtype)
    assert np.isfinite(got).all()
    err_chunk = max(float(np.abs(got[q_start[0] + chunk_rows, hq] - want[(0, hq)]).max())
                    for hq in range(Hq))
    err_dec = max(float(np.abs(got[q_start[b], hq] - want[(b, hq)][0]).max())
                  for b in range(1, B) for hq in range(Hq))
    say(f"  chunk rows: max |gpu - oracle| = {err_chunk:.3e}; decode rows: {err_dec:.3e} "
        f"(tol {TOL[w.dtype]:.0e})")
    assert err_chunk <= TOL[w.dtype] and err_dec <= TOL[w.dtype]


def test_gemma_2b_mqa_static_decode_with_garbage_past_lengths():
    w = synth.gemma_2b_static_decode()
    say(f"workload {w.name}")
    cap = w.context
    lens = synth.valid_lengths(w, 1024, cap)
    K = logical_kv(w, cap, synth.S_K)
    V = logical_kv(w, cap, synth.S_V)
    for b in range(w.batch):    # slots past each length hold arbitrary bits (NaN/Inf included)
        n = cap - int(lens[b])
        K[b, 0, lens[b]:] = synth.garbage_bits(w.seed, 0, b, shape=(n, w.head_dim), dtype=w.dtype)
        V[b, 0, lens[b]:] = synth.garbage_bits(w.seed, 1, b, shape=(n, w.head_dim), dtype=w.dtype)
    cache = Cache(w, fill="nan", identity=True)
    cache.append_logical(K, V, 0, cap, chunk=4096)
    cache.set_lens(lens)
    q = q_decode(w, 0)
    got = to_host_f64(cache.decode(q), w.dtype)
    want = oracle_decode(w, q, K, V, lens, cache.mask)
    check_close(got, want, w.dtype, w.name)


@pytest.mark.timeout(600)
def test_long_context_decode_1m_tokens_64_steps():
    w = synth.long_context_decode()
    say(f"workload {w.name}")
    L0 = w.context
    cache = Cache(w, fill="nan")
    mask = cache.mask
    # fill 1,048,576 tokens head by head in 64K-token pieces (setup, not checked here)
    piece = 65536
    for s in range(0, L0, piece):
        kn = np.empty((1, piece, w.num_kv_heads, w.head_dim), np.uint16)
        vn = np.empty_like(kn)
        for h in range(w.num_kv_heads):
            kn[0, :, h] = synth.f32_to_storage(synth.kv_tokens(w, synth.S_K, 0, h, s, s + piece), w.dtype)
            vn[0, :, h] = synth.f32_to_storage(synth.kv_tokens(w, synth.S_V, 0, h, s, s + piece), w.dtype)
        cache.append(kn, vn)
    say("  filled")
    check_steps = {1, 32, 64}
    Lf = L0 + w.steps
    full = {}
    for h in range(w.num_kv_heads):
        if mask[h]:
            full[h] = (oracle.to_f64(synth.f32_to_storage(synth.kv_tokens(w, synth.S_K, 0, h, 0, Lf), w.dtype), w.dtype),
                       oracle.to_f64(synth.f32_to_storage(synth.kv_tokens(w, synth.S_V, 0, h, 0, Lf), w.dtype), w.dtype))
    for step in range(1, w.steps + 1):
        L = L0 + step
        kn = np.empty((1, 1, w.num_kv_heads, w.head_dim), np.uint16)
        vn = np.empty_like(kn)
        for h in range(w.num_kv_heads):
            kn[0, 0, h] = synth.f32_to_storage(synth.kv_tokens(w, synth.S_K, 0, h, L - 1, L), w.dtype)[0]
            vn[0, 0, h] = synth.f32_to_storage(synth.kv_tokens(w, synth.S_V, 0, h, L - 1, L), w.dtype)[0]
        cache.append(kn, vn)
        q = q_decode(w, step)
        out = cache.decode(q)
        if step not in check_steps:
            continue
        got = to_host_f64(out, w.dtype)
        want = np.empty_like(got)
        for hq in range(w.num_q_heads):
            h = hq // w.group
            J = oracle.visible_positions(L - 1, retrieval=bool(mask[h]), sink=w.sink,
                                         recent=w.recent)
            if mask[h]:
                Kf, Vf = full[h]
                Kj, Vj = Kf[J], Vf[J]
            else:
                # sinks then the recent window (disjoint at this length)
                assert J.tolist() == list(range(w.sink)) + list(range(L - w.recent, L))
                parts = [(0, w.sink), (L - w.recent, L)]
                Kj = oracle.to_f64(np.concatenate([synth.f32_to_storage(
                    synth.kv_tokens(w, synth.S_K, 0, h, a, e), w.dtype) for a, e in parts]), w.dtype)
                Vj = oracle.to_f64(np.concatenate([synth.f32_to_storage(
                    synth.kv_tokens(w, synth.S_V, 0, h, a, e), w.dtype) for a, e in parts]), w.dtype)
            want[0, hq] = oracle.attend_row(oracle.to_f64(q[0, hq], w.dtype), Kj, Vj, w.scale)
        check_close(got, want, w.dtype, f"1M decode step {step}")
