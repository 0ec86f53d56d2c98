"""GPU parity of Dual Chunk Attention (dca_attn_prefill, dca_attn_decode) against the CPU oracle
(oracle.dca).

The cache is filled through kv_append_circular with every kv head a full head; the three query sets
and the per-row mscale are seeded. Bar: max abs error <= 2e-2 (bf16 / fp16) against fp64. Pools
start filled with NaN, so any slot the kernel must not read is poisoned.
"""
import os

import numpy as np
import pytest
import torch

import kv_cache_sparsity_amd as duo
import oracle
import synth
from tests.gpu_harness import Cache, check_close, logical_kv, say, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(duo.LIB_PATH):
        pytest.fail("libduoattn.so is not built; the GPU tests need the HIP library")


def _queries(w, call, q_len):
    """q, q_succ, q_inter as storage bits and mscale float32 for one call."""
    qs = [synth.f32_to_storage(synth.queries(w, 3 * call + k, q_len=q_len), w.dtype)
          for k in range(3)]
    return qs, synth.row_scales(w, call, q_len)


def _run_dca(cache, qs, ms, chunk_len, ws=None):
    w = cache.w
    q, q_succ, q_inter = (to_dev(x, w.dtype) for x in qs)
    out = torch.empty_like(q)
    if ws is None:
        ws = duo.dca_prefill_workspace(q, cache.table)
    duo.dca_attn_prefill(q, q_succ, q_inter, torch.from_numpy(ms).cuda(), chunk_len, cache.k_pool,
                         cache.v_pool, cache.table, cache.lens, w.scale, out, ws)
    return out


CASES = [
    # one chunk of 300 rows from position 0: all three kinds, wave rows aligned to the chunks
    dict(name="bf16-d128-gqa2-c64-q300", dtype=synth.BF16, head_dim=128, group=2, kv=2,
         block_size=16, chunk_len=64, chunks=[300]),
    # second call's rows start at 200: chunk boundaries fall inside waves (per-lane query kinds)
    dict(name="f16-d64-mha-c128-q200+333", dtype=synth.F16, head_dim=64, group=1, kv=3,
         block_size=16, chunk_len=128, chunks=[200, 333]),
    # long key range (split workgroups), 64-slot pages
    dict(name="bf16-d128-mha-c256-bs64-800+700", dtype=synth.BF16, head_dim=128, group=1, kv=2,
         block_size=64, chunk_len=256, chunks=[800, 700]),
    # decode-like calls: 1 and 3 rows at the end of a long context, GQA 4
    dict(name="bf16-d64-gqa4-c64-777+1+3", dtype=synth.BF16, head_dim=64, group=4, kv=2,
         block_size=16, chunk_len=64, chunks=[777, 1, 3]),
    # one chunk covering everything: only the intra query is used
    dict(name="f16-d128-gqa2-c1024-q500", dtype=synth.F16, head_dim=128, group=2, kv=1,
         block_size=32, chunk_len=1024, chunks=[500]),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_dca_prefill_parity(case):
    say(f"dca {case['name']}")
    chunks = case["chunks"]
    total = sum(chunks)
    kv = case["kv"]
    w = synth.small(case["name"], batch=2, q_heads=kv * case["group"], kv_heads=kv,
                    head_dim=case["head_dim"], dtype=case["dtype"], block_size=case["block_size"],
                    sink=0, recent=1, retrieval=tuple(range(kv)), context=total,
                    q_len=max(chunks), seed=61)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, total, synth.S_K)
    V = logical_kv(w, total, synth.S_V)
    pos = 0
    for ci, n in enumerate(chunks):
        cache.append_logical(K, V, pos, pos + n)
        pos += n
        qs, ms = _queries(w, ci, n)
        got = to_host_f64(_run_dca(cache, qs, ms, case["chunk_len"]), w.dtype)
        want = oracle.attend_dca(*qs, K, V, np.full(w.batch, pos), ms,
                                 chunk_len=case["chunk_len"], scale=w.scale, dtype=w.dtype)
        check_close(got, want, w.dtype, f"{case['name']} call {ci}")


def test_dca_prefill_is_deterministic_and_reuses_its_workspace():
    w = synth.small("dca-det", batch=1, q_heads=4, kv_heads=2, head_dim=128, dtype=synth.BF16,
                    sink=0, recent=1, retrieval=(0, 1), context=600, q_len=600, seed=62)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, 600, synth.S_K)
    V = logical_kv(w, 600, synth.S_V)
    cache.append_logical(K, V, 0, 600)
    qs, ms = _queries(w, 0, 600)
    q = to_dev(qs[0], w.dtype)
    ws = duo.dca_prefill_workspace(q, cache.table)
    a = _run_dca(cache, qs, ms, 128, ws)
    b = _run_dca(cache, qs, ms, 128, ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_dca_qwen2_72b_tp4_share_last_chunk_row_tiles():
    """The Qwen2-72B one-GPU share (16 q / 2 kv heads, D 128, bf16, chunk_len 32768): the last
    32768-row chunk of a 131072-token context, at full size. Two rows of every 256-row tile (its
    first and a random one) are compared on every q head; the oracle takes a head's rows in blocks
    (oracle.attend_dca_rows)."""
    w = synth.qwen2_72b_dca_prefill()
    C, L, n = w.extra["chunk_len"], w.context, w.q_len
    say(f"dca {w.name}: filling {L} tokens")
    cache = Cache(w, fill="nan")
    K = logical_kv(w, L, synth.S_K)
    V = logical_kv(w, L, synth.S_V)
    cache.append_logical(K, V, 0, L)
    qs, ms = _queries(w, w.steps - 1, n)
    got = to_host_f64(_run_dca(cache, qs, ms, C), w.dtype)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(7)
    rows = np.array(sorted({r for t0 in range(0, n, 256)
                            for r in (t0, t0 + int(rng.integers(1, 256)))}), dtype=np.int64)
    errs = []
    for hq in range(w.num_q_heads):
        h = hq // w.group
        Kf = oracle.to_f64(K[0, h], w.dtype)
        Vf = oracle.to_f64(V[0, h], w.dtype)
        for r0 in range(0, len(rows), 64):
            r = rows[r0:r0 + 64]
            qv = tuple(oracle.to_f64(x[0, r, hq], w.dtype) for x in qs)
            want = oracle.attend_dca_rows(qv, L - n + r, Kf, Vf, C, w.scale, ms[0, r])
            errs.append(np.abs(got[0, r, hq] - want).max())
        say(f"  q head {hq}: {len(rows)} rows, max err so far {max(errs):.3e}")
    check_close(np.array([max(errs)]), np.zeros(1), w.dtype,
                f"{w.name} ({len(rows)} rows x {w.num_q_heads} q heads)")


# ------------------------------------------------------------------------------------------------
# dca_attn_decode
# ------------------------------------------------------------------------------------------------
def _fill_per_sequence(cache, K, V, lens):
    """Sequence b holds positions [0, lens[b]) (batch-1 appends on table row slices)."""
    w = cache.w
    final = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    for b in range(w.batch):
        L = int(lens[b])
        kn = np.ascontiguousarray(K[b:b + 1, :, :L].transpose(0, 2, 1, 3))
        vn = np.ascontiguousarray(V[b:b + 1, :, :L].transpose(0, 2, 1, 3))
        before = torch.zeros(1, dtype=torch.int32, device="cuda")
        after = torch.zeros(1, dtype=torch.int32, device="cuda")
        duo.kv_append_circular(cache.k_pool, cache.v_pool, cache.table[b:b + 1],
                               to_dev(kn, w.dtype), to_dev(vn, w.dtype), before, after,
                               cache.mask, w.sink, w.recent, w.ring_blocks)
        final[b] = after[0]
    cache.lens = final


def _run_dca_decode(cache, qs, ms, chunk_len, split_tokens=0):
    w = cache.w
    q, q_succ, q_inter = (to_dev(x, w.dtype) for x in qs)
    out = torch.empty_like(q)
    ws = duo.decode_workspace(q, cache.table, w.block_size, split_tokens)
    duo.dca_attn_decode(q, q_succ, q_inter, torch.from_numpy(ms).cuda(), chunk_len, cache.k_pool,
                        cache.v_pool, cache.table, cache.lens, w.scale, out, ws, split_tokens)
    return out


DECODE_CASES = [
    dict(name="bf16-d128-gqa4-c64", dtype=synth.BF16, head_dim=128, group=4, kv=2, block_size=16,
         chunk_len=64, lens=[1, 63, 64, 65, 1000], splits=[128, 0]),
    dict(name="f16-d64-mha-c256-bs64", dtype=synth.F16, head_dim=64, group=1, kv=3, block_size=64,
         chunk_len=256, lens=[300, 4000, 257], splits=[512, 0]),
    dict(name="bf16-d64-gqa16-c128", dtype=synth.BF16, head_dim=64, group=16, kv=1, block_size=16,
         chunk_len=128, lens=[129, 2500], splits=[256, 0]),
    dict(name="f16-d128-gqa24-c64", dtype=synth.F16, head_dim=128, group=24, kv=2, block_size=16,
         chunk_len=64, lens=[65, 1100], splits=[128, 0]),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c["name"] for c in DECODE_CASES])
def test_dca_decode_parity(case):
    say(f"dca decode {case['name']}")
    lens = np.asarray(case["lens"])
    kv = case["kv"]
    w = synth.small(case["name"], batch=len(lens), q_heads=kv * case["group"], kv_heads=kv,
                    head_dim=case["head_dim"], dtype=case["dtype"], block_size=case["block_size"],
                    sink=0, recent=1, retrieval=tuple(range(kv)), context=int(lens.max()),
                    q_len=1, seed=63)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, int(lens.max()), synth.S_K)
    V = logical_kv(w, int(lens.max()), synth.S_V)
    _fill_per_sequence(cache, K, V, lens)
    q4, ms = _queries(w, 0, 1)
    qs = [x[:, 0] for x in q4]
    want = oracle.attend_dca(*q4, K, V, lens, ms, chunk_len=case["chunk_len"], scale=w.scale,
                             dtype=w.dtype)[:, 0]
    for split in case["splits"]:
        got = to_host_f64(_run_dca_decode(cache, qs, ms[:, 0].copy(), case["chunk_len"], split),
                          w.dtype)
        check_close(got, want, w.dtype, f"{case['name']} split {split}")


def test_dca_decode_qwen2_72b_tp4_share():
    """Decode of the Qwen2-72B one-GPU share after the 131072-token context: batch 4, every row
    checked (chunk_len 32768, so each query meets all three kinds)."""
    w = synth.replace(synth.qwen2_72b_dca_prefill(), batch=4)
    C, L = w.extra["chunk_len"], w.context
    say(f"dca decode {w.name} batch 4: filling {L} tokens")
    cache = Cache(w, fill="nan")
    K = logical_kv(w, L, synth.S_K)
    V = logical_kv(w, L, synth.S_V)
    cache.append_logical(K, V, 0, L)
    q4, ms = _queries(w, 9, 1)
    got = to_host_f64(_run_dca_decode(cache, [x[:, 0] for x in q4], ms[:, 0].copy(), C), w.dtype)
    want = oracle.attend_dca(*q4, K, V, np.full(4, L), ms, chunk_len=C, scale=w.scale,
                             dtype=w.dtype)[:, 0]
    check_close(got, want, w.dtype, f"{w.name} decode")
