"""duo_attn_decode_noalloc: the decode without a workspace argument (the library's static per-GPU
scratch serves instead), through the C ABI, against duo_attn_decode with a caller-owned workspace
on the same inputs, and against the oracle. Two calls in a row, the second with a smaller input,
so the second finds the scratch as the first left it. Last, the call inside a captured HIP graph
(the callers it is for cannot allocate while capturing), replayed with eager work and a changed
query between replays, each replay checked against an eager call and the oracle."""
import os

import numpy as np
import pytest
import torch

import kv_cache_sparsity_amd as duo
import synth
from tests.gpu_harness import Cache, check_close, logical_kv, oracle_decode, q_decode, say, \
    to_dev, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(duo.LIB_PATH):
        pytest.fail("libduoattn.so is not built; the GPU tests need the HIP library")


CASES = [
    dict(name="bf16-d128-g4-b4", batch=4, q_heads=32, kv_heads=8, head_dim=128, dtype=synth.BF16,
         sink=64, recent=256, ret=(1, 2, 5, 7), lens=[9000, 4096, 17, 12000]),
    dict(name="f16-d64-g2-b2", batch=2, q_heads=4, kv_heads=2, head_dim=64, dtype=synth.F16,
         sink=4, recent=32, ret=(0,), lens=[700, 65]),
]


def _setup(case, seed):
    lens = np.asarray(case["lens"])
    Lmax = int(lens.max())
    w = synth.small(case["name"], batch=case["batch"], q_heads=case["q_heads"],
                    kv_heads=case["kv_heads"], head_dim=case["head_dim"], dtype=case["dtype"],
                    block_size=16, sink=case["sink"], recent=case["recent"], retrieval=case["ret"],
                    context=Lmax, seed=seed)
    cache = Cache(w, fill="nan")
    K = logical_kv(w, Lmax, synth.S_K)
    V = logical_kv(w, Lmax, synth.S_V)
    for b in range(w.batch):   # sequence b holds positions [0, lens[b])
        L = int(lens[b])
        kn = np.ascontiguousarray(K[b:b + 1, :, :L].transpose(0, 2, 1, 3))
        vn = np.ascontiguousarray(V[b:b + 1, :, :L].transpose(0, 2, 1, 3))
        z = torch.zeros(1, dtype=torch.int32, device="cuda")
        duo.kv_append_circular(cache.k_pool, cache.v_pool, cache.table[b:b + 1],
                               to_dev(kn, w.dtype), to_dev(vn, w.dtype), z, torch.empty_like(z),
                               cache.mask, w.sink, w.recent, w.ring_blocks)
    cache.set_lens(lens)
    return w, cache, K, V, lens


def test_noalloc_decode_matches_the_workspace_decode_on_two_calls():
    for i, case in enumerate(CASES):            # the second call has the smaller input
        say(f"noalloc decode call {i}: {case['name']}")
        w, cache, K, V, lens = _setup(case, 90 + i)
        q = q_decode(w, 0)
        ref = to_host_f64(cache.decode(q), w.dtype)
        qd = to_dev(q, w.dtype)
        out = torch.full_like(qd, float("nan"))
        duo.duo_attn_decode_noalloc(qd, cache.k_pool, cache.v_pool, cache.table, cache.lens,
                                    cache.mask, w.sink, w.recent, w.ring_blocks, w.scale, out)
        got = to_host_f64(out, w.dtype)
        check_close(got, ref, w.dtype, f"{case['name']}: noalloc vs workspace decode")
        check_close(got, oracle_decode(w, q, K, V, lens, cache.mask), w.dtype,
                    f"{case['name']}: noalloc vs oracle")


def test_noalloc_decode_repeats_with_explicit_splits():
    """Many splits per row (two-level merge) and again the library's split: the tickets the first
    call leaves are cleared or reused correctly by the next."""
    case = CASES[0]
    w, cache, K, V, lens = _setup(case, 95)
    q = q_decode(w, 1)
    want = oracle_decode(w, q, K, V, lens, cache.mask)
    qd = to_dev(q, w.dtype)
    for split in (128, 0, 256, 0):
        out = torch.full_like(qd, float("nan"))
        duo.duo_attn_decode_noalloc(qd, cache.k_pool, cache.v_pool, cache.table, cache.lens,
                                    cache.mask, w.sink, w.recent, w.ring_blocks, w.scale, out,
                                    split_tokens=split)
        check_close(to_host_f64(out, w.dtype), want, w.dtype, f"noalloc split {split}")


def test_noalloc_decode_replays_from_a_captured_graph():
    case = CASES[0]
    say(f"graph capture of the no-alloc decode {case['name']}")
    w, cache, K, V, lens = _setup(case, 81)
    queries = [q_decode(w, s) for s in range(3)]
    q = to_dev(queries[0], w.dtype)
    out = torch.empty_like(q)

    def call(stream=None):
        duo.duo_attn_decode_noalloc(q, cache.k_pool, cache.v_pool, cache.table, cache.lens,
                                    cache.mask, w.sink, w.recent, w.ring_blocks, w.scale, out,
                                    stream=stream)

    call()                      # first call on this device: the scratch address is looked up here
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(stream=side)       # a warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(stream=side)
    torch.cuda.synchronize()

    for rep, qi in enumerate([0, 0, 1, 2, 1]):
        q.copy_(to_dev(queries[qi], w.dtype))
        # eager reference on the same inputs, then unrelated eager work, then the replay
        call()
        torch.cuda.synchronize()
        eager = to_host_f64(out, w.dtype)
        out.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = to_host_f64(out, w.dtype)
        assert np.isfinite(got).all(), f"replay {rep}: non-finite output"
        err = float(np.abs(got - eager).max())
        say(f"  replay {rep} (query {qi}): max |replay - eager| = {err:.3e}; scratch {float(scratch):.1f}")
        assert err <= 1e-2
        check_close(got, oracle_decode(w, queries[qi], K, V, lens, cache.mask), w.dtype,
                    f"replay {rep}")
