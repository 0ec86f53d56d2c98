"""The algorithmic units bench.py divides by (CPU): decode bytes and prefill FLOP.

The roofline fractions the bench reports are these counts over measured times, so they are pinned
here to something other than bench.py's own closed forms:

* small workloads counted pair by pair from the oracle's visible sets (oracle.visible_positions),
  with one block-table entry per page of a head's walk over those keys: the sink pages, then the
  ring's pages counted along the positions from the window's first key to its last (a window that
  wraps the ring reads the same entry once per pass, as the walk does), including windows that wrap;
* the totals quoted for the benchmark workloads (Llama-3-8B decode at 32768 tokens in three cache
  formats, the Llama-2-7B chunked prefill pass).
"""
import numpy as np
import pytest

import bench
import oracle
import synth


def _decode_bytes_by_pairs(w, lens):
    row = 2 * w.head_dim * w.elem_bytes
    total = 0
    for b in range(w.batch):
        L = int(lens[b])
        for h in range(w.num_kv_heads):
            ret = h in w.retrieval
            J = oracle.visible_positions(L - 1, retrieval=ret, sink=w.sink, recent=w.recent)
            bs = w.block_size
            walk = {("sink" if ret or t < w.sink else "ring",
                     t // bs if ret or t < w.sink else (t - w.sink) // bs) for t in J.tolist()}
            total += len(J) * row + 4 * len(walk)
    return total + 2 * w.batch * w.num_q_heads * w.head_dim * w.elem_bytes


@pytest.mark.parametrize("lens,sink,recent,bs", [
    ([1, 17, 200, 1000], 4, 24, 16),        # windows past the sinks, ring wrapped several times
    ([5, 64, 65, 333], 0, 64, 16),          # no sinks; a window of exactly four pages
    ([40, 41, 700, 2], 20, 100, 32),        # sink longer than some sequences
    ([300, 300], 16, 16, 16),               # window and sinks page-aligned
])
def test_decode_bytes_match_the_oracles_visible_keys_and_pages(lens, sink, recent, bs):
    w = synth.small("acct", batch=len(lens), q_heads=8, kv_heads=4, head_dim=64, dtype=synth.BF16,
                    block_size=bs, sink=sink, recent=recent, retrieval=(1, 2),
                    context=max(lens), q_len=1)
    lens = np.asarray(lens)
    assert bench.decode_bytes(w, lens) == _decode_bytes_by_pairs(w, lens)


def test_quantized_decode_bytes_differ_only_in_the_row_size():
    w = synth.small("acct-q", batch=3, q_heads=8, kv_heads=4, head_dim=128, dtype=synth.BF16,
                    block_size=16, sink=8, recent=40, retrieval=(0,), context=500, q_len=1)
    lens = np.array([500, 7, 120])
    keys = sum(len(oracle.visible_positions(int(L) - 1, retrieval=h in w.retrieval, sink=w.sink,
                                            recent=w.recent))
               for L in lens for h in range(w.num_kv_heads))
    plain = bench.decode_bytes(w, lens)
    # int8: 2 D one-byte codes and two fp32 scales per key instead of 2 D two-byte elements
    assert bench.decode_bytes(w, lens, int8_cache=True) == plain - keys * (2 * 128 * 2 - 2 * 128 - 8)
    # 4-bit: D bytes of codes per key, plus the per-channel K and V scales once per kv head
    assert bench.decode_bytes(w, lens, int4_cache=True) == (
        plain - keys * (2 * 128 * 2 - 128) + 2 * w.num_kv_heads * 128 * 4)


@pytest.mark.parametrize("L,q_len,sink,recent", [(300, 300, 8, 40), (700, 129, 0, 64), (64, 64, 100, 5)])
def test_prefill_flops_count_the_oracles_visible_pairs(L, q_len, sink, recent):
    w = synth.small("acct-p", batch=2, q_heads=6, kv_heads=3, head_dim=128, dtype=synth.BF16,
                    block_size=16, sink=sink, recent=recent, retrieval=(2,), context=L, q_len=q_len)
    pairs = sum(len(oracle.visible_positions(p, retrieval=(hq // w.group) in w.retrieval,
                                             sink=sink, recent=recent))
                for hq in range(w.num_q_heads) for p in range(L - q_len, L))
    assert bench.prefill_flops(w, L, q_len) == 4 * w.head_dim * pairs * w.batch


def test_benchmark_workload_totals():
    w = synth.llama3_8b_decode()
    lens = np.full(w.batch, w.context)
    assert bench.decode_bytes(w, lens) == 542_509_568
    assert bench.decode_bytes(w, lens, int8_cache=True) == 279_923_200
    assert bench.decode_bytes(w, lens, int4_cache=True) == 135_932_416
    wp = synth.llama2_7b_chunked_prefill()
    total = sum(bench.prefill_flops(wp, (c + 1) * wp.q_len, wp.q_len) for c in range(wp.steps))
    assert total == 2_654_800_183_296
