"""The Python binding rejects tensors that do not match the call before any pointer reaches the
C ABI (CPU only: every check runs before the library is called, so CPU tensors suffice; a call
whose tensors are all well formed but on the CPU is refused for not being on a GPU)."""
import pytest
import torch

import kv_cache_sparsity_amd as duo

B, HQ, HKV, D, NB, BS, MB = 2, 4, 2, 64, 40, 16, 20


def _decode_args(**over):
    a = dict(q=torch.zeros(B, HQ, D, dtype=torch.bfloat16),
             k_pool=torch.zeros(NB, BS, D, dtype=torch.bfloat16),
             v_pool=torch.zeros(NB, D, BS, dtype=torch.bfloat16),
             block_table=torch.zeros(B, HKV, MB, dtype=torch.int32),
             seq_lens=torch.zeros(B, dtype=torch.int32), head_is_retrieval=[1, 0],
             sink_size=4, recent_size=16, ring_blocks=2, softmax_scale=0.125,
             out=torch.zeros(B, HQ, D, dtype=torch.bfloat16),
             workspace=torch.zeros(1024, dtype=torch.uint8))
    a.update(over)
    return a


DECODE_BAD = {
    "seq_lens int64": (dict(seq_lens=torch.zeros(B, dtype=torch.int64)), TypeError),
    "table int64": (dict(block_table=torch.zeros(B, HKV, MB, dtype=torch.int64)), TypeError),
    "table batch": (dict(block_table=torch.zeros(B + 1, HKV, MB, dtype=torch.int32)), ValueError),
    "seq_lens short": (dict(seq_lens=torch.zeros(B - 1, dtype=torch.int32)), ValueError),
    "mask short": (dict(head_is_retrieval=[1]), ValueError),
    "mask long": (dict(head_is_retrieval=[1, 0, 1]), ValueError),
    "mask value 2": (dict(head_is_retrieval=[2, 0]), ValueError),
    "k_pool dtype": (dict(k_pool=torch.zeros(NB, BS, D, dtype=torch.float16)), TypeError),
    "v_pool dtype": (dict(v_pool=torch.zeros(NB, D, BS, dtype=torch.float32)), TypeError),
    "v_pool token-major": (dict(v_pool=torch.zeros(NB, BS, D, dtype=torch.bfloat16)), ValueError),
    "out dtype": (dict(out=torch.zeros(B, HQ, D, dtype=torch.float16)), TypeError),
    "out small": (dict(out=torch.zeros(B, HQ - 1, D, dtype=torch.bfloat16)), ValueError),
    "head_dim": (dict(q=torch.zeros(B, HQ, 128, dtype=torch.bfloat16)), ValueError),
    "no workspace": (dict(workspace=None), ValueError),
}


@pytest.mark.parametrize("name", list(DECODE_BAD))
def test_decode_rejects(name):
    over, exc = DECODE_BAD[name]
    with pytest.raises(exc):
        duo.duo_attn_decode(**_decode_args(**over))


def test_decode_refuses_host_tensors():
    with pytest.raises(ValueError, match="GPU"):
        duo.duo_attn_decode(**_decode_args())


def _prefill_args(**over):
    a = dict(q=torch.zeros(B, 8, HQ, D, dtype=torch.float16),
             k_pool=torch.zeros(NB, BS, D, dtype=torch.float16),
             v_pool=torch.zeros(NB, D, BS, dtype=torch.float16),
             block_table=torch.zeros(B, HKV, MB, dtype=torch.int32),
             seq_lens=torch.zeros(B, dtype=torch.int32), head_is_retrieval=[0, 1],
             sink_size=4, recent_size=16, ring_blocks=2, softmax_scale=0.125,
             out=torch.zeros(B, 8, HQ, D, dtype=torch.float16), workspace=None)
    a.update(over)
    return a


@pytest.mark.parametrize("over,exc", [
    (dict(out=torch.zeros(B, 7, HQ, D, dtype=torch.float16)), ValueError),
    (dict(seq_lens=torch.zeros(B, dtype=torch.int64)), TypeError),
    (dict(head_is_retrieval=[0]), ValueError),
    (dict(k_pool=torch.zeros(NB, BS, D, dtype=torch.bfloat16)), TypeError),
])
def test_prefill_rejects(over, exc):
    with pytest.raises(exc):
        duo.duo_attn_prefill(**_prefill_args(**over))


def test_varlen_rejects_int64_offsets_and_short_tables():
    a = _prefill_args(q=torch.zeros(9, HQ, D, dtype=torch.float16),
                      out=torch.zeros(9, HQ, D, dtype=torch.float16))
    q_start = torch.tensor([0, 8, 9], dtype=torch.int64)
    with pytest.raises(TypeError):
        duo.duo_attn_prefill_varlen(a["q"], a["k_pool"], a["v_pool"], a["block_table"],
                                    a["seq_lens"], q_start, 8, a["head_is_retrieval"], 4, 16, 2,
                                    0.125, a["out"], None)
    with pytest.raises(ValueError):
        duo.duo_attn_prefill_varlen(a["q"], a["k_pool"], a["v_pool"],
                                    torch.zeros(B - 1, HKV, MB, dtype=torch.int32), a["seq_lens"],
                                    q_start.to(torch.int32), 8, a["head_is_retrieval"], 4, 16, 2,
                                    0.125, a["out"], None)


def test_append_rejects_mismatched_new_rows_and_mask():
    kp = torch.zeros(NB, BS, D, dtype=torch.bfloat16)
    vp = torch.zeros(NB, D, BS, dtype=torch.bfloat16)
    tab = torch.zeros(B, HKV, MB, dtype=torch.int32)
    lens = torch.zeros(B, dtype=torch.int32)
    kn = torch.zeros(B, 3, HKV, D, dtype=torch.bfloat16)
    with pytest.raises(TypeError):     # new rows of another dtype than the pools
        duo.kv_append_circular(kp, vp, tab, kn.half(), kn.half(), lens, None, [1, 0], 4, 16, 2)
    with pytest.raises(ValueError):    # v_new shorter than k_new
        duo.kv_append_circular(kp, vp, tab, kn, kn[:, :2].contiguous(), lens, None, [1, 0], 4, 16, 2)
    with pytest.raises(ValueError):    # mask shorter than num_kv_heads
        duo.kv_append_circular(kp, vp, tab, kn, kn, lens, None, [1], 4, 16, 2)
    with pytest.raises(TypeError):     # seq_lens_after int64
        duo.kv_append_circular(kp, vp, tab, kn, kn, lens, torch.zeros(B, dtype=torch.int64),
                               [1, 0], 4, 16, 2)
    with pytest.raises(ValueError, match="GPU"):
        duo.kv_append_circular(kp, vp, tab, kn, kn, lens, None, [1, 0], 4, 16, 2)


def test_int8_calls_reject_wrong_scale_pools():
    kp = torch.zeros(NB, BS, D, dtype=torch.int8)
    vp = torch.zeros(NB, D, BS, dtype=torch.int8)
    ks = torch.zeros(NB, BS, dtype=torch.float32)
    tab = torch.zeros(B, HKV, MB, dtype=torch.int32)
    lens = torch.zeros(B, dtype=torch.int32)
    q = torch.zeros(B, HQ, D, dtype=torch.bfloat16)
    ws = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(TypeError):
        duo.duo_attn_decode_int8(q, kp, vp, ks.half(), ks, tab, lens, [1, 0], 4, 16, 2, 0.1,
                                 q.clone(), ws)
    with pytest.raises(ValueError):
        duo.duo_attn_decode_int8(q, kp, vp, ks[:-1], ks, tab, lens, [1, 0], 4, 16, 2, 0.1,
                                 q.clone(), ws)
    with pytest.raises(TypeError):
        duo.duo_attn_decode_int8(q, kp.to(torch.uint8), vp, ks, ks, tab, lens, [1, 0], 4, 16, 2,
                                 0.1, q.clone(), ws)
    with pytest.raises(ValueError, match="GPU"):
        duo.duo_attn_decode_int8(q, kp, vp, ks, ks, tab, lens, [1, 0], 4, 16, 2, 0.1, q.clone(), ws)


def test_dca_rejects_wrong_mscale_and_query_sets():
    q = torch.zeros(B, 8, HQ, D, dtype=torch.bfloat16)
    kp = torch.zeros(NB, BS, D, dtype=torch.bfloat16)
    vp = torch.zeros(NB, D, BS, dtype=torch.bfloat16)
    tab = torch.zeros(B, HKV, MB, dtype=torch.int32)
    lens = torch.zeros(B, dtype=torch.int32)
    ms = torch.ones(B, 8, dtype=torch.float32)
    with pytest.raises(TypeError):
        duo.dca_attn_prefill(q, q, q, ms.double(), 64, kp, vp, tab, lens, 0.1, q.clone(), None)
    with pytest.raises(ValueError):
        duo.dca_attn_prefill(q, q[:, :7].contiguous(), q, ms, 64, kp, vp, tab, lens, 0.1,
                             q.clone(), None)
    with pytest.raises(ValueError):
        duo.dca_attn_decode(q[:, 0].contiguous(), q[:, 0].contiguous(), q[:, 0].contiguous(), ms,
                            64, kp, vp, tab, lens, 0.1, q[:, 0].contiguous(), torch.zeros(8))
