"""GPU parity for the 4-bit cache, through the C ABI, against the CPU oracle on the same seeded bits.

* kv_append_circular_int4: whole byte pools bit-exact against oracle.append_int4. The pools start
  filled with a sentinel byte, so a nibble written that should not be, or missed, shows. Calls longer
  than the ring wrap it, and some start the surviving window inside a 16-slot run, so two
  workgroups of one call share V words.
* duo_attn_decode_int4: max abs error within 2e-2 of oracle.attend_int4 over the codes the oracle's
  quantizer gives for the same rows and the same per-channel scales.
"""
import os

import numpy as np
import pytest
import torch

import kv_cache_sparsity_amd as duo
import oracle
import synth
from tests.gpu_harness import check_close, logical_kv, q_decode, say, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

SENTINEL = 0x55


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(duo.LIB_PATH):
        pytest.fail("libduoattn.so is not built; the GPU tests need the HIP library")


class Int4Cache:
    """Device 4-bit pools + per-channel scales + block table, filled by kv_append_circular_int4."""

    def __init__(self, w: synth.Workload, mask=None):
        self.w = w
        self.mask = np.asarray(mask if mask is not None else w.retrieval_mask, dtype=np.uint8)
        self.table_h, self.num_blocks = synth.block_table(w)
        self.table = torch.from_numpy(self.table_h).cuda()
        ks, vs = oracle.pool4_shapes(self.num_blocks, w.block_size, w.head_dim)
        self.k_pool = torch.full(ks, SENTINEL, dtype=torch.uint8, device="cuda")
        self.v_pool = torch.full(vs, SENTINEL, dtype=torch.uint8, device="cuda")
        self.ks_h = synth.channel_scales(w, synth.S_K)
        self.vs_h = synth.channel_scales(w, synth.S_V)
        self.k_scale = torch.from_numpy(self.ks_h).cuda()
        self.v_scale = torch.from_numpy(self.vs_h).cuda()
        self.lens = torch.zeros(w.batch, dtype=torch.int32, device="cuda")

    def append(self, kn_bits, vn_bits, table=None, before=None):
        w = self.w
        before = self.lens if before is None else before
        after = torch.empty_like(before)
        duo.kv_append_circular_int4(self.k_pool, self.v_pool, self.k_scale, self.v_scale,
                                    self.table if table is None else table,
                                    to_dev(kn_bits, w.dtype), to_dev(vn_bits, w.dtype), before,
                                    after, self.mask, w.sink, w.recent, w.ring_blocks)
        return after

    def fill_per_sequence(self, K, V, lens, chunk=8192):
        final = torch.zeros(self.w.batch, dtype=torch.int32, device="cuda")
        for b in range(self.w.batch):
            L = int(lens[b])
            before = torch.zeros(1, dtype=torch.int32, device="cuda")
            for s in range(0, L, chunk):
                e = min(L, s + chunk)
                kn = np.ascontiguousarray(K[b:b + 1, :, s:e].transpose(0, 2, 1, 3))
                vn = np.ascontiguousarray(V[b:b + 1, :, s:e].transpose(0, 2, 1, 3))
                before = self.append(kn, vn, table=self.table[b:b + 1], before=before)
            final[b] = before[0] if L > 0 else 0
        self.lens = final

    def decode(self, q_bits, split_tokens=0):
        w = self.w
        q = to_dev(q_bits, w.dtype)
        out = torch.empty_like(q)
        ws = duo.decode_workspace(q, self.table, w.block_size, split_tokens)
        duo.duo_attn_decode_int4(q, self.k_pool, self.v_pool, self.k_scale, self.v_scale,
                                 self.table, self.lens, self.mask, w.sink, w.recent, w.ring_blocks,
                                 w.scale, out, ws, split_tokens)
        return out

    def logical_codes(self, K, V):
        """The oracle's codes of logical storage K, V [B][Hkv][L][D], per kv head."""
        w = self.w
        kc = np.stack([np.stack([oracle.quantize_rows4(K[b, h], self.ks_h[h], w.dtype)
                                 for h in range(w.num_kv_heads)]) for b in range(w.batch)])
        vc = np.stack([np.stack([oracle.quantize_rows4(V[b, h], self.vs_h[h], w.dtype)
                                 for h in range(w.num_kv_heads)]) for b in range(w.batch)])
        return kc, vc


APPEND_CASES = [
    # ring of 32 slots; the 70-token call wraps it twice and its window starts mid-run
    dict(name="bf16-d128-bs16-sink4-ring2", dtype=synth.BF16, head_dim=128, block_size=16, sink=4,
         recent=24, ring_blocks=2, kv=3, ret=(0,), calls=[5, 40, 1, 1, 70, 3]),
    dict(name="f16-d64-bs32-sink0-ring1", dtype=synth.F16, head_dim=64, block_size=32, sink=0,
         recent=20, ring_blocks=1, kv=2, ret=(1,), calls=[33, 2, 64, 7, 45]),
    dict(name="f16-d256-bs16-sink20-ring3", dtype=synth.F16, head_dim=256, block_size=16, sink=20,
         recent=40, ring_blocks=3, kv=2, ret=(), calls=[1, 19, 3, 100, 16, 57]),
    dict(name="bf16-d64-bs64-sink9-ring2", dtype=synth.BF16, head_dim=64, block_size=64, sink=9,
         recent=70, ring_blocks=2, kv=2, ret=(0,), calls=[17, 3, 130, 1, 200]),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[c["name"] for c in APPEND_CASES])
def test_append_int4_bit_exact(case):
    say(f"append int4 {case['name']}")
    total = sum(case["calls"])
    w = synth.small(case["name"], batch=2, q_heads=case["kv"], kv_heads=case["kv"],
                    head_dim=case["head_dim"], dtype=case["dtype"], block_size=case["block_size"],
                    sink=case["sink"], recent=case["recent"], retrieval=case["ret"], context=total,
                    q_len=1, seed=55, ring_blocks=case["ring_blocks"])
    cache = Int4Cache(w)
    ks, vs = oracle.pool4_shapes(cache.num_blocks, w.block_size, w.head_dim)
    kp = np.full(ks, SENTINEL, np.uint8)
    vp = np.full(vs, SENTINEL, np.uint8)
    lens = np.zeros(w.batch, np.int64)
    pos = 0
    for n in case["calls"]:
        kn = synth.f32_to_storage(synth.kv_new(w, synth.S_K, pos, pos + n), w.dtype)
        vn = synth.f32_to_storage(synth.kv_new(w, synth.S_V, pos, pos + n), w.dtype)
        cache.lens = cache.append(kn, vn)
        lens = oracle.append_int4(kp, vp, cache.ks_h, cache.vs_h, cache.table_h, kn, vn, lens,
                                  cache.mask, w.dtype, sink=w.sink, block_size=w.block_size,
                                  ring_blocks=w.ring_blocks,
                                  max_blocks_per_head=w.max_blocks_per_head)
        pos += n
        torch.cuda.synchronize()
        assert np.array_equal(cache.lens.cpu().numpy(), lens)
        assert cache.k_pool.cpu().numpy().tobytes() == kp.tobytes(), f"K pool after {pos} tokens"
        assert cache.v_pool.cpu().numpy().tobytes() == vp.tobytes(), f"V pool after {pos} tokens"


DECODE_CASES = [
    dict(name="bf16-d128-gqa4", dtype=synth.BF16, head_dim=128, group=4, kv=2, ret=(1,),
         block_size=16, sink=4, recent=64, lens=[700, 333, 1]),
    dict(name="f16-d64-gqa2-bs64", dtype=synth.F16, head_dim=64, group=2, kv=3, ret=(0, 2),
         block_size=64, sink=9, recent=100, lens=[1, 1500]),
    dict(name="bf16-d256-gqa8-all-retrieval", dtype=synth.BF16, head_dim=256, group=8, kv=1,
         ret=(0,), block_size=16, sink=0, recent=16, lens=[1024, 77, 3000]),
    dict(name="f16-d128-mha-bs32-streaming", dtype=synth.F16, head_dim=128, group=1, kv=4,
         ret=(), block_size=32, sink=30, recent=50, lens=[2000, 31, 80]),
    dict(name="bf16-d128-gqa16", dtype=synth.BF16, head_dim=128, group=16, kv=2, ret=(0,),
         block_size=16, sink=16, recent=256, lens=[5000, 4097]),
    dict(name="f16-d64-gqa33", dtype=synth.F16, head_dim=64, group=33, kv=1, ret=(0,),
         block_size=16, sink=0, recent=16, lens=[3000, 1]),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c["name"] for c in DECODE_CASES])
def test_decode_int4_parity(case):
    say(f"decode int4 {case['name']}")
    lens = np.asarray(case["lens"])
    Lmax = int(lens.max())
    w = synth.small(case["name"], batch=len(lens), q_heads=case["kv"] * case["group"],
                    kv_heads=case["kv"], head_dim=case["head_dim"], dtype=case["dtype"],
                    block_size=case["block_size"], sink=case["sink"], recent=case["recent"],
                    retrieval=case["ret"], context=Lmax, q_len=1, seed=56)
    cache = Int4Cache(w)
    K = logical_kv(w, Lmax, synth.S_K)
    V = logical_kv(w, Lmax, synth.S_V)
    cache.fill_per_sequence(K, V, lens)
    kc, vc = cache.logical_codes(K, V)
    q = q_decode(w, 0)
    want = oracle.attend_int4(q[:, None], kc, vc, cache.ks_h, cache.vs_h, lens, cache.mask,
                              sink=w.sink, recent=w.recent, scale=w.scale, dtype=w.dtype)[:, 0]
    for split in (0, 128, 1024):
        got = to_host_f64(cache.decode(q, split_tokens=split), w.dtype)
        check_close(got, want, w.dtype, f"{case['name']} split {split}")


def test_llama3_8b_gqa_decode_int4_batch8_ctx32768():
    w = synth.llama3_8b_decode()
    say(f"workload {w.name}, 4-bit cache")
    L = w.context
    cache = Int4Cache(w)
    K = logical_kv(w, L, synth.S_K)
    V = logical_kv(w, L, synth.S_V)
    cache.fill_per_sequence(K, V, np.full(w.batch, L))
    kc, vc = cache.logical_codes(K, V)
    q = q_decode(w, 0)
    got = to_host_f64(cache.decode(q), w.dtype)
    want = oracle.attend_int4(q[:, None], kc, vc, cache.ks_h, cache.vs_h, np.full(w.batch, L),
                              cache.mask, sink=w.sink, recent=w.recent, scale=w.scale,
                              dtype=w.dtype)[:, 0]
    check_close(got, want, w.dtype, w.name + " int4")
