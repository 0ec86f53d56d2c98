"""C-ABI checks that need no GPU: the library loads, exports every function include/duo_attn.h
declares, and rejects invalid arguments with the documented status before any device work.

Each rejected call below is constructed so that validation fails; a call that passed validation
would launch a kernel, which these tests never do.
"""
import ctypes
import os
import re

import pytest

import kv_cache_sparsity_amd as duo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "duo_attn.h")

OK, INVALID, UNSUPPORTED, CAPACITY, WORKSPACE = 0, 1, 2, 3, 4

pytestmark = pytest.mark.skipif(not os.path.exists(duo.LIB_PATH),
                                reason="libduoattn.so not built (run __graft_entry__.build())")

FAKE = 0x100000  # a 4 KiB-aligned, never dereferenced address
MASK_RS = (ctypes.c_uint8 * 2)(1, 0)
MASK_R = (ctypes.c_uint8 * 2)(1, 1)
MASK_S = (ctypes.c_uint8 * 2)(0, 0)
MASK_BAD = (ctypes.c_uint8 * 2)(1, 2)


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:int32_t|size_t|const char\*)\s+(\w+)\(", text, flags=re.M)


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("kv_append_circular", "duo_attn_decode", "duo_attn_prefill"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = duo.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(duo.SYMBOLS) == set(declared_functions())


def test_version_and_status_strings():
    assert duo.abi_version() == 15
    with open(os.path.join(ROOT, "include", "duo_attn.h")) as fh:
        assert f"#define DUO_ATTN_ABI_VERSION {duo.abi_version()}" in fh.read()
    assert duo.status_string(0) == "ok"
    assert "capacity" in duo.status_string(3)
    assert duo.status_string(99) == "unknown status"


# ---- kv_append_circular --------------------------------------------------------------------------
def append(**kw):
    a = dict(k_pool=FAKE, v_pool=FAKE, table=FAKE, num_blocks=64, bs=16, mbph=8, k_new=FAKE,
             v_new=FAKE, lb=FAKE, la=FAKE + 256, batch=2, t_new=5, hkv=2, d=128, dtype=2,
             mask=ctypes.cast(MASK_RS, ctypes.c_void_p), sink=4, recent=16, rb=2)
    a.update(kw)
    return duo.lib().kv_append_circular(a["k_pool"], a["v_pool"], a["table"], a["num_blocks"],
                                        a["bs"], a["mbph"], a["k_new"], a["v_new"], a["lb"], a["la"],
                                        a["batch"], a["t_new"], a["hkv"], a["d"], a["dtype"],
                                        a["mask"], a["sink"], a["recent"], a["rb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k_pool=None), INVALID), (dict(v_new=None), INVALID), (dict(lb=None), INVALID),
    (dict(mask=None), INVALID), (dict(k_new=FAKE + 8), INVALID), (dict(la=FAKE), INVALID),
    (dict(batch=0), INVALID), (dict(t_new=0), INVALID), (dict(num_blocks=0), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED), (dict(bs=12), UNSUPPORTED),
    (dict(bs=512), UNSUPPORTED), (dict(hkv=65), UNSUPPORTED),
    (dict(mask=ctypes.cast(MASK_BAD, ctypes.c_void_p)), INVALID),
    (dict(sink=-1), INVALID), (dict(rb=0), INVALID), (dict(rb=8), CAPACITY),
])
def test_append_rejects(kw, status):
    assert append(**kw) == status


def test_append_ring_checks_skipped_without_streaming_heads():
    # all heads retrieval: ring arguments are not used, but other errors still surface
    assert append(mask=ctypes.cast(MASK_R, ctypes.c_void_p), rb=0, d=96) == UNSUPPORTED


# ---- decode ----------------------------------------------------------------------------------
def decode(**kw):
    a = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, table=FAKE, num_blocks=64, bs=16, mbph=20,
             lens=FAKE, batch=2, hq=8, hkv=2, d=128, dtype=2,
             mask=ctypes.cast(MASK_RS, ctypes.c_void_p), sink=4, recent=16, rb=2, scale=0.1,
             out=FAKE, ws=FAKE, ws_bytes=1 << 30, split=0)
    a.update(kw)
    return duo.lib().duo_attn_decode(a["q"], a["k_pool"], a["v_pool"], a["table"], a["num_blocks"],
                                     a["bs"], a["mbph"], a["lens"], a["batch"], a["hq"], a["hkv"],
                                     a["d"], a["dtype"], a["mask"], a["sink"], a["recent"], a["rb"],
                                     a["scale"], a["out"], a["ws"], a["ws_bytes"], a["split"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(table=FAKE + 2), INVALID),
    (dict(hq=6, hkv=4), INVALID), (dict(d=80), UNSUPPORTED),
    (dict(bs=8), UNSUPPORTED), (dict(bs=24), UNSUPPORTED), (dict(dtype=3), UNSUPPORTED),
    (dict(recent=0), INVALID), (dict(rb=0), INVALID), (dict(recent=33), CAPACITY),
    (dict(recent=-3), CAPACITY),            # three 16-position blocks > a ring of 32 slots
    (dict(recent=-2**31), CAPACITY),
    (dict(mbph=2, rb=2), CAPACITY), (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE),
    (dict(split=100), INVALID), (dict(split=-128), INVALID),
    (dict(mask=ctypes.cast(MASK_BAD, ctypes.c_void_p)), INVALID), (dict(batch=70000), UNSUPPORTED),
])
def test_decode_rejects(kw, status):
    assert decode(**kw) == status


# ---- fused append + decode ---------------------------------------------------------------------
LENS_AFTER = FAKE + 1024


def append_decode(**kw):
    a = dict(q=FAKE, k_new=FAKE + 4096, v_new=FAKE + 8192, k_pool=FAKE, v_pool=FAKE, table=FAKE,
             num_blocks=64, bs=16, mbph=20, before=FAKE, after=LENS_AFTER, batch=2, hq=8, hkv=2,
             d=128, dtype=2, mask=ctypes.cast(MASK_RS, ctypes.c_void_p), sink=4, recent=16, rb=2,
             scale=0.1, out=FAKE, ws=FAKE, ws_bytes=1 << 30, split=0)
    a.update(kw)
    return duo.lib().duo_attn_append_decode(
        a["q"], a["k_new"], a["v_new"], a["k_pool"], a["v_pool"], a["table"], a["num_blocks"],
        a["bs"], a["mbph"], a["before"], a["after"], a["batch"], a["hq"], a["hkv"], a["d"],
        a["dtype"], a["mask"], a["sink"], a["recent"], a["rb"], a["scale"], a["out"], a["ws"],
        a["ws_bytes"], a["split"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k_new=None), INVALID), (dict(v_new=FAKE + 2), INVALID),
    (dict(after=FAKE), INVALID),              # the new lengths may not overwrite the old ones
    (dict(after=FAKE + 2), INVALID),
    (dict(q=None), INVALID), (dict(d=80), UNSUPPORTED), (dict(bs=8), UNSUPPORTED),
    (dict(recent=33), CAPACITY), (dict(recent=0), INVALID), (dict(ws=None), WORKSPACE),
    (dict(mask=ctypes.cast(MASK_BAD, ctypes.c_void_p)), INVALID),
])
def test_append_decode_rejects(kw, status):
    assert append_decode(**kw) == status


def append_decode_int8(**kw):
    a = dict(q=FAKE, k_new=FAKE + 4096, v_new=FAKE + 8192, k_pool=FAKE, v_pool=FAKE,
             ks=FAKE + 12288, vs=FAKE + 16384, table=FAKE, num_blocks=64, bs=16, mbph=20,
             before=FAKE, after=LENS_AFTER, batch=2, hq=8, hkv=2, d=128, dtype=2,
             mask=ctypes.cast(MASK_RS, ctypes.c_void_p), sink=4, recent=16, rb=2, scale=0.1,
             out=FAKE, ws=FAKE, ws_bytes=1 << 30, split=0)
    a.update(kw)
    return duo.lib().duo_attn_append_decode_int8(
        a["q"], a["k_new"], a["v_new"], a["k_pool"], a["v_pool"], a["ks"], a["vs"], a["table"],
        a["num_blocks"], a["bs"], a["mbph"], a["before"], a["after"], a["batch"], a["hq"],
        a["hkv"], a["d"], a["dtype"], a["mask"], a["sink"], a["recent"], a["rb"], a["scale"],
        a["out"], a["ws"], a["ws_bytes"], a["split"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k_new=None), INVALID), (dict(ks=None), INVALID), (dict(vs=FAKE + 8), INVALID),
    (dict(after=FAKE), INVALID), (dict(d=80), UNSUPPORTED), (dict(recent=33), CAPACITY),
    (dict(ws=None), WORKSPACE),
])
def test_append_decode_int8_rejects(kw, status):
    assert append_decode_int8(**kw) == status


def append_decode_int4(**kw):
    a = dict(q=FAKE, k_new=FAKE + 4096, v_new=FAKE + 8192, k_pool=FAKE, v_pool=FAKE,
             ks=FAKE + 12288, vs=FAKE + 16384, table=FAKE, num_blocks=64, bs=16, mbph=20,
             before=FAKE, after=LENS_AFTER, batch=2, hq=8, hkv=2, d=128, dtype=2,
             mask=ctypes.cast(MASK_RS, ctypes.c_void_p), sink=4, recent=16, rb=2, scale=0.1,
             out=FAKE, ws=FAKE, ws_bytes=1 << 30, split=0)
    a.update(kw)
    return duo.lib().duo_attn_append_decode_int4(
        a["q"], a["k_new"], a["v_new"], a["k_pool"], a["v_pool"], a["ks"], a["vs"], a["table"],
        a["num_blocks"], a["bs"], a["mbph"], a["before"], a["after"], a["batch"], a["hq"],
        a["hkv"], a["d"], a["dtype"], a["mask"], a["sink"], a["recent"], a["rb"], a["scale"],
        a["out"], a["ws"], a["ws_bytes"], a["split"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(v_new=None), INVALID), (dict(ks=None), INVALID), (dict(after=FAKE), INVALID),
    (dict(dtype=0), UNSUPPORTED), (dict(d=80), UNSUPPORTED), (dict(recent=33), CAPACITY),
    (dict(ws=None), WORKSPACE),
])
def test_append_decode_int4_rejects(kw, status):
    assert append_decode_int4(**kw) == status


# ---- varlen prefill ---------------------------------------------------------------------------
def prefill_varlen(**kw):
    a = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, table=FAKE, num_blocks=64, bs=16, mbph=40, lens=FAKE,
             qs=FAKE + 512, batch=2, total=300, maxq=200, hq=8, hkv=2, d=128, dtype=2,
             mask=ctypes.cast(MASK_RS, ctypes.c_void_p), sink=4, recent=16, rb=16, scale=0.1,
             out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return duo.lib().duo_attn_prefill_varlen(
        a["q"], a["k_pool"], a["v_pool"], a["table"], a["num_blocks"], a["bs"], a["mbph"], a["lens"],
        a["qs"], a["batch"], a["total"], a["maxq"], a["hq"], a["hkv"], a["d"], a["dtype"], a["mask"],
        a["sink"], a["recent"], a["rb"], a["scale"], a["out"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qs=None), INVALID), (dict(qs=FAKE + 2), INVALID), (dict(total=0), INVALID),
    (dict(maxq=0), INVALID), (dict(q=None), INVALID), (dict(d=80), UNSUPPORTED),
    (dict(maxq=300), CAPACITY), (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE),
])
def test_prefill_varlen_rejects(kw, status):
    assert prefill_varlen(**kw) == status


# ---- int8 cache ------------------------------------------------------------------------------
def append_int8(**kw):
    a = dict(k_pool=FAKE, v_pool=FAKE, ks=FAKE + 4096, vs=FAKE + 8192, table=FAKE, num_blocks=64,
             bs=16, mbph=8, k_new=FAKE, v_new=FAKE, lb=FAKE, la=FAKE + 256, batch=2, t_new=5, hkv=2,
             d=128, dtype=2, mask=ctypes.cast(MASK_RS, ctypes.c_void_p), sink=4, recent=16, rb=2)
    a.update(kw)
    return duo.lib().kv_append_circular_int8(
        a["k_pool"], a["v_pool"], a["ks"], a["vs"], a["table"], a["num_blocks"], a["bs"], a["mbph"],
        a["k_new"], a["v_new"], a["lb"], a["la"], a["batch"], a["t_new"], a["hkv"], a["d"],
        a["dtype"], a["mask"], a["sink"], a["recent"], a["rb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), INVALID), (dict(vs=None), INVALID), (dict(ks=FAKE + 4), INVALID),
    (dict(vs=FAKE + 4096), INVALID), (dict(k_pool=None), INVALID), (dict(d=96), UNSUPPORTED),
    (dict(dtype=7), UNSUPPORTED), (dict(rb=8), CAPACITY),
])
def test_append_int8_rejects(kw, status):
    assert append_int8(**kw) == status


def decode_noalloc(**kw):
    a = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, table=FAKE, num_blocks=64, bs=16, mbph=20,
             lens=FAKE, batch=2, hq=8, hkv=2, d=128, dtype=2,
             mask=ctypes.cast(MASK_RS, ctypes.c_void_p), sink=4, recent=16, rb=2, scale=0.1,
             out=FAKE, split=0)
    a.update(kw)
    return duo.lib().duo_attn_decode_noalloc(
        a["q"], a["k_pool"], a["v_pool"], a["table"], a["num_blocks"], a["bs"], a["mbph"],
        a["lens"], a["batch"], a["hq"], a["hkv"], a["d"], a["dtype"], a["mask"], a["sink"],
        a["recent"], a["rb"], a["scale"], a["out"], a["split"], None)


MASK_64 = (ctypes.c_uint8 * 64)(*([1] * 64))


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(recent=33), CAPACITY),
    (dict(split=100), INVALID), (dict(mask=ctypes.cast(MASK_BAD, ctypes.c_void_p)), INVALID),
    # 64 sequences x 64 kv heads x 128-key splits over 1M slots: more than the scratch holds
    (dict(batch=64, hq=256, hkv=64, d=256, mbph=65540, split=128,
          mask=ctypes.cast(MASK_64, ctypes.c_void_p)), WORKSPACE),
])
def test_decode_noalloc_rejects(kw, status):
    """Every check runs before the call touches a device (this container has none)."""
    assert decode_noalloc(**kw) == status


def test_decode_noalloc_scratch_bounds_the_workspace_of_the_workloads():
    """The workloads' decode workspaces (library split, worst mask) fit the no-alloc scratch."""
    sizes = [duo.duo_attn_decode_workspace_size(8, 32, 8, 128, 2048, 16, 0),      # Llama-3-8B
             duo.duo_attn_decode_workspace_size(16, 8, 1, 256, 512, 16, 0),       # Gemma-2b
             duo.duo_attn_decode_workspace_size(1, 32, 8, 128, 65540, 16, 0),     # 1M context
             duo.duo_attn_decode_workspace_size(1, 16, 2, 128, 8192, 16, 0)]      # Qwen2-72B share
    assert all(0 < s <= duo.NOALLOC_SCRATCH_BYTES for s in sizes), sizes


def decode_int8(**kw):
    a = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, ks=FAKE + 4096, vs=FAKE + 8192, table=FAKE,
             num_blocks=64, bs=16, mbph=20, lens=FAKE, batch=2, hq=8, hkv=2, d=128, dtype=2,
             mask=ctypes.cast(MASK_RS, ctypes.c_void_p), sink=4, recent=16, rb=2, scale=0.1,
             out=FAKE, ws=FAKE, ws_bytes=1 << 30, split=0)
    a.update(kw)
    return duo.lib().duo_attn_decode_int8(
        a["q"], a["k_pool"], a["v_pool"], a["ks"], a["vs"], a["table"], a["num_blocks"], a["bs"],
        a["mbph"], a["lens"], a["batch"], a["hq"], a["hkv"], a["d"], a["dtype"], a["mask"],
        a["sink"], a["recent"], a["rb"], a["scale"], a["out"], a["ws"], a["ws_bytes"], a["split"],
        None)


@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), INVALID), (dict(vs=FAKE + 8), INVALID), (dict(q=None), INVALID),
    (dict(d=80), UNSUPPORTED), (dict(bs=8), UNSUPPORTED), (dict(recent=33), CAPACITY),
    (dict(ws=None), WORKSPACE), (dict(hq=6, hkv=4), INVALID),
])
def test_decode_int8_rejects(kw, status):
    assert decode_int8(**kw) == status


def test_decode_workspace_size_query():
    L = duo.lib()
    n = L.duo_attn_decode_workspace_size(8, 32, 8, 128, 2048, 16, 0)
    assert n > 0 and n % 4 == 0
    # a smaller split cannot need less workspace
    assert L.duo_attn_decode_workspace_size(8, 32, 8, 128, 2048, 16, 256) >= n
    assert L.duo_attn_decode_workspace_size(8, 32, 8, 96, 2048, 16, 0) == 0
    assert L.duo_attn_decode_workspace_size(8, 32, 6, 128, 2048, 16, 0) == 0
    assert L.duo_attn_decode_workspace_size(8, 32, 8, 128, 2048, 16, 100) == 0
    # one byte short of the query is rejected
    assert decode(ws_bytes=L.duo_attn_decode_workspace_size(2, 8, 2, 128, 20, 16, 0) - 1) == WORKSPACE


def test_decode_workspace_holds_two_level_merge_records():
    """Past 16 splits per row the decode merges in two levels: the workspace then holds, beside the
    tickets, every split's partial and one record per group of 16 splits (G x (D + 2) floats each)."""
    L = duo.lib()
    B, hq, hkv, D, mbph, bs = 6, 8, 2, 128, 320, 16          # 5120 keys of capacity
    G = hq // hkv
    rec = G * (D + 2) * 4
    for split, n_split in ((128, 40), (256, 20), (512, 10)):
        groups = -(-n_split // 16) if n_split > 16 else 0
        n = L.duo_attn_decode_workspace_size(B, hq, hkv, D, mbph, bs, split)
        assert n >= B * hkv * (n_split + groups) * rec + B * hkv * 4, (split, n)
    # the ticket region does not move with the split size: a smaller split only adds partials
    sizes = [L.duo_attn_decode_workspace_size(B, hq, hkv, D, mbph, bs, s) for s in (128, 256, 512)]
    assert sizes[0] > sizes[1] > sizes[2]


# ---- prefill ---------------------------------------------------------------------------------
def prefill(**kw):
    a = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, table=FAKE, num_blocks=64, bs=16, mbph=20,
             lens=FAKE, batch=1, q_len=32, hq=4, hkv=2, d=128, dtype=2,
             mask=ctypes.cast(MASK_RS, ctypes.c_void_p), sink=4, recent=16, rb=4, scale=0.1,
             out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return duo.lib().duo_attn_prefill(a["q"], a["k_pool"], a["v_pool"], a["table"],
                                      a["num_blocks"], a["bs"], a["mbph"], a["lens"], a["batch"],
                                      a["q_len"], a["hq"], a["hkv"], a["d"], a["dtype"], a["mask"],
                                      a["sink"], a["recent"], a["rb"], a["scale"], a["out"],
                                      a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(q_len=0), INVALID), (dict(lens=None), INVALID),
    (dict(d=256, dtype=0), UNSUPPORTED), (dict(d=32), UNSUPPORTED), (dict(bs=4), UNSUPPORTED),
    (dict(q_len=50), CAPACITY),            # ring of 64 slots < recent 16 + q_len 50 - 1
    (dict(recent=-3), CAPACITY),           # ring of 64 slots < 3 blocks of 16 + q_len 32 - 1
    (dict(recent=0), INVALID),
    (dict(rb=20), CAPACITY),               # 1 sink page + 20 ring pages > 20 table columns
])
def test_prefill_rejects(kw, status):
    assert prefill(**kw) == status


def test_prefill_workspace_size_query():
    L = duo.lib()
    rs = ctypes.cast(MASK_RS, ctypes.c_void_p)
    n = L.duo_attn_prefill_workspace_size(1, 32, 4, 2, 128, 2, rs)
    assert n > 0 and n % 4 == 0
    # more rows or more retrieval heads need more room; no retrieval head needs almost none
    assert L.duo_attn_prefill_workspace_size(1, 4096, 4, 2, 128, 2, rs) > n
    r_only = ctypes.cast(MASK_R, ctypes.c_void_p)
    assert L.duo_attn_prefill_workspace_size(1, 32, 4, 2, 128, 2, r_only) > n
    s_only = ctypes.cast(MASK_S, ctypes.c_void_p)
    assert L.duo_attn_prefill_workspace_size(1, 32, 4, 2, 128, 2, s_only) == 256
    # invalid sizes
    assert L.duo_attn_prefill_workspace_size(1, 0, 4, 2, 128, 2, rs) == 0
    assert L.duo_attn_prefill_workspace_size(1, 32, 4, 3, 128, 2, rs) == 0
    assert L.duo_attn_prefill_workspace_size(1, 32, 4, 2, 96, 2, rs) == 0
    assert L.duo_attn_prefill_workspace_size(1, 32, 4, 2, 128, 7, rs) == 0
    assert L.duo_attn_prefill_workspace_size(1, 32, 4, 2, 128, 2, None) == 0
    # a call with a missing or short workspace is rejected before anything is launched
    assert prefill(ws=None) == WORKSPACE
    assert prefill(ws_bytes=n - 1) == WORKSPACE


def test_all_retrieval_prefill_ignores_ring_geometry_but_checks_the_rest():
    mask = ctypes.cast(MASK_R, ctypes.c_void_p)
    assert prefill(mask=mask, rb=0, recent=0, d=96) == UNSUPPORTED


# ---- dca_attn_prefill ----------------------------------------------------------------------------
def dca(**kw):
    a = dict(q=FAKE, qs=FAKE, qi=FAKE, ms=FAKE, chunk=256, k_pool=FAKE, v_pool=FAKE, table=FAKE,
             num_blocks=64, bs=16, mbph=20, lens=FAKE, batch=1, q_len=32, hq=4, hkv=2, d=128,
             dtype=2, scale=0.1, out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return duo.lib().dca_attn_prefill(a["q"], a["qs"], a["qi"], a["ms"], a["chunk"], a["k_pool"],
                                      a["v_pool"], a["table"], a["num_blocks"], a["bs"], a["mbph"],
                                      a["lens"], a["batch"], a["q_len"], a["hq"], a["hkv"], a["d"],
                                      a["dtype"], a["scale"], a["out"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qs=None), INVALID), (dict(qi=None), INVALID), (dict(ms=None), INVALID),
    (dict(qi=FAKE + 8), INVALID), (dict(ms=FAKE + 2), INVALID), (dict(q=None), INVALID),
    (dict(chunk=0), INVALID), (dict(q_len=0), INVALID), (dict(lens=None), INVALID),
    (dict(hkv=0), INVALID), (dict(scale=0.0), INVALID), (dict(hq=5), INVALID),
    (dict(chunk=100), UNSUPPORTED), (dict(dtype=0), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(bs=8), UNSUPPORTED), (dict(hkv=65, hq=65), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=1024), WORKSPACE),
])
def test_dca_prefill_rejects(kw, status):
    assert dca(**kw) == status


def test_dca_workspace_is_the_all_retrieval_prefill_workspace():
    L = duo.lib()
    r_only = ctypes.cast(MASK_R, ctypes.c_void_p)
    n = L.dca_attn_prefill_workspace_size(1, 32, 4, 2, 128, 2)
    assert n == L.duo_attn_prefill_workspace_size(1, 32, 4, 2, 128, 2, r_only) > 256
    assert L.dca_attn_prefill_workspace_size(1, 32, 4, 0, 128, 2) == 0
    assert L.dca_attn_prefill_workspace_size(1, 32, 4, 65, 128, 2) == 0
    assert dca(ws_bytes=n - 1) == WORKSPACE


def dca_dec(**kw):
    a = dict(q=FAKE, qs=FAKE, qi=FAKE, ms=FAKE, chunk=256, k_pool=FAKE, v_pool=FAKE, table=FAKE,
             num_blocks=64, bs=16, mbph=20, lens=FAKE, batch=2, hq=8, hkv=2, d=128, dtype=2,
             scale=0.1, out=FAKE, ws=FAKE, ws_bytes=1 << 30, split=0)
    a.update(kw)
    return duo.lib().dca_attn_decode(a["q"], a["qs"], a["qi"], a["ms"], a["chunk"], a["k_pool"],
                                     a["v_pool"], a["table"], a["num_blocks"], a["bs"], a["mbph"],
                                     a["lens"], a["batch"], a["hq"], a["hkv"], a["d"], a["dtype"],
                                     a["scale"], a["out"], a["ws"], a["ws_bytes"], a["split"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qs=None), INVALID), (dict(qi=FAKE + 4), INVALID), (dict(ms=None), INVALID),
    (dict(chunk=-64), INVALID), (dict(q=None), INVALID), (dict(out=FAKE + 2), INVALID),
    (dict(batch=0), INVALID), (dict(hkv=0), INVALID), (dict(scale=-1.0), INVALID),
    (dict(split=100), INVALID),
    (dict(chunk=96), UNSUPPORTED), (dict(dtype=0), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(hq=34, hkv=4), INVALID),              # 34 q heads over 4 kv heads
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=64), WORKSPACE),
])
def test_dca_decode_rejects(kw, status):
    assert dca_dec(**kw) == status
