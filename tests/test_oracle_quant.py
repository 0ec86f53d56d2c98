"""Pins for the oracle's int8 KV cache (oracle/quant.py), each tied to something other than itself:

* rows worked by hand from the definition, including ties that round half to even;
* values on a power-of-two grid (code * 2^e, largest |code| = 127) come back exactly;
* closed-form bounds: the largest magnitude maps to +-127 and every value is reconstructed within
  half a quantization step (plus fp32 rounding);
* sign symmetry and all-zero rows;
* placement: the codes and scales land in the slots that the unquantized cache's append uses;
* attention over a cache whose values sit on the grid equals attention over the unquantized values;
* planted mistakes in a copy of the quantizer fail these pins.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import quant as oquant

F32, BF16 = 0, 2


def _row(vals):
    return np.asarray([vals], dtype=np.float32)


def test_hand_worked_rows():
    # amax 1: inv = 127; -0.5 * 127 = -63.5 rounds half to even -> -64; 0.25 * 127 = 31.75 -> 32
    codes, scales = oracle.quantize_rows(_row([1.0, -0.5, 0.25, 0.0]), F32)
    assert codes.tolist() == [[127, -64, 32, 0]]
    assert scales[0] == np.float32(1.0) / np.float32(127.0)
    # amax 127: inv = 1, so the codes are the values rounded half to even
    codes, scales = oracle.quantize_rows(_row([127.0, 2.5, 3.5, -2.5, -0.5, 0.5, -126.5]), F32)
    assert codes.tolist() == [[127, 2, 4, -2, 0, 0, -126]]
    assert scales[0] == np.float32(1.0)
    # amax 3: inv = fp32(127 / 3) = 42.33...; 1 -> 42 and both extremes -> +-127
    codes, _ = oracle.quantize_rows(_row([3.0, 1.0, -3.0]), F32)
    assert codes.tolist() == [[127, 42, -127]]


def test_grid_values_come_back_exactly():
    rng = np.random.default_rng(5)
    for e in (-9, -3, 0, 4):
        k = rng.integers(-127, 128, size=(64, 128))
        k[:, 0] = np.where(rng.random(64) < 0.5, 127, -127)
        x = (k * np.float32(2.0 ** e)).astype(np.float32)
        bits = synth.f32_to_storage(x, BF16)   # |k| <= 127 needs 7 bits: exact in bf16
        codes, scales = oracle.quantize_rows(bits, BF16)
        assert np.array_equal(codes.astype(np.int64), k)
        assert np.all(scales == np.float32(2.0 ** e))


def test_extremes_map_to_127_and_error_is_half_a_step():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((512, 128)) * rng.uniform(1e-3, 50, (512, 1))).astype(np.float32)
    bits = synth.f32_to_storage(x, BF16)
    xf = synth.storage_to_f32(bits, BF16).astype(np.float64)
    codes, scales = oracle.quantize_rows(bits, BF16)
    amax = np.abs(xf).max(axis=1)
    at_max = np.abs(xf) == amax[:, None]
    assert np.all(np.abs(codes[at_max].astype(np.int64)) == 127)
    assert np.all(np.abs(codes.astype(np.int64)) <= 127)
    err = np.abs(xf - oracle.dequantize(codes, scales))
    bound = 0.5 * scales.astype(np.float64)[:, None] * (1 + 1e-5) + 1e-6 * amax[:, None]
    assert np.all(err <= bound)


def test_sign_symmetry_and_zero_rows():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    x[3] = 0.0
    c1, s1 = oracle.quantize_rows(x, F32)
    c2, s2 = oracle.quantize_rows(-x, F32)
    assert np.array_equal(c2, -c1) and np.array_equal(s1, s2)
    assert not c1[3].any() and s1[3] == 0.0


def _small_cache(ret=(0,), T=(40, 1, 1, 9), ring_blocks=3, sink=5, bs=16, D=64, seed=8):
    """Append token batches into an int8 cache; returns what each call wrote, per position."""
    w = synth.small("q8-oracle", batch=2, q_heads=4, kv_heads=2, head_dim=D, dtype=BF16,
                    block_size=bs, sink=sink, recent=ring_blocks * bs - 8, retrieval=ret,
                    context=sum(T), q_len=1, seed=seed, ring_blocks=ring_blocks)
    table, nb = synth.block_table(w)
    ks, vs = oracle.pool_shapes(nb, bs, D)
    kp, vp = np.zeros(ks, np.int8), np.zeros(vs, np.int8)
    ksc = np.zeros(oracle.scale_pool_shape(nb, bs), np.float32)
    vsc = np.zeros_like(ksc)
    lens = np.zeros(w.batch, np.int64)
    K = {}
    for n in T:
        kn = synth.f32_to_storage(synth.kv_new(w, synth.S_K, int(lens[0]), int(lens[0]) + n), BF16)
        vn = synth.f32_to_storage(synth.kv_new(w, synth.S_V, int(lens[0]), int(lens[0]) + n), BF16)
        for i in range(n):
            K[int(lens[0]) + i] = (kn[:, i], vn[:, i])
        lens = oracle.append_int8(kp, vp, ksc, vsc, table, kn, vn, lens, w.retrieval_mask, BF16,
                                  sink=w.sink, block_size=bs, ring_blocks=ring_blocks,
                                  max_blocks_per_head=w.max_blocks_per_head)
    return w, table, (kp, vp, ksc, vsc), K, int(lens[0])


def test_int8_append_places_codes_and_scales_in_the_unquantized_slots():
    w, table, (kp, vp, ksc, vsc), K, L = _small_cache()
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            ret = bool(w.retrieval_mask[h])
            resident = oracle.visible_positions(L - 1, retrieval=ret, sink=w.sink,
                                                recent=w.ring_blocks * w.block_size)
            for t in resident:
                col, row = oracle.table_position(int(t), retrieval=ret, sink=w.sink,
                                                 block_size=w.block_size, ring_blocks=w.ring_blocks)
                page = table[b, h, col]
                kc, ks = oracle.quantize_rows(K[int(t)][0][b, h][None], BF16)
                vc, vs = oracle.quantize_rows(K[int(t)][1][b, h][None], BF16)
                assert np.array_equal(kp[page, row, :], kc[0]) and ksc[page, row] == ks[0]
                assert np.array_equal(vp[page, :, row], vc[0]) and vsc[page, row] == vs[0]


def test_attention_over_grid_values_equals_unquantized_attention():
    rng = np.random.default_rng(9)
    B, Hkv, G, D, L = 2, 2, 2, 64, 70
    def grid(shape):
        k = rng.integers(-127, 128, size=shape)
        k[..., 0] = 127
        s = 2.0 ** rng.integers(-8, -2, size=shape[:-1])
        return k.astype(np.int8), s.astype(np.float32), (k * s[..., None]).astype(np.float32)
    kc, ks, kx = grid((B, Hkv, L, D))
    vc, vs, vx = grid((B, Hkv, L, D))
    q = rng.standard_normal((B, 3, Hkv * G, D)).astype(np.float32)
    lens = np.array([L, 50])
    mask = np.array([1, 0], np.uint8)
    kw = dict(sink=4, recent=20, scale=0.125, dtype=F32)
    got = oracle.attend_int8(q, kc, ks, vc, vs, lens, mask, **kw)
    want = oracle.attend(q, kx, vx, lens, mask, **kw)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ---- planted mistakes: each must fail a pin -----------------------------------------------------
def _round_half_away(x, dtype):
    xf = oquant.to_f32(x, dtype)
    amax = np.abs(xf).max(axis=-1)
    inv = (np.float32(127) / amax).astype(np.float32)
    prod = xf * inv[..., None]
    return (np.sign(prod) * np.floor(np.abs(prod) + 0.5)).astype(np.int8), (amax / 127).astype(np.float32)


def _scale_over_128(x, dtype):
    xf = oquant.to_f32(x, dtype)
    amax = np.abs(xf).max(axis=-1)
    inv = (np.float32(128) / amax).astype(np.float32)
    return np.clip(np.rint(xf * inv[..., None]), -127, 127).astype(np.int8), (amax / 128).astype(np.float32)


@pytest.mark.parametrize("bug", [_round_half_away, _scale_over_128])
def test_planted_quantizer_bugs_are_caught(monkeypatch, bug):
    monkeypatch.setattr(oracle, "quantize_rows", bug)
    with pytest.raises(AssertionError):
        test_hand_worked_rows()
