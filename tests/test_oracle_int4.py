"""Pins for the 4-bit cache oracle (oracle/quant4.py), on the CPU.

* hand-worked rows: ties round half to even, values past 7.5 steps saturate at +-7, a zero scale
  stores code 0;
* a hand-packed word and the byte order of the layout, and pack/unpack round trips;
* values on a power-of-two grid (k * s, s a power of two, |k| <= 7) come back exactly;
* attention over a 4-bit cache whose values sit on the grid equals oracle.attend over the values;
* the append places codes in the slots of the unquantized append and leaves other nibbles alone;
* planted mistakes (round half away from zero, clamp at +-8, the division in float64, halves of a
  word swapped) fail a pin.
"""
import numpy as np
import pytest

import oracle
from oracle import quant4 as oq4

F32, F16, BF16 = 0, 1, 2


def _f32(*v):
    return np.array(v, dtype=np.float32)


def test_hand_worked_row():
    # scale 0.5: x / s = 0.48, 0.5, 0.52, -1.5, 6.8, 7.2, 200, -200, 2.5, -0.5, 3.5, 0
    x = _f32(0.24, 0.25, 0.26, -0.75, 3.4, 3.6, 100.0, -100.0, 1.25, -0.25, 1.75, 0.0)
    s = np.full(12, 0.5, np.float32)
    got = oracle.quantize_rows4(x, s, F32)
    assert got.tolist() == [0, 0, 1, -2, 7, 7, 7, -7, 2, 0, 4, 0]


def test_zero_scale_channels_store_zero():
    x = _f32(1.0, -2.0, 3.0, 4.0)
    s = _f32(0.0, 1.0, 0.0, 2.0)
    assert oracle.quantize_rows4(x, s, F32).tolist() == [0, -2, 0, 2]


def test_division_is_one_rounded_fp32_division():
    # x / s is 5.49999989... exactly, which rounds to 5; its correctly rounded fp32 quotient is the
    # tie 5.5, which rounds half to even to 6
    x, s = _f32(3.1041348), _f32(0.56438816)
    assert float(x[0]) / float(s[0]) < 5.5 and x[0] / s[0] == np.float32(5.5)
    assert oracle.quantize_rows4(x, s, F32).tolist() == [6]


def test_bf16_inputs_are_upcast_exactly():
    bits = np.array([0x3F80, 0xC040, 0x4120], np.uint16)         # 1.0, -3.0, 10.0
    assert oracle.quantize_rows4(bits, _f32(1.0, 1.0, 1.0), BF16).tolist() == [1, -3, 7]


def test_hand_packed_word():
    # codes 1, -1, 2, -2, 3, -3, 7, -7 -> u = 9, 7, 10, 6, 11, 5, 15, 1; even elements (9, 10, 11,
    # 15) fill the low half lowest first: 0xFBA9; odd elements (7, 6, 5, 1) the high half: 0x1567
    got = oracle.pack4(np.array([1, -1, 2, -2, 3, -3, 7, -7]))
    assert got.tolist() == [0xA9, 0xFB, 0x67, 0x15]
    assert oracle.unpack4(got).tolist() == [1, -1, 2, -2, 3, -3, 7, -7]


def test_pack_unpack_round_trip_and_code_range():
    rng = np.random.default_rng(0)
    c = rng.integers(-7, 8, size=(3, 5, 64)).astype(np.int8)
    b = oracle.pack4(c)
    assert b.shape == (3, 5, 32) and b.dtype == np.uint8
    assert np.array_equal(oracle.unpack4(b), c)
    # every byte of every field is u in 1..15 (no code maps to 0)
    assert ((b & 15) >= 1).all() and ((b >> 4) >= 1).all()


@pytest.mark.parametrize("s", [0.25, 0.5, 2.0])
def test_grid_values_come_back_exactly(s):
    k = np.arange(-7, 8, dtype=np.float32)
    x = (k * np.float32(s)).astype(np.float32)
    codes = oracle.quantize_rows4(x, np.full(15, s, np.float32), F32)
    assert codes.tolist() == k.astype(int).tolist()
    assert np.array_equal(oracle.dequantize4(codes, np.full(15, s, np.float32)), x.astype(np.float64))


def test_error_is_at_most_half_a_step_inside_the_range():
    rng = np.random.default_rng(1)
    s = rng.uniform(0.1, 1.0, 32).astype(np.float32)
    x = (rng.uniform(-7.4, 7.4, (50, 32)) * s).astype(np.float32)
    got = oracle.dequantize4(oracle.quantize_rows4(x, s, F32), s)
    assert np.all(np.abs(got - x) <= 0.5 * s.astype(np.float64) * (1 + 1e-6))


def test_attention_over_grid_values_equals_attention_over_the_values():
    rng = np.random.default_rng(2)
    B, Hkv, G, L, D = 2, 2, 2, 40, 16
    ks = np.float32(2.0) ** rng.integers(-3, 0, (Hkv, D)).astype(np.float32)
    vs = np.float32(2.0) ** rng.integers(-3, 0, (Hkv, D)).astype(np.float32)
    kc = rng.integers(-7, 8, (B, Hkv, L, D)).astype(np.int8)
    vc = rng.integers(-7, 8, (B, Hkv, L, D)).astype(np.int8)
    K = (kc * ks[None, :, None, :]).astype(np.float32)
    V = (vc * vs[None, :, None, :]).astype(np.float32)
    q = rng.standard_normal((B, 3, Hkv * G, D)).astype(np.float32)
    lens, mask = np.array([40, 23]), np.array([1, 0], np.uint8)
    a = oracle.attend_int4(q, kc, vc, ks, vs, lens, mask, sink=3, recent=8, scale=0.3, dtype=F32)
    b = oracle.attend(q, K, V, lens, mask, sink=3, recent=8, scale=0.3, dtype=F32)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_append_places_codes_in_the_unquantized_slots_and_keeps_other_nibbles():
    rng = np.random.default_rng(3)
    B, Hkv, D, bs, ring, sink = 2, 2, 16, 16, 2, 5
    NB, mbph = 40, 8
    table = rng.permutation(NB)[:B * Hkv * mbph].reshape(B, Hkv, mbph).astype(np.int32)
    mask = np.array([1, 0], np.uint8)
    ks = rng.uniform(0.2, 0.6, (Hkv, D)).astype(np.float32)
    vs = rng.uniform(0.2, 0.6, (Hkv, D)).astype(np.float32)
    kshape, vshape = oracle.pool4_shapes(NB, bs, D)
    kp, vp = np.full(kshape, 0x55, np.uint8), np.full(vshape, 0x55, np.uint8)
    lens = np.zeros(B, np.int64)
    K = rng.standard_normal((B, 60, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((B, 60, Hkv, D)).astype(np.float32)
    for a, e in ((0, 7), (7, 30), (30, 31), (31, 60)):
        lens = oracle.append_int4(kp, vp, ks, vs, table, K[:, a:e], V[:, a:e], lens, mask, F32,
                                  sink=sink, block_size=bs, ring_blocks=ring, max_blocks_per_head=mbph)
    assert lens.tolist() == [60, 60]
    kcodes, vcodes = oracle.unpack4(kp), oracle.unpack4(vp)
    touched = np.zeros((NB, bs), bool)
    for b in range(B):
        for h in range(Hkv):
            ret = bool(mask[h])
            live = range(60) if ret else [t for t in range(60) if t < sink or t >= 60 - ring * bs]
            for t in live:
                blk, row = oracle.table_position(t, retrieval=ret, sink=sink, block_size=bs,
                                                 ring_blocks=ring)
                page = table[b, h, blk]
                touched[page, row] = True
                assert np.array_equal(kcodes[page, row], oracle.quantize_rows4(K[b, t, h], ks[h], F32))
                assert np.array_equal(vcodes[page, :, row], oracle.quantize_rows4(V[b, t, h], vs[h], F32))
    # slots never written keep the sentinel's fields (0x55: u = 5, code -3)
    assert (kcodes[~touched] == -3).all()
    assert (vcodes.transpose(0, 2, 1)[~touched] == -3).all()


# ---- planted mistakes ----------------------------------------------------------------------------
def _round_half_away(x, scales, dtype):
    xf = oracle.to_f64(x, dtype).astype(np.float32)
    s = np.asarray(scales, np.float32)
    q = (xf / np.where(s > 0, s, 1)).astype(np.float32)
    c = np.clip(np.sign(q) * np.floor(np.abs(q) + 0.5), -7, 7)
    return np.where(s > 0, c, 0).astype(np.int8)


def _divide_in_f64(x, scales, dtype):
    xf = oracle.to_f64(x, dtype)
    s = np.asarray(scales, np.float32).astype(np.float64)
    c = np.clip(np.rint(xf / np.where(s > 0, s, 1)), -7, 7)
    return np.where(s > 0, c, 0).astype(np.int8)


def _clamp_eight(x, scales, dtype):
    xf = oracle.to_f64(x, dtype).astype(np.float32)
    s = np.asarray(scales, np.float32)
    c = np.clip(np.rint((xf / np.where(s > 0, s, 1)).astype(np.float32)), -8, 7)
    return np.where(s > 0, c, 0).astype(np.int8)


def _pack_halves_swapped(codes):
    c = np.asarray(codes, dtype=np.int64)
    n = c.shape[-1]
    u = (c + 8).reshape(c.shape[:-1] + (n // 8, 8)).astype(np.uint32)
    word = np.zeros(u.shape[:-1], dtype=np.uint32)
    for i in range(4):
        word |= u[..., 2 * i + 1] << np.uint32(4 * i)
        word |= u[..., 2 * i] << np.uint32(16 + 4 * i)
    return np.ascontiguousarray(word.astype("<u4")).view(np.uint8).reshape(c.shape[:-1] + (n // 2,))


@pytest.mark.parametrize("name,fn,pin", [
    ("round_half_away", _round_half_away, test_hand_worked_row),
    ("clamp_eight", _clamp_eight, test_hand_worked_row),
    ("divide_in_f64", _divide_in_f64, test_division_is_one_rounded_fp32_division),
])
def test_planted_quantizer_mistakes_fail_a_pin(monkeypatch, name, fn, pin):
    monkeypatch.setattr(oq4, "quantize_rows4", fn)
    monkeypatch.setattr(oracle, "quantize_rows4", fn)
    with pytest.raises(AssertionError):
        pin()


def test_planted_packing_mistake_fails_a_pin(monkeypatch):
    monkeypatch.setattr(oq4, "pack4", _pack_halves_swapped)
    monkeypatch.setattr(oracle, "pack4", _pack_halves_swapped)
    with pytest.raises(AssertionError):
        test_hand_packed_word()
