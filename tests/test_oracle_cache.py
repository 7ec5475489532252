"""Pins for the oracle cache: append semantics, the bf16 precision tail
(aitrends.kr article 92204, glossary "Precision Tail": newest tokens kept in
bf16), chunk invariance and layout."""

import numpy as np
import pytest

from oracle import (OracleCache, rotate_f32, quantize_blocks, pack_rows,
                    bf16_round, f32_to_bf16_bits, dequantize_reference)
from oracle.kvcache import planes_to_rows, plane_codes
from oracle.blockquant import codes_to_vtiles, vtiles_to_codes, v_tile_bytes


def _data(B, n, H, d, seed=0):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, n, H, d)).astype(np.float32)
    v = rng.standard_normal((B, n, H, d)).astype(np.float32)
    k[..., 5] *= 20
    return k, v


def _same(a, b):
    pa, pb = a.physical(), b.physical()
    return all(np.array_equal(pa[key], pb[key]) for key in pa)


@pytest.mark.parametrize("T", (0, 8, 64))
@pytest.mark.parametrize("bits", ((4, 4), (8, 4), (5, 8), (6, 6)))
def test_chunk_invariance(T, bits):
    B, H, d, n = 2, 2, 64, 150
    k, v = _data(B, n, H, d, seed=T)
    one = OracleCache(B, H, d, bits[0], bits[1], T, 192)
    one.append(k, v, [0, 0], dtype="f32")
    step = OracleCache(B, H, d, bits[0], bits[1], T, 192)
    for i in range(n):
        step.append(k[:, i:i + 1], v[:, i:i + 1], [i, i], dtype="f32")
    assert _same(one, step)
    rng = np.random.default_rng(1)
    cuts = np.sort(rng.choice(np.arange(1, n), size=6, replace=False))
    rnd = OracleCache(B, H, d, bits[0], bits[1], T, 192)
    prev = 0
    for c in list(cuts) + [n]:
        rnd.append(k[:, prev:c], v[:, prev:c], [prev, prev], dtype="f32")
        prev = c
    assert _same(one, rnd)


def test_tail_holds_newest_tokens_in_bf16():
    B, H, d, n, T = 1, 2, 64, 100, 16
    k, v = _data(B, n, H, d, seed=3)
    c = OracleCache(B, H, d, 4, 4, T, 128)
    c.append(k, v, [0], dtype="f32")
    ph = c.physical()
    for p in range(n - T, n):
        want = f32_to_bf16_bits(rotate_f32(k[0, p]))
        assert np.array_equal(ph["k_tail"][0, :, p % T], want)
    # older tokens are quantized from the bf16-rounded rotated value
    rows = planes_to_rows(ph["k_codes"][0, 1], d, 4, n - T)
    codes, scales = quantize_blocks(bf16_round(rotate_f32(k[0, : n - T, 1])), 4)
    assert np.array_equal(rows, pack_rows(codes, 4))
    assert np.array_equal(ph["k_scales"][0, 1, : n - T], scales)


def test_no_tail_quantizes_float32_directly():
    B, H, d, n = 1, 1, 128, 64
    k, v = _data(B, n, H, d, seed=5)
    c = OracleCache(B, H, d, 8, 8, 0, 64)
    c.append(k, v, [0], dtype="f32")
    got = plane_codes(c.physical()["v_codes"][0, 0], d, 8, n, "v")
    codes, _ = quantize_blocks(rotate_f32(v[0, :, 0]), 8)
    assert np.array_equal(got, codes)


def test_bf16_input_widened_exactly():
    B, H, d, n = 1, 1, 64, 64
    k, v = _data(B, n, H, d, seed=6)
    kb, vb = f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    a = OracleCache(B, H, d, 4, 4, 0, 64)
    a.append(kb, vb, [0], dtype="bf16")
    b = OracleCache(B, H, d, 4, 4, 0, 64)
    b.append(bf16_round(k), bf16_round(v), [0], dtype="f32")
    assert _same(a, b)


def test_capacity_is_enforced():
    c = OracleCache(1, 1, 64, 4, 4, 0, 64)
    k, v = _data(1, 65, 1, 64)
    with pytest.raises(ValueError):
        c.append(k, v, [0], dtype="f32")


def test_dequantize_reference_spaces():
    B, H, d, n, T = 1, 2, 64, 80, 8
    k, v = _data(B, n, H, d, seed=8)
    c = OracleCache(B, H, d, 8, 8, T, 128)
    c.append(k, v, [0], dtype="f32")
    ph = c.physical()
    rot = dequantize_reference(ph, 0, 0, 0, n, n, H, d, 8, T, space=0)
    orig = dequantize_reference(ph, 0, 0, 0, n, n, H, d, 8, T, space=1)
    # rotated-space values are within half a quantization step of the rotated
    # input, and the tail rows are the exact bf16 values
    y = bf16_round(rotate_f32(k[0]))
    assert np.array_equal(rot[n - T:], y[n - T:])
    assert np.max(np.abs(rot - y)) < 0.05 * np.max(np.abs(y))
    # original space is the rotated value rotated again (H is its own inverse)
    assert np.array_equal(orig, rotate_f32(rot))
    assert np.max(np.abs(orig - k[0])) < 0.05 * np.max(np.abs(k[0]))


# ---------------------------------------------------------------- V tile layout
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [4, 5, 6, 8])
def test_v_tiles_round_trip_and_size(d, bits):
    qmax = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(d * 10 + bits)
    codes = rng.integers(-qmax, qmax + 1, size=(128, d)).astype(np.int8)
    plane = codes_to_vtiles(codes, bits)
    assert plane.size == 2 * v_tile_bytes(d, bits) == 2 * 64 * d * bits // 8
    assert np.array_equal(vtiles_to_codes(plane, 128, d, bits), codes)


def _one_code_plane(d, bits, t, e, c):
    codes = np.zeros((64, d), dtype=np.int8)
    codes[t, e] = c
    base = codes_to_vtiles(np.zeros((64, d), dtype=np.int8), bits)
    return codes_to_vtiles(codes, bits), base


def test_v_tile_positions_by_hand():
    # d = 64, token 9, element 20: half j = 0, lane group 1, slot 1; element
    # group 1, lane 16 + 4 = 20; item (0*64 + 20) * 4 + 1 = 81.
    # 4-bit: word 81, nibble 4*(1 % 2) + 1 // 2 = 4 -> byte 326, low nibble.
    plane, base = _one_code_plane(64, 4, 9, 20, 5)
    diff = np.nonzero(plane != base)[0]
    assert list(diff) == [326] and plane[326] == ((5 + 8) | (8 << 4))
    # 8-bit: byte 81*8 + 1 = 649 holds c + 128.
    plane, base = _one_code_plane(64, 8, 9, 20, -3)
    diff = np.nonzero(plane != base)[0]
    assert list(diff) == [649] and plane[649] == 125
    # 5-bit: u = 16 - 9 = 7 -> nibble 7 in byte 326 (low); its high bit (0,
    # where every zero code has 1) is bit 4 of byte 32*64 + 81 = 2129.
    plane, base = _one_code_plane(64, 5, 9, 20, -9)
    diff = np.nonzero(plane != base)[0]
    assert list(diff) == [326, 2129]
    assert plane[326] & 15 == 7 and base[2129] == 0xFF and plane[2129] == 0xEF
    # token 45 (j 1, lane group 1, slot 5), element 3 (group 0, lane 19):
    # item (64 + 19) * 4 + 0 = 332; 4-bit nibble 4*1 + 2 = 6 -> byte 1331, low.
    plane, base = _one_code_plane(64, 4, 45, 3, -7)
    diff = np.nonzero(plane != base)[0]
    assert list(diff) == [1331] and plane[1331] & 15 == 1
    # 6-bit, token 9 element 20 (item 81, slot 1, nibble 4): u = 32 + 21 = 53
    # = 0b110101 -> low nibble 5 in byte 326; bits 4-5 (0b11, where a zero
    # code has 0b10) at bits 2*4 = 8..9 of the 16-bit field 32*64 + 2*81 =
    # 2210, i.e. bits 0..1 of byte 2211
    plane, base = _one_code_plane(64, 6, 9, 20, 21)
    diff = np.nonzero(plane != base)[0]
    assert list(diff) == [326, 2211]
    assert plane[326] & 15 == 5 and base[2211] & 3 == 2 and plane[2211] & 3 == 3
