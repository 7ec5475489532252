"""Pins for the oracle's block quantizer and code packing.

Byte counts: aiwitness.kr post 1txlhxu, table "Qwen 3.6 27B Q5_K_S + 64k
context KLD results" (cache size column).  Absmax scaling: velog.io post
"fix KV cache quantization outliers", section on why outliers ruin
quantization (the scale follows the extreme values of the group)."""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (QMAX, quantize_blocks, dequantize_blocks, pack_rows,
                    unpack_rows, row_bytes, rows_to_tiled, tiled_to_rows,
                    padded_row_bytes)
from oracle.blockquant import _hibit_position, _hi2_position

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BITS = (4, 5, 6, 8)


def _blocks(seed, nblk=400):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((nblk, 32)).astype(np.float32)
    x *= np.exp(rng.uniform(-12, 12, (nblk, 1))).astype(np.float32)
    x[::7, 5] *= 30                                  # outliers
    x[3] = 0                                         # zero block
    x[4] = np.float32(1e-30)                         # scale underflows to 0
    x[5, 0] = np.float32(3e6)                        # saturating scale
    x[6] = np.float32(2.0 ** -20) * rng.standard_normal(32).astype(np.float32)  # subnormal fp16 scale
    return x


@pytest.mark.parametrize("bits", BITS)
def test_codes_are_bruteforce_nearest_level(bits):
    x = _blocks(bits)
    codes, sbits = quantize_blocks(x, bits)
    qmax = QMAX[bits]
    s = sbits.view(np.float16).astype(np.float32)
    levels = np.arange(-qmax, qmax + 1)
    for i in range(x.shape[0]):
        if s[i, 0] == 0:
            assert np.all(codes[i] == 0)
            continue
        r = np.float32(1) / s[i, 0]
        for e in range(32):
            t = Fraction(float(np.float32(x[i, e] * r)))
            dist = [abs(t - L) for L in levels]
            best = min(dist)
            cands = [L for L, dd in zip(levels, dist) if dd == best]
            want = cands[0] if len(cands) == 1 else [L for L in cands if L % 2 == 0][0]
            assert codes[i, e] == want, (i, e)


@pytest.mark.parametrize("bits", BITS)
def test_scale_is_rounded_absmax_over_qmax(bits):
    x = _blocks(bits + 10)
    _, sbits = quantize_blocks(x, bits)
    s16 = sbits.view(np.float16)
    for i in range(x.shape[0]):
        a = Fraction(float(np.max(np.abs(x[i]))))
        target = min(a / QMAX[bits], Fraction(65504))
        got = Fraction(float(s16[i, 0]))
        # nearest fp16 to the (float32-rounded) quotient: neighbours are no closer
        slack = target * Fraction(1, 2 ** 23)
        up = np.nextafter(s16[i, 0], np.float16(np.inf))
        if np.isfinite(up):
            assert abs(got - target) <= abs(Fraction(float(up)) - target) + slack
        else:
            assert got == 65504
        dn = Fraction(float(np.nextafter(s16[i, 0], np.float16(0))))
        assert abs(got - target) <= abs(dn - target) + slack


@pytest.mark.parametrize("bits", BITS)
def test_reconstruction_error_and_full_range(bits):
    x = _blocks(bits + 20)
    codes, sbits = quantize_blocks(x, bits)
    xh = dequantize_blocks(codes, sbits)
    s = sbits.view(np.float16).astype(np.float64)
    qmax = QMAX[bits]
    for i in range(x.shape[0]):
        a = np.max(np.abs(x[i]))
        if s[i, 0] == 0 or a / qmax > 65504:
            continue
        xi = x[i].astype(np.float64)
        inside = np.abs(xi) <= (qmax + 0.5) * s[i, 0]
        # elements the grid covers are within half a step; the rest (possible
        # when a subnormal fp16 scale rounded down) clamp to +-qmax
        assert np.all(np.abs(xi - xh[i])[inside] <= s[i, 0] / 2 * (1 + 2.0 ** -10))
        assert np.all(codes[i][~inside] == np.sign(xi[~inside]) * qmax)
        if s[i, 0] >= 2.0 ** -14:                 # normal fp16 scale
            assert np.max(np.abs(codes[i])) == qmax
    assert np.all(np.abs(codes.astype(int)) <= qmax)


def test_textbook_absmax_when_scale_is_exact():
    # rotation off, scale a/qmax exactly representable: the quantizer is the
    # textbook x / scale rounded half-to-even
    rng = np.random.default_rng(0)
    for bits in BITS:
        qmax = QMAX[bits]
        for k in (-6, 0, 3):
            x = rng.uniform(-1, 1, (20, 32)).astype(np.float32) * np.float32(qmax * 2.0 ** k)
            x[:, 0] = np.float32(qmax * 2.0 ** k)
            codes, sbits = quantize_blocks(x, bits)
            assert np.all(sbits.view(np.float16).astype(np.float64) == 2.0 ** k)
            for v, c in zip(x.reshape(-1), codes.reshape(-1)):
                q = Fraction(float(v)) / Fraction(2) ** k
                fl = q.numerator // q.denominator
                rem = q - fl
                want = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
                assert c == want


@pytest.mark.parametrize("bits", BITS)
def test_pack_unpack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    qmax = QMAX[bits]
    for d in (64, 128, 256):
        c = rng.integers(-qmax, qmax + 1, size=(17, d)).astype(np.int8)
        rows = pack_rows(c, bits)
        assert rows.shape == (17, row_bytes(d, bits))
        assert np.array_equal(unpack_rows(rows, bits, d), c)


def test_packing_byte_conventions():
    c = np.zeros(64, np.int8)
    c[0], c[1] = -7, 7
    r4 = pack_rows(c, 4)
    assert r4[0] == (1 | (15 << 4)) and np.all(r4[1:] == 0x88)
    r8 = pack_rows(c, 8)
    assert r8[0] == 0xF9 and r8[1] == 7
    # 5-bit: codes never produce the all-zero offset value, bit plane bijective
    assert sorted(_hibit_position(w) for w in range(32)) == list(range(32))
    c5 = np.full(64, -15, np.int8)
    r5 = pack_rows(c5, 5)
    assert np.all(r5[:32] == 0x11) and np.all(r5[32:] == 0)
    c5[:] = 15
    r5 = pack_rows(c5, 5)
    assert np.all(r5[:32] == 0xFF) and np.all(r5[32:] == 0xFF)
    # 6-bit: each high word holds the 2-bit fields of 16 elements, covering
    # its 32 bits once; extreme codes give 0x01/0x00 and 0xFF/0xFF bytes
    for word in (0, 1):
        bits_used = sorted(b for w in range(32) if w // 16 == word
                           for b in (_hi2_position(w), _hi2_position(w) + 1))
        assert bits_used == list(range(32))
    c6 = np.full(64, -31, np.int8)
    r6 = pack_rows(c6, 6)
    assert np.all(r6[:32] == 0x11) and np.all(r6[32:] == 0)
    c6[:] = 31
    r6 = pack_rows(c6, 6)
    assert np.all(r6[:32] == 0xFF) and np.all(r6[32:] == 0xFF)
    # element 17 of block 1 (code 31 - 32 + 48 = u 47 = 0b101111): nibble 15,
    # bits 4-5 = 0b10 at bits 8*0 + 4*0 + 2*1 = 2..3 of word 1 of block 1
    c6[:] = 0
    c6[32 + 17] = 15
    r6 = pack_rows(c6, 6)
    w = r6[32:].view("<u4")
    assert (w[2 * 1 + 1] >> 2) & 3 == ((15 + 32) >> 4) & 3


def test_tiled_layout_positions():
    d, bits = 128, 8
    pad = padded_row_bytes(d, bits)
    rows = np.random.default_rng(1).integers(0, 256, (128, pad), dtype=np.uint8)
    plane = rows_to_tiled(rows, pad)
    for t in (0, 1, 63, 64, 100, 127):
        for c in range(pad // 16):
            off = (t // 64) * 64 * pad + (c * 64 + t % 64) * 16
            assert np.array_equal(plane[off:off + 16], rows[t, c * 16:(c + 1) * 16])
    assert np.array_equal(tiled_to_rows(plane, 128, pad, pad), rows)


def _golden_percent():
    out = {}
    with open(os.path.join(GOLDEN, "page3_cache_size_percent.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, pct = line.split()
                out[name] = float(pct)
    return out


def test_block_bytes_match_page3_cache_sizes():
    bits_of = {"q4_0": 4, "q5_0": 5, "q6_0": 6, "q8_0": 8, "q5_1": 5}
    table = _golden_percent()
    assert table.pop("bf16") == 100.0
    for name, pct in table.items():
        parts = name.split("-")
        k, v = parts[0], parts[-1]
        # one 32-element block: packed codes plus a 2-byte scale (and a 2-byte
        # minimum for the _1 formats), vs 64 bytes of bf16
        per = [Fraction(row_bytes(32, bits_of[p]) + (4 if p.endswith("_1") else 2), 64) * 100
               for p in (k, v)]
        mean = sum(per) / 2
        # the table prints one decimal, rounding halves up (q5_0-q4_0: 31.25 -> 31.3)
        assert int(mean * 10 + Fraction(1, 2)) == round(pct * 10), name
