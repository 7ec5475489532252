"""Pins for the scale-and-min blocks q4_1 / q5_1 (reading R22).  The cache
sizes the aiwitness.kr table prints for q5_1 are checked in
test_oracle_quant.py; here: brute-force nearest levels, the reconstruction
bound, the textbook case, chunk invariance and the asymmetric-range benefit."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import (quantize_blocks, dequantize_blocks, quantize_blocks_min,
                    dequantize_blocks_min, OracleCache, pack_rows, unpack_rows)


def _blocks(seed, nblk=300):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((nblk, 32)).astype(np.float32)
    x *= np.exp(rng.uniform(-8, 8, (nblk, 1))).astype(np.float32)
    x += rng.uniform(-3, 3, (nblk, 1)).astype(np.float32) * np.abs(x).max(axis=1, keepdims=True)
    x[3] = 0                                   # zero block
    x[4] = np.float32(1.5)                     # constant block: s = 0
    x[5, 0] = np.float32(1e6)                  # wide range
    return x


@pytest.mark.parametrize("bits", (4, 5))
def test_min_codes_are_nearest_levels(bits):
    x = _blocks(bits)
    codes, pairs = quantize_blocks_min(x, bits)
    u = codes.astype(int) + (1 << (bits - 1))
    pr = pairs.view(np.float16).astype(np.float32)
    umax = (1 << bits) - 1
    for i in range(x.shape[0]):
        s, m = pr[i, 0, 0], pr[i, 0, 1]
        if s == 0:
            assert np.all(u[i] == 0)
            continue
        r = np.float32(1) / s
        for e in range(32):
            t = Fraction(float(np.float32(np.float32(x[i, e] - m) * r)))
            dist = [abs(t - L) for L in range(umax + 1)]
            best = min(dist)
            cands = [L for L, dd in enumerate(dist) if dd == best]
            want = cands[0] if len(cands) == 1 else [L for L in cands if L % 2 == 0][0]
            assert u[i, e] == want, (i, e)


@pytest.mark.parametrize("bits", (4, 5))
def test_min_reconstruction_within_half_step(bits):
    x = _blocks(bits + 7)
    codes, pairs = quantize_blocks_min(x, bits)
    xh = dequantize_blocks_min(codes, pairs, bits)
    pr = pairs.view(np.float16).astype(np.float64)
    umax = (1 << bits) - 1
    for i in range(x.shape[0]):
        s, m = pr[i, 0, 0], pr[i, 0, 1]
        xi = x[i].astype(np.float64)
        if s == 0:
            assert np.all(xh[i] == np.float32(m))
            continue
        inside = (xi >= m - s / 2) & (xi <= m + (umax + 0.5) * s)
        tol = s / 2 * (1 + 2.0 ** -9) + 2.0 ** -22 * np.abs(xi)
        assert np.all(np.abs(xi - xh[i])[inside] <= tol[inside]), i
        # the block's extremes are represented (min at level 0 or 1 of the
        # rounded minimum, max near the top level)
        assert u_range_ok(codes[i], bits)


def u_range_ok(c, bits):
    u = c.astype(int) + (1 << (bits - 1))
    return u.min() >= 0 and u.max() <= (1 << bits) - 1


def test_min_textbook_when_exact():
    # lo and s exactly representable: u = round_half_even((x - lo) / s)
    rng = np.random.default_rng(1)
    for bits in (4, 5):
        umax = (1 << bits) - 1
        for s_exp in (-4, 0, 2):
            s = 2.0 ** s_exp
            lo = -3.0 * s
            u = rng.integers(0, umax + 1, (10, 32))
            frac = rng.choice([-0.5, -0.25, 0.0, 0.25, 0.5], (10, 32))
            x = (lo + np.clip(u + frac, 0, umax) * s).astype(np.float32)
            x[:, 0] = np.float32(lo)
            x[:, 1] = np.float32(lo + umax * s)
            codes, pairs = quantize_blocks_min(x, bits)
            pr = pairs.view(np.float16).astype(np.float64)
            assert np.all(pr[..., 0] == s) and np.all(pr[..., 1] == lo)
            got = codes.astype(int) + (1 << (bits - 1))
            q = (x.astype(np.float64) - lo) / s
            want = np.clip(np.round(q), 0, umax)           # numpy rounds halves to even
            assert np.array_equal(got, want)


def test_min_beats_symmetric_on_shifted_data():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((500, 32)) + 4.0).astype(np.float32)
    for bits in (4, 5):
        sym = dequantize_blocks(*quantize_blocks(x, bits))
        c, p = quantize_blocks_min(x, bits)
        asym = dequantize_blocks_min(c, p, bits)
        assert np.mean((asym - x) ** 2) < 0.5 * np.mean((sym - x) ** 2)


@pytest.mark.parametrize("T", [0, 8])
def test_min_chunk_invariance_and_storage(T):
    B, H, d = 1, 2, 64
    rng = np.random.default_rng(3 + T)
    k = (rng.standard_normal((B, 100, H, d)) + 2).astype(np.float32)
    v = (rng.standard_normal((B, 100, H, d)) - 1).astype(np.float32)
    one = OracleCache(B, H, d, 4, 5, T, 128, k_min=True, v_min=True)
    one.append(k, v, [0], dtype="f32")
    step = OracleCache(B, H, d, 4, 5, T, 128, k_min=True, v_min=True)
    n = 0
    for c in (1, 30, 7, 62):
        step.append(k[:, n:n + c], v[:, n:n + c], [n], dtype="f32")
        n += c
    a, b = one.physical(), step.physical()
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    assert a["k_scales"].shape[-1] == 2 * d // 32          # (s, m) pairs
    # codes hold u = c + 2^(b-1), packed like the symmetric formats
    c4 = np.array([[-8, 7] * 32], np.int8)
    assert np.array_equal(unpack_rows(pack_rows(c4, 4), 4, 64), c4)


def test_min_decode_is_attention_on_dequantized_rows():
    # decode through the planes equals softmax attention on rows quantized
    # block by block with the scale-and-min rule, taken back with H^T
    from oracle import hadamard, rotate_f32, softmax_attention, decode_reference
    B, Hkv, Hq, d, n = 1, 1, 2, 64, 70
    rng = np.random.default_rng(11)
    k = (rng.standard_normal((B, n, Hkv, d)) + 1.5).astype(np.float32)
    v = (rng.standard_normal((B, n, Hkv, d)) * 2 - 3).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    for kb, vb, km, vm in ((4, 5, True, True), (5, 8, True, False), (8, 4, False, True)):
        cache = OracleCache(B, Hkv, d, kb, vb, 0, 128, k_min=km, v_min=vm)
        cache.append(k, v, [0], dtype="f32")
        out = decode_reference(cache.physical(), q, [n], Hkv, d, kb, vb, 0, k_min=km, v_min=vm)

        def deq(x, bits, mf):
            xr = rotate_f32(x).reshape(n, d // 32, 32)
            if mf:
                return dequantize_blocks_min(*quantize_blocks_min(xr, bits), bits).reshape(n, d)
            return dequantize_blocks(*quantize_blocks(xr, bits)).reshape(n, d)
        K = deq(k[0, :, 0], kb, km).astype(np.float64)
        V = deq(v[0, :, 0], vb, vm).astype(np.float64)
        H = hadamard(d)
        for h in range(Hq):
            want = H.T @ softmax_attention(H @ q[0, h].astype(np.float64), K, V, 1 / np.sqrt(d))
            assert np.allclose(out[0, h], want, rtol=1e-12, atol=1e-12), (kb, vb, km, vm)
