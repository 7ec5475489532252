"""Pins for the randomized-sign rotation R = H diag(s) (reading R21; the
velog.io post "fix KV cache quantization outliers" names random-sign variants
in section "application and background").

The sign sequence itself is a definition (SplitMix64 of seed * 2^32 + e) with
no external test vector in the pages: parity unpinned for the exact signs.
What the mathematics fixes is pinned: R is orthogonal for every sign vector,
the float32 forward / inverse pair undoes itself, attention is unchanged by
R, the signs are balanced, and rotation with signs still spreads outliers
(lower 4-bit error, section "Hadamard rotation")."""

import numpy as np

import workloads
from oracle import (hadamard, hadamard_signs, rotation_matrix, rotate_f32, unrotate_f32,
                    softmax_attention, quantize_blocks, dequantize_blocks, OracleCache,
                    dequantize_reference, decode_reference, splitmix64, bf16_round)


def test_seed_zero_is_plain_hadamard():
    assert hadamard_signs(128, 0) is None
    assert np.array_equal(rotation_matrix(128, 0), hadamard(128))
    x = np.random.default_rng(0).standard_normal((5, 128)).astype(np.float32)
    assert np.array_equal(rotate_f32(x, True, None), rotate_f32(x))


def test_signs_balanced_and_seed_dependent():
    seen = set()
    for seed in range(1, 21):
        s = hadamard_signs(256, seed)
        assert set(np.unique(s)) <= {-1.0, 1.0}
        neg = int(np.sum(s < 0))
        assert 80 <= neg <= 176, (seed, neg)          # binomial(256, 1/2) within 6 sigma
        seen.add(tuple(s))
    assert len(seen) == 20
    # the generator's top bit over many counters is unbiased
    tops = [splitmix64((7 << 32) | e) >> 63 for e in range(20000)]
    assert abs(sum(tops) - 10000) < 6 * 71


def test_rotation_matrix_orthogonal():
    for d in (64, 128, 256):
        for seed in (1, 99, 123456):
            R = rotation_matrix(d, seed)
            assert np.allclose(R @ R.T, np.eye(d), atol=1e-14)
            assert np.allclose(R, hadamard(d) @ np.diag(hadamard_signs(d, seed)), atol=0)


def test_float32_forward_and_inverse():
    rng = np.random.default_rng(3)
    for d in (64, 128, 256):
        s = hadamard_signs(d, 17)
        x = rng.standard_normal((20, d)).astype(np.float32)
        y = rotate_f32(x, True, s)
        ref = x.astype(np.float64) @ rotation_matrix(d, 17).T
        # first-order FWHT bound plus rounding of the scale and product
        bound = (np.log2(d) * 2.0 ** -23 * np.abs(x).sum(-1, keepdims=True) / np.sqrt(d)
                 + 2.0 ** -22 * np.abs(ref))
        assert np.all(np.abs(y - ref) <= bound)
        back = unrotate_f32(y, True, s)
        assert np.allclose(back, x, rtol=0, atol=1e-5 * np.abs(x).max())


def test_attention_invariant_under_signed_rotation():
    rng = np.random.default_rng(5)
    d = 128
    R = rotation_matrix(d, 4242)
    q = rng.standard_normal(d)
    K = rng.standard_normal((50, d))
    V = rng.standard_normal((50, d))
    ref = softmax_attention(q, K, V, 1 / np.sqrt(d))
    rot = R.T @ softmax_attention(R @ q, K @ R.T, V @ R.T, 1 / np.sqrt(d))
    assert np.linalg.norm(rot - ref) <= 1e-12 * np.linalg.norm(ref)


def test_signed_rotation_lowers_4bit_error_on_outliers():
    w = workloads.workload("tiny")
    for seed in range(5):
        rng = np.random.default_rng(seed)
        x = rng.standard_normal((w["n"], 64)).astype(np.float32)
        x[:, [3, 41]] *= 20
        s = hadamard_signs(64, 1000 + seed)
        plain = dequantize_blocks(*quantize_blocks(x, 4))
        back = unrotate_f32(dequantize_blocks(*quantize_blocks(rotate_f32(x, True, s), 4)), True, s)
        assert np.mean((back - x) ** 2) < 0.5 * np.mean((plain - x) ** 2)


def test_signed_cache_reads_back_and_attends():
    # all-tail cache: the stored rows are bf16(R x); reading back in the
    # original space returns x to bf16 precision, and decode attention equals
    # textbook attention on those rows
    B, Hkv, Hq, d, n, seed = 1, 2, 4, 64, 30, 77
    rng = np.random.default_rng(6)
    k = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    c = OracleCache(B, Hkv, d, 4, 4, 64, 64, sign_seed=seed)
    c.append(k, v, [0], dtype="f32")
    planes = c.physical()
    back = dequantize_reference(planes, 0, 0, 0, n, n, Hkv, d, 4, 64, 1, sign_seed=seed)
    assert np.allclose(back, k[0], rtol=0, atol=2e-2 * np.abs(k).max())
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    out = decode_reference(planes, q, [n], Hkv, d, 4, 4, 64, sign_seed=seed)
    s = hadamard_signs(d, seed)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        Kr = bf16_round(rotate_f32(k[0, :, g], True, s)).astype(np.float64)
        Vr = bf16_round(rotate_f32(v[0, :, g], True, s)).astype(np.float64)
        R = rotation_matrix(d, seed)
        ref = R.T @ softmax_attention(R @ q[0, h], Kr, Vr, 1 / np.sqrt(d))
        assert np.allclose(out[0, h], ref, rtol=1e-12, atol=1e-12)
