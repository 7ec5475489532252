"""Pins for the rotation of head_dim values that are multiples of 64 but not
powers of two (velog.io post, section "application and background", admits
them; reading R23: block-diagonal normalized H_64), at d = 192."""

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import (block_hadamard, rotation_block, rotation_matrix, rotate_f32, unrotate_f32,
                    fwht_f32, hadamard_signs, OracleCache, decode_reference, bf16_round,
                    softmax_attention)


def test_blocks_and_rejections():
    assert [rotation_block(d) for d in (64, 128, 256, 192, 320, 384)] == [64, 128, 256, 64, 64, 64]
    for d in (96, 100):
        with pytest.raises(ValueError):
            rotation_block(d)


def test_block_matrix_is_scipy_block_diagonal():
    H64 = scipy.linalg.hadamard(64).astype(np.float64) / 8.0
    want = scipy.linalg.block_diag(H64, H64, H64)
    assert np.array_equal(block_hadamard(192), want)
    R = rotation_matrix(192, 5)
    assert np.allclose(R @ R.T, np.eye(192), atol=1e-14)
    assert np.array_equal(R, want * hadamard_signs(192, 5)[None, :])


def test_blockwise_fwht_is_exact_on_integers_and_matches_a_scalar_loop():
    rng = np.random.default_rng(0)
    x = rng.integers(-1000, 1000, (20, 192)).astype(np.float32)
    want = x.astype(np.int64) @ (scipy.linalg.block_diag(*[scipy.linalg.hadamard(64)] * 3)).T
    assert np.array_equal(fwht_f32(x, 64), want.astype(np.float32))
    # float inputs: bit-equal to a scalar loop over each group, h = 1..32
    y = rng.standard_normal(192).astype(np.float32)
    ref = [np.float32(v) for v in y]
    for g in range(3):
        h = 1
        while h < 64:
            for i in range(64 * g, 64 * g + 64):
                if (i - 64 * g) & h == 0:
                    a, b = ref[i], ref[i + h]
                    ref[i], ref[i + h] = np.float32(a + b), np.float32(a - b)
            h *= 2
    got = rotate_f32(y)
    assert np.array_equal(got, np.array(ref, np.float32) * np.float32(0.125))


def test_rotation_preserves_dot_products_and_inverts():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 192)).astype(np.float32)
    x[:, 100] *= 20
    y = rng.standard_normal((50, 192)).astype(np.float32)
    lhs = np.sum(rotate_f32(x).astype(np.float64) * rotate_f32(y), axis=1)
    rhs = np.sum(x.astype(np.float64) * y, axis=1)
    norm = np.linalg.norm(x, axis=1) * np.linalg.norm(y, axis=1)
    assert np.all(np.abs(lhs - rhs) <= 1e-5 * norm)
    s = hadamard_signs(192, 9)
    back = unrotate_f32(rotate_f32(x, signs=s), signs=s)
    assert np.allclose(back, x, rtol=0, atol=1e-5 * np.abs(x).max())


def test_d192_all_tail_is_textbook_attention():
    B, Hkv, Hq, d, n = 1, 2, 4, 192, 30
    rng = np.random.default_rng(4)
    k = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    cache = OracleCache(B, Hkv, d, 4, 5, tail_len=64, max_ctx=64)
    cache.append(k, v, [0], dtype="f32")
    out = decode_reference(cache.physical(), q, [n], Hkv, d, 4, 5, 64)
    H = torch.tensor(block_hadamard(d))
    for h in range(Hq):
        g = h // 2
        Kr = torch.tensor(bf16_round(rotate_f32(k[0, :, g])), dtype=torch.float64)
        Vr = torch.tensor(bf16_round(rotate_f32(v[0, :, g])), dtype=torch.float64)
        qr = H @ torch.tensor(q[0, h], dtype=torch.float64)
        o = torch.nn.functional.scaled_dot_product_attention(qr[None, None, None], Kr[None, None],
                                                             Vr[None, None])[0, 0, 0]
        assert np.allclose(out[0, h], (H @ o).numpy(), rtol=1e-12, atol=1e-12)


def test_d192_quantized_rotation_helps_on_outliers():
    rng = np.random.default_rng(2)
    n, d = 128, 192
    K = rng.standard_normal((n, d)).astype(np.float32)
    V = rng.standard_normal((n, d)).astype(np.float32)
    K[:, [5, 130]] *= 20
    V[:, [70]] *= 20
    q = rng.standard_normal(d)
    exact = softmax_attention(q, K, V, 1 / np.sqrt(d))
    errs = {}
    for rot in (True, False):
        c = OracleCache(1, 1, d, 4, 4, 0, n, rotate_k=rot, rotate_v=rot)
        c.append(K[None, :, None], V[None, :, None], [0], dtype="f32")
        out = decode_reference(c.physical(), q[None, None], [n], 1, d, 4, 4, 0,
                               rotate_k=rot, rotate_v=rot)
        errs[rot] = np.linalg.norm(out[0, 0] - exact) / np.linalg.norm(exact)
    assert errs[True] < 0.5 * errs[False]


@pytest.mark.parametrize("bits,minf", [(4, False), (5, False), (6, False), (8, False),
                                       (4, True), (5, True)])
def test_d192_planes_round_trip(bits, minf):
    # the code planes of d = 192 (row padding, 5/6-bit high words, V tiles
    # of 12 items per token) give back the blockwise-quantized rotated rows
    from oracle import (quantize_blocks, dequantize_blocks, quantize_blocks_min,
                        dequantize_blocks_min)
    from oracle.kvcache import dequantize_rows
    rng = np.random.default_rng(bits)
    n, d = 70, 192
    k = rng.standard_normal((1, n, 1, d)).astype(np.float32)
    v = (rng.standard_normal((1, n, 1, d)) + 1).astype(np.float32)
    c = OracleCache(1, 1, d, bits, bits, 0, n, k_min=minf, v_min=minf)
    c.append(k, v, [0], dtype="f32")
    ph = c.physical()
    for p, x in (("k", k), ("v", v)):
        xr = rotate_f32(x[0, :, 0]).reshape(n, d // 32, 32)
        if minf:
            want = dequantize_blocks_min(*quantize_blocks_min(xr, bits), bits).reshape(n, d)
        else:
            want = dequantize_blocks(*quantize_blocks(xr, bits)).reshape(n, d)
        got = dequantize_rows(ph[p + "_codes"][0, 0], ph[p + "_scales"][0, 0], d, bits, n, p, minf)
        assert np.array_equal(got, want), p
