"""Pins for the oracle's attention: rotation leaves attention unchanged
(velog.io post "fix KV cache quantization outliers", section "Hadamard
rotation"), rotation lowers low-bit error on outlier data (same section),
brute force on tiny inputs, and the textbook case with an all-bf16 cache."""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import (hadamard, rotate_f32, softmax_attention, OracleCache,
                    decode_reference, quantize_blocks, dequantize_blocks,
                    bf16_round)


def test_softmax_attention_bruteforce():
    rng = np.random.default_rng(0)
    q = rng.standard_normal(4)
    K = rng.standard_normal((5, 4))
    V = rng.standard_normal((5, 4))
    s = [0.5 * sum(q[i] * K[t, i] for i in range(4)) for t in range(5)]
    e = [math.exp(x) for x in s]
    want = [sum(e[t] * V[t, j] for t in range(5)) / sum(e) for j in range(4)]
    assert np.allclose(softmax_attention(q, K, V, 0.5), want, rtol=1e-13, atol=0)


def _tiny():
    w = workloads.workload("tiny")
    K = workloads.kv_numpy(w, 1, 0, w["n"])[0, :, 0]    # [n][d] fp32
    V = workloads.kv_numpy(w, 2, 0, w["n"])[0, :, 0]
    q = workloads.q_numpy(w)[0, 0]
    return w, K, V, q


def test_rotated_attention_equals_unrotated():
    w, K, V, q = _tiny()
    d = w["d"]
    H = hadamard(d)
    ref = softmax_attention(q, K, V, 1 / np.sqrt(d))
    rot = H @ softmax_attention(H @ q, K @ H.T, V @ H.T, 1 / np.sqrt(d))
    assert np.linalg.norm(rot - ref) <= 1e-12 * np.linalg.norm(ref)
    # float32 rotation as stored in the cache
    rot32 = rotate_f32(softmax_attention(rotate_f32(q), rotate_f32(K), rotate_f32(V),
                                         1 / np.sqrt(d)).astype(np.float32))
    assert np.linalg.norm(rot32 - ref) <= 1e-5 * np.linalg.norm(ref)


@pytest.mark.parametrize("seed", range(5))
def test_rotation_lowers_4bit_error_on_outliers(seed):
    w = workloads.workload("tiny")
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((w["n"], 64)).astype(np.float32)
    x[:, [3, 41]] *= 20
    plain = dequantize_blocks(*quantize_blocks(x, 4))
    rq = dequantize_blocks(*quantize_blocks(rotate_f32(x), 4))
    back = rotate_f32(rq)
    mse_plain = np.mean((plain - x) ** 2)
    mse_rot = np.mean((back - x) ** 2)
    assert mse_rot < 0.5 * mse_plain


def test_all_tail_cache_is_textbook_attention():
    # T >= n: nothing is quantized; the cache holds bf16(H k), bf16(H v) and
    # decode attention must equal textbook attention on those rows
    B, Hkv, Hq, d, n = 2, 2, 4, 64, 40
    rng = np.random.default_rng(4)
    k = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    cache = OracleCache(B, Hkv, d, 4, 4, tail_len=64, max_ctx=128)
    cache.append(k, v, [0, 0], dtype="f32")
    out = decode_reference(cache.physical(), q, [n, n], Hkv, d, 4, 4, 64)
    H = torch.tensor(hadamard(d))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            Kr = torch.tensor(bf16_round(rotate_f32(k[b, :, g])), dtype=torch.float64)
            Vr = torch.tensor(bf16_round(rotate_f32(v[b, :, g])), dtype=torch.float64)
            qr = H @ torch.tensor(q[b, h], dtype=torch.float64)
            o = torch.nn.functional.scaled_dot_product_attention(
                qr[None, None, None], Kr[None, None], Vr[None, None])[0, 0, 0]
            assert np.allclose(out[b, h], (H @ o).numpy(), rtol=1e-12, atol=1e-12)


def test_quantized_decode_error_ordering():
    # more bits -> closer to exact attention, and at every width the rotated
    # cache beats the unrotated one on this outlier-heavy input (velog.io
    # post, section "Hadamard rotation": outliers spread, loss drops)
    w, K, V, q = _tiny()
    d, n = w["d"], w["n"]
    exact = softmax_attention(q, K, V, 1 / np.sqrt(d))
    errs = {}
    for bits in (8, 6, 5, 4):
        for rot in (True, False):
            cache = OracleCache(1, 1, d, bits, bits, 0, n, rotate_k=rot, rotate_v=rot)
            cache.append(K[None, :, None], V[None, :, None], [0], dtype="f32")
            out = decode_reference(cache.physical(), q[None, None], [n], 1, d, bits,
                                   bits, 0, rotate_k=rot, rotate_v=rot)
            errs[bits, rot] = np.linalg.norm(out[0, 0] - exact) / np.linalg.norm(exact)
    # rotated, every width is well inside the regime where more bits help;
    # unrotated, the x20 outlier channels push 4..6 bits past 40% error, where
    # softmax noise (not the element error, which is monotone) orders them
    assert errs[8, True] < errs[6, True] < errs[5, True] < errs[4, True]
    assert errs[8, False] < errs[5, False] < errs[4, False]
    for bits in (8, 6, 5, 4):
        assert errs[bits, True] < 0.5 * errs[bits, False]
    assert errs[8, True] < 0.05


def test_rotate_flags_partial():
    # rotate_k only: q and K rotated, V and output not; with no quantization
    # loss (all tail) this still equals plain attention on bf16 rows
    B, Hkv, Hq, d, n = 1, 1, 2, 64, 16
    rng = np.random.default_rng(9)
    k = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    for rk, rv in ((True, False), (False, True), (False, False)):
        cache = OracleCache(B, Hkv, d, 8, 8, tail_len=n, max_ctx=64, rotate_k=rk, rotate_v=rv)
        cache.append(k, v, [0], dtype="f32")
        out = decode_reference(cache.physical(), q, [n], Hkv, d, 8, 8, n,
                               rotate_k=rk, rotate_v=rv)
        for h in range(Hq):
            ref = softmax_attention(q[0, h], k[0, :, 0].astype(np.float64),
                                    v[0, :, 0].astype(np.float64), 1 / np.sqrt(d))
            assert np.linalg.norm(out[0, h] - ref) <= 1e-2 * np.linalg.norm(ref)
