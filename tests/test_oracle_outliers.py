"""Pins of the outlier-channel split (reading R25; velog.io post, section
"application and background", mixed precision with the outlier channels at
8 bits).

* An empty outlier set reduces to the plain rotated format, byte for byte.
* Before quantization the split is exact: R^T (R x_R) + scatter(x_O) = x and
  q.x = (R q).(R x_R) + q[O].x_O (float64).
* The outlier block is the 8-bit quantizer, checked by brute force over all
  255 levels.
* The rotated rest is within half a step of the dense float64 rotation of x
  with the outlier channels zeroed (a missed zeroing or a wrong index moves
  outlier energy into it).
* On the tiny workload (channels 3 and 41 x20, 4-bit), keeping a 32-channel
  set that holds the outliers at 8 bits lowers the reconstruction MSE below
  half of rotation alone.
* Attention in the split form equals attention over the float32
  reconstruction, for plain and random-sign rotations (a transposed rotation
  or a wrong gather fails it)."""

import numpy as np
import pytest

import workloads
from oracle import rotate_f32, quantize_blocks, softmax_attention, rotation_matrix, hadamard_signs
from oracle.outliers import (split_outliers, quantize_rows_outliers, dequantize_parts,
                             reconstruct_f32, attention_outliers)


def _set(d, must, seed=0):
    rng = np.random.default_rng(seed)
    rest = [c for c in rng.permutation(d) if c not in must]
    return np.array(list(must) + rest[: 32 - len(must)], dtype=np.int64)


def test_empty_set_is_the_plain_format():
    x = np.random.default_rng(1).standard_normal((7, 128)).astype(np.float32)
    parts = quantize_rows_outliers(x, [], 4)
    c, s = quantize_blocks(rotate_f32(x), 4)
    assert np.array_equal(parts["rest_codes"], c) and np.array_equal(parts["rest_scales"], s)
    assert parts["out_codes"].shape == (7, 0)


@pytest.mark.parametrize("seed", [0, 9])
def test_split_is_exact_before_quantization(seed):
    d = 128
    rng = np.random.default_rng(2)
    x = rng.standard_normal(d)
    q = rng.standard_normal(d)
    idx = _set(d, [5, 77, 100])
    xr, xo = split_outliers(x, idx)
    assert np.all(xr[idx] == 0) and np.array_equal(xo, x[idx])
    R = rotation_matrix(d, seed)
    back = R.T @ (R @ xr)
    back[idx] += xo
    assert np.max(np.abs(back - x)) < 1e-12
    assert abs((R @ q) @ (R @ xr) + q[idx] @ xo - q @ x) < 1e-12


def test_outlier_block_is_the_8bit_quantizer():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((20, 64)) * rng.choice([1e-3, 1.0, 40.0], (20, 1))).astype(np.float32)
    idx = _set(64, [3, 41])
    parts = quantize_rows_outliers(x, idx, 4)
    xo = x[:, idx]
    levels = np.arange(-127, 128)
    for i in range(xo.shape[0]):
        a = np.float32(np.max(np.abs(xo[i])))
        s16 = np.float16(min(a / np.float32(127.0), np.float32(65504.0)))
        assert parts["out_scales"][i, 0] == s16.view(np.uint16)
        r = np.float32(1.0) / np.float32(s16)
        t = (xo[i] * r).astype(np.float32).astype(np.float64)
        for e in range(32):
            dist = np.abs(t[e] - levels)
            best = levels[dist == dist.min()]
            want = best[0] if best.size == 1 else best[best % 2 == 0][0]
            assert parts["out_codes"][i, e] == want


@pytest.mark.parametrize("bits,minf", [(4, False), (5, True), (8, False)])
def test_rest_is_the_rotation_without_the_outliers(bits, minf):
    d = 128
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, d)).astype(np.float32)
    idx = _set(d, [7, 64])
    x[:, [7, 64]] *= 50.0
    parts = quantize_rows_outliers(x, idx, bits, minf=minf)
    y, _ = dequantize_parts(parts, bits, minf)
    xr = x.astype(np.float64).copy()
    xr[:, idx] = 0
    exact = xr @ rotation_matrix(d).T
    if minf:
        step = parts["rest_scales"][..., 0].view(np.float16).astype(np.float64)
    else:
        step = parts["rest_scales"].view(np.float16).astype(np.float64)
    bound = np.repeat(step, 32, axis=-1) / 2 + 1e-5 * np.max(np.abs(exact))
    assert np.all(np.abs(y - exact) <= bound)


def test_outlier_set_lowers_mse_on_the_tiny_workload():
    w = workloads.workload("tiny")
    x = workloads.kv_numpy(w, 1, 0, w["n"])[0, :, 0, :].astype(np.float32)   # [256][64]
    idx = _set(64, list(w["channels"]))
    rot_only = quantize_rows_outliers(x, [], 4)
    mixed = quantize_rows_outliers(x, idx, 4)
    mse_rot = np.mean((reconstruct_f32(rot_only, [], 4) - x) ** 2)
    mse_mix = np.mean((reconstruct_f32(mixed, idx, 4) - x) ** 2)
    assert mse_mix < 0.5 * mse_rot, (mse_mix, mse_rot)


@pytest.mark.parametrize("seed,rk,rv", [(0, True, True), (5, True, True), (5, True, False),
                                        (0, False, True)])
def test_split_attention_equals_attention_on_the_reconstruction(seed, rk, rv):
    d, n = 64, 90
    rng = np.random.default_rng(6)
    k = rng.standard_normal((n, d)).astype(np.float32)
    v = rng.standard_normal((n, d)).astype(np.float32)
    k[:, 3] *= 20.0
    v[:, 41] *= 20.0
    q = rng.standard_normal(d).astype(np.float32)
    ki, vi = _set(d, [3], 1), _set(d, [41], 2)
    signs = hadamard_signs(d, seed)
    kp = quantize_rows_outliers(k, ki, 4, rotate=rk, signs=signs)
    vp = quantize_rows_outliers(v, vi, 5, rotate=rv, signs=signs)
    got = attention_outliers(q, kp, vp, ki, vi, 4, 5, 0.125, rk, rv, seed)
    K = reconstruct_f32(kp, ki, 4, rotate=rk, signs=signs)
    V = reconstruct_f32(vp, vi, 5, rotate=rv, signs=signs)
    want = softmax_attention(q, K, V, 0.125)
    assert np.linalg.norm(got - want) <= 1e-5 * np.linalg.norm(want)


# ------------------------------------------------------------ the cache
def _cache_inputs(seed, B=2, n=130, H=2, d=128):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, n, H, d)).astype(np.float32)
    v = rng.standard_normal((B, n, H, d)).astype(np.float32)
    k[..., 9] *= 25.0
    v[..., d - 28] *= 25.0
    ki = np.stack([_set(d, [9], 10 + g) for g in range(H)])
    vi = np.stack([_set(d, [d - 28], 20 + g) for g in range(H)])
    return k, v, ki, vi


@pytest.mark.parametrize("kb,vb,km,vm", [(4, 4, False, False), (8, 5, False, True), (5, 8, True, False)])
def test_cache_rest_planes_are_the_plain_cache_of_the_zeroed_rest(kb, vb, km, vm):
    from oracle import OracleCache
    from oracle.outliers import OutlierCache
    k, v, ki, vi = _cache_inputs(1)
    B, n, H, d = k.shape
    oc = OutlierCache(B, H, d, kb, vb, n + 3, ki, vi, k_min=km, v_min=vm)
    oc.append(k, v, [0, 0], dtype="f32")
    kr, vr = k.copy(), v.copy()
    for g in range(H):
        kr[:, :, g, ki[g]] = 0
        vr[:, :, g, vi[g]] = 0
    plain = OracleCache(B, H, d, kb, vb, 0, n + 3, k_min=km, v_min=vm)
    plain.append(kr, vr, [0, 0], dtype="f32")
    got, want = oc.physical(), plain.physical()
    for key in want:
        assert np.array_equal(got[key], want[key]), key


def test_cache_outlier_planes_hold_the_8bit_blocks_of_the_gathered_channels():
    from oracle.outliers import OutlierCache, outlier_values
    k, v, ki, vi = _cache_inputs(2)
    B, n, H, d = k.shape
    oc = OutlierCache(B, H, d, 4, 4, n, ki, vi)
    # two appends (chunking must not matter)
    oc.append(k[:, :70], v[:, :70], [0, 0], dtype="f32")
    oc.append(k[:, 70:], v[:, 70:], [70, 70], dtype="f32")
    planes = oc.physical()
    for b in range(B):
        for g in range(H):
            for p, x, idx in (("k", k, ki), ("v", v, vi)):
                codes, scales = quantize_blocks(x[b, :, g][:, idx[g]], 8)
                got = outlier_values(planes, p, b, g, n)
                from oracle import dequantize_blocks
                assert np.array_equal(got, dequantize_blocks(codes, scales))
                assert np.array_equal(planes[p + "_out_scales"][b, g][:n], scales[:, 0])


def test_cache_attention_equals_attention_on_the_reconstruction():
    from oracle.outliers import OutlierCache, decode_reference_outliers, outlier_values
    from oracle import dequantize_reference, rotation_matrix as rm
    k, v, ki, vi = _cache_inputs(3, B=1, n=100, H=2, d=64)
    B, n, H, d = k.shape
    oc = OutlierCache(B, H, d, 4, 5, n, ki, vi, sign_seed=7)
    oc.append(k, v, [0], dtype="f32")
    planes = oc.physical()
    q = np.random.default_rng(4).standard_normal((B, 2 * H, d))
    got = decode_reference_outliers(planes, q, [n], H, d, 4, 5, ki, vi, sign_seed=7)
    R = rm(d, 7)
    from oracle.kvcache import dequantize_rows
    for g in range(H):
        # the full reconstruction: R^T rest + outliers at their channels
        K = dequantize_rows(planes["k_codes"][0, g], planes["k_scales"][0, g], d, 4, n, "k") @ R
        V = dequantize_rows(planes["v_codes"][0, g], planes["v_scales"][0, g], d, 5, n, "v") @ R
        K[:, ki[g]] += outlier_values(planes, "k", 0, g, n)
        V[:, vi[g]] += outlier_values(planes, "v", 0, g, n)
        for h in (2 * g, 2 * g + 1):
            want = softmax_attention(q[0, h], K, V, 1.0 / np.sqrt(d))
            assert np.linalg.norm(got[0, h] - want) <= 1e-10 * np.linalg.norm(want)
