"""Pins for the oracle's rotation (velog.io post "fix KV cache quantization
outliers", section "Hadamard rotation": normalized Hadamard, orthogonal, dot
products preserved)."""

import decimal

import numpy as np
import pytest
import scipy.linalg

from oracle import hadamard, rot_scale_f32, fwht_f32, rotate_f32

DIMS = (64, 128, 256)


@pytest.mark.parametrize("d", DIMS)
def test_hadamard_orthogonal_symmetric(d):
    H = hadamard(d)
    assert np.array_equal(H, H.T)
    assert np.max(np.abs(H @ H.T - np.eye(d))) < 1e-14
    assert np.max(np.abs(H @ H - np.eye(d))) < 1e-14


@pytest.mark.parametrize("d", DIMS)
def test_hadamard_is_sylvester(d):
    # library routine: scipy builds Sylvester's matrix in natural order
    assert np.array_equal(hadamard(d) * np.sqrt(d), scipy.linalg.hadamard(d).astype(float))


@pytest.mark.parametrize("d", DIMS)
def test_rot_scale_is_nearest_float32(d):
    decimal.getcontext().prec = 60
    exact = decimal.Decimal(1) / decimal.Decimal(d).sqrt()
    c = rot_scale_f32(d)
    lo = np.nextafter(c, np.float32(0))
    hi = np.nextafter(c, np.float32(1))
    err = abs(decimal.Decimal(float(c)) - exact)
    assert err <= abs(decimal.Decimal(float(lo)) - exact)
    assert err <= abs(decimal.Decimal(float(hi)) - exact)


@pytest.mark.parametrize("d", DIMS)
def test_fwht_exact_on_small_integers(d):
    # integer inputs keep every partial sum exact in float32, so the fast
    # transform must equal the dense integer product exactly; a wrong sign,
    # index or stage fails here
    rng = np.random.default_rng(d)
    x = rng.integers(-1000, 1000, size=(20, d)).astype(np.float32)
    want = x.astype(np.int64) @ scipy.linalg.hadamard(d).T
    assert np.array_equal(fwht_f32(x), want.astype(np.float32))


def _scalar_fwht(v):
    """Independent scalar loop with per-operation float32 rounding."""
    v = [np.float32(t) for t in v]
    d = len(v)
    h = 1
    while h < d:
        for i in range(d):
            if i & h == 0:
                a, b = v[i], v[i + h]
                v[i], v[i + h] = np.float32(a + b), np.float32(a - b)
        h *= 2
    return np.array(v, dtype=np.float32)


@pytest.mark.parametrize("d", (64, 128))
def test_fwht_matches_scalar_stage_order(d):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((3, d)) * np.exp(rng.uniform(-8, 8, (3, d)))).astype(np.float32)
    got = fwht_f32(x)
    for r in range(3):
        assert np.array_equal(got[r].view(np.uint32), _scalar_fwht(x[r]).view(np.uint32))


@pytest.mark.parametrize("d", DIMS)
def test_rotate_within_rounding_bound_of_dense(d):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((50, d)).astype(np.float32)
    x[:, 3] *= 20
    y = rotate_f32(x).astype(np.float64)
    exact = x.astype(np.float64) @ hadamard(d).T
    u = 2.0 ** -24
    l1 = np.sum(np.abs(x.astype(np.float64)), axis=1, keepdims=True)
    bound = (np.log2(d) * u * l1 / np.sqrt(d) + 2 * u * np.abs(exact)) * 1.01
    assert np.all(np.abs(y - exact) <= bound)


@pytest.mark.parametrize("d", DIMS)
def test_rotate_twice_is_identity(d):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((10, d)).astype(np.float32)
    back = rotate_f32(rotate_f32(x))
    assert np.max(np.abs(back - x)) < 4 * np.log2(d) * 2.0 ** -24 * np.max(np.sum(np.abs(x), 1)) / np.sqrt(d) + 1e-6


@pytest.mark.parametrize("d", DIMS)
def test_dot_products_preserved(d):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((100, d)).astype(np.float32)
    y = rng.standard_normal((100, d)).astype(np.float32)
    x[:, 7] *= 20
    lhs = np.sum(rotate_f32(x) * rotate_f32(y), axis=1, dtype=np.float32)
    rhs = np.sum(x * y, axis=1, dtype=np.float32)
    norm = np.linalg.norm(x, axis=1) * np.linalg.norm(y, axis=1)
    assert np.all(np.abs(lhs - rhs) <= 1e-5 * norm)


def test_rotation_disabled_is_identity():
    x = np.arange(128, dtype=np.float32)
    assert np.array_equal(rotate_f32(x, enabled=False), x)


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        fwht_f32(np.zeros(192, np.float32))
