"""Pins for two primitives the oracle writes out by hand, against sources
other than the oracle itself.

* bfloat16 round-to-nearest-even (aitrends.kr article 92204, glossary entry
  "Precision Tail": the newest tokens are kept in bf16).  The oracle's bit
  trick and the input generator's copy of it are compared with torch's own
  float32 -> bfloat16 conversion, a library routine, over every exponent,
  both signs, constructed exact ties and carries into the next binade.
* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; Vigna's public-domain reference implementation),
  the generator behind the random-sign rotation (velog.io post "fix KV cache
  quantization outliers", section "application and background").  Its
  published outputs for state 0 are asserted directly.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle.blockquant import f32_to_bf16_bits, bf16_round, bf16_bits_to_f32
from oracle.rotation import splitmix64, hadamard_signs


def _torch_bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _finite_probe_values():
    """Float32 values over the whole finite range: every exponent (subnormals
    included), both signs, random mantissas, exact ties between two bf16
    neighbours (odd and even), and mantissas just below a carry into the next
    binade."""
    rng = np.random.default_rng(2024)
    parts = []
    exps = np.arange(0, 255, dtype=np.uint32)          # biased exponent 0..254
    for sign in (0, 1):
        mant = rng.integers(0, 1 << 23, size=(exps.size, 64), dtype=np.uint32)
        bits = (np.uint32(sign) << 31) | (exps[:, None] << 23) | mant
        parts.append(bits.ravel())
        # ties: low 16 bits exactly 0x8000, the kept bit both even and odd
        hi = rng.integers(0, 1 << 7, size=(exps.size, 16), dtype=np.uint32)
        tie = (np.uint32(sign) << 31) | (exps[:, None] << 23) | (hi << 16) | 0x8000
        parts.append(tie.ravel())
        parts.append((tie | 0x10000).ravel())          # odd kept bit
        parts.append((tie - 1).ravel())                # just below a tie
        parts.append((tie + 1).ravel())                # just above a tie
        # all-ones kept mantissa: rounding up carries into the exponent
        carry = (np.uint32(sign) << 31) | (exps[:, None] << 23) | np.uint32(0x7F8000)
        parts.append(carry.ravel())
        parts.append((carry | 0x7FFF).ravel())
    bits = np.concatenate(parts)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]          # finite only
    return bits.view(np.float32)


def test_bf16_rne_matches_torch_conversion():
    x = _finite_probe_values()
    # values whose rounding overflows to infinity are outside the contract
    ref = _torch_bf16_bits(x)
    keep = (ref & 0x7F80) != 0x7F80
    assert keep.mean() > 0.99
    x, ref = x[keep], ref[keep]
    assert x.size > 60000
    ours = f32_to_bf16_bits(x)
    assert np.array_equal(ours, ref), int(np.sum(ours != ref))
    gen = workloads.to_bf16_bits(x)
    assert np.array_equal(gen, ref)
    # the float-valued helper is the same rounding
    assert np.array_equal(bf16_round(x).view(np.uint32), bf16_bits_to_f32(ref).view(np.uint32))


def test_bf16_rne_ties_go_to_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: even (1.0) wins;
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6: up.
    one = np.float32(1.0)
    cases = {
        np.float32(1.0 + 2.0 ** -8): 0x3F80,
        np.float32(1.0 + 3 * 2.0 ** -8): 0x3F82,
        np.float32(-(1.0 + 2.0 ** -8)): 0xBF80,
        np.float32(2.0 - 2.0 ** -8): 0x4000,      # carries into the next binade
        one: 0x3F80,
    }
    for v, want in cases.items():
        assert int(f32_to_bf16_bits(np.array([v]))[0]) == want, hex(int(np.array([v]).view(np.uint32)[0]))


def test_bf16_truncation_would_fail():
    # a truncating conversion disagrees with torch on the probe set, so the
    # comparison above does tell rounding modes apart
    x = _finite_probe_values()
    trunc = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.sum(trunc != _torch_bf16_bits(x)) > 1000


# Published outputs of SplitMix64 started from state 0: the state advances by
# the golden-gamma increment before each output, so output k (1-based) mixes
# k * gamma, which is the oracle's splitmix64((k - 1) * gamma).
_SPLITMIX64_FROM_ZERO = (
    0xE220A8397B1DCDAF,
    0x6E789E6AA1B965F4,
    0x06C45D188009454F,
    0xF88BB8A8724C81EC,
    0x1B39896A51A8749B,
)
_GAMMA = 0x9E3779B97F4A7C15


def test_splitmix64_published_outputs():
    for k, want in enumerate(_SPLITMIX64_FROM_ZERO):
        assert splitmix64((k * _GAMMA) & ((1 << 64) - 1)) == want, k


def test_sign_rule_reads_top_bit_of_counter():
    # reading R21: sign e of seed s is -1 iff the top bit of
    # splitmix64(s * 2^32 + e) is set.  Counter 0 (seed 0 is "no signs", so
    # use the counter arithmetic directly): splitmix64(0) = 0xE220... has its
    # top bit set.
    assert splitmix64(0) >> 63 == 1
    s = hadamard_signs(64, 1)
    for e in range(64):
        assert (s[e] < 0) == bool(splitmix64((1 << 32) | e) >> 63)
