"""Device rounding primitives, checked through the product path against
NumPy and PyTorch CPU conversions (not against the oracle's code).

The append quantizes each 32-element block with an fp16 scale
s = fp16_rne(fp32(absmax / qmax)) (a correctly rounded float32 divide, then
round-to-nearest-even to fp16), codes rint(clamp(x * fp32(1 / s))) with ties
to even, and the precision tail stores bf16_rne(x) (aitrends.kr article 92204,
glossary "Precision Tail"; the block formats of the aiwitness.kr table
"Qwen 3.6 27B Q5_K_S + 64k context KLD results").  Rotation is off here, so
the crafted values reach those steps unchanged:

* scale ties: absmax / qmax lands exactly halfway between two fp16 values
  (both tie directions);
* division: absmax values for which multiplying by a rounded reciprocal
  instead of dividing gives a different fp16 scale (found by a search over
  float32 values with NumPy);
* code ties: s = 1 and elements k + 1/2, which rint sends to the even
  neighbour;
* bf16 tail ties: float32 inputs whose low 16 bits are 0x8000 (ties), 0x7FFF
  and 0x8001, against torch's float32 -> bfloat16 conversion.

Codes are read back with kvq_dequantize (code * s, exact in float32), the
scales from the scale plane."""

import numpy as np
import pytest
import torch

import decode_attention_rotate_amd as kvq
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu


def _qmax(bits):
    return (1 << (bits - 1)) - 1


def division_cases(q, n, seed=0):
    """float32 absmax values a where fp16(a / q) != fp16(a * fp32(1 / q))."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        a = (rng.random(1 << 20) * 100 + 0.01).astype(np.float32)
        d = (a / np.float32(q)).astype(np.float32).astype(np.float16)
        m = (a * (np.float32(1) / np.float32(q))).astype(np.float32).astype(np.float16)
        out.extend(a[d != m].tolist())
    return np.asarray(out[:n], np.float32)


def tie_absmax(q):
    """absmax values with absmax / q exactly halfway between fp16 neighbours:
    (1 + 2^-11) rounds down to 1 (even), (1 + 3 * 2^-11) up to 1 + 2^-9."""
    return np.asarray([q * (1 + 2.0 ** -11), q * (1 + 3 * 2.0 ** -11),
                       q * 4 * (1 + 5 * 2.0 ** -11), q * 0.25 * (1 + 7 * 2.0 ** -11)], np.float32)


def rows_for(bits, d, n_rows, seed):
    """[n_rows][d] float32 rows: blocks with crafted absmax values, and
    blocks of code ties."""
    q = _qmax(bits)
    rng = np.random.default_rng(seed)
    special = np.concatenate([tie_absmax(q), division_cases(q, 24, seed) if q in (7, 15) else []])
    x = (rng.standard_normal((n_rows, d)) * 0.01).astype(np.float32)
    k = 0
    for r in range(n_rows):
        for blk in range(d // 32):
            lo = 32 * blk
            if (r + blk) % 2 == 0 and k < len(special):
                x[r, lo + (r % 32)] = special[k] * (1 if k % 3 else -1)
                k += 1
            else:
                # s = fp16(q / q) = 1: codes of k + 1/2 round to even
                ties = np.asarray([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, -3.5], np.float32)
                x[r, lo:lo + 32] = np.resize(ties, 32)
                x[r, lo + 31] = q
    assert k == len(special), "rows too few for the crafted values"
    return x


def expected(x, bits):
    """(scale fp16 bits, codes) per 32-element block from NumPy's IEEE
    arithmetic: s = fp16(fp32(a / q)), r = fp32(1 / s), c = rint(clip(x * r))."""
    q = np.float32(_qmax(bits))
    blocks = x.reshape(x.shape[0], -1, 32)
    a = np.abs(blocks).max(axis=-1)
    s16 = np.minimum(a / q, np.float32(65504)).astype(np.float32).astype(np.float16)
    sf = s16.astype(np.float32)
    r = np.where(sf != 0, np.float32(1) / np.where(sf != 0, sf, 1), 0).astype(np.float32)
    t = (blocks * r[..., None]).astype(np.float32)
    c = np.rint(np.clip(t, -q, q))
    return s16.view(np.uint16), c


@pytest.mark.parametrize("bits", [4, 5, 6, 8])
def test_scale_division_and_code_ties(bits):
    d, n = 128, 40
    x = rows_for(bits, d, n, seed=bits)
    cfg = kvq.kvq_config(1, 1, d, 128, bits, bits, 0, False, False)
    cache = kvq.KVCache(cfg, DEV)
    kx = torch.from_numpy(x.reshape(1, n, 1, d)).to(DEV)
    say("primitives append", "bits=%d" % bits)
    kvq.kvq_rotate_quantize_append(cfg, cache, kx, kx.clone(), [0])
    torch.cuda.synchronize()
    s_bits, codes = expected(x, bits)
    for which, plane in ((0, "k_scales"), (1, "v_scales")):
        got_s = cache[plane].cpu().numpy().view(np.uint16).reshape(-1, d // 32)[:n]
        assert np.array_equal(got_s, s_bits), (which, np.argwhere(got_s != s_bits)[:4])
        xh = kvq.kvq_dequantize(cfg, cache, which, 0, 0, n, [n], 0).cpu().numpy().reshape(n, d // 32, 32)
        sf = s_bits.view(np.float16).astype(np.float32)
        want = (codes * sf[..., None]).astype(np.float32)
        assert np.array_equal(xh, want), (which, np.argwhere(xh != want)[:4])


def test_bf16_tail_rounding_ties():
    d, T = 128, 16
    rng = np.random.default_rng(3)
    hi = rng.integers(0x3000, 0x4800, size=(T, d), dtype=np.uint32)
    low = np.resize(np.asarray([0x8000, 0x7FFF, 0x8001, 0x0000], np.uint32), (T, d))
    sign = (rng.random((T, d)) < 0.5).astype(np.uint32) << 31
    x = ((hi << 16) | low | sign).view(np.float32)
    cfg = kvq.kvq_config(1, 1, d, 64, 8, 8, T, False, False)
    cache = kvq.KVCache(cfg, DEV)
    kx = torch.from_numpy(x.reshape(1, T, 1, d).copy()).to(DEV)
    say("primitives tail", "T=%d" % T)
    kvq.kvq_rotate_quantize_append(cfg, cache, kx, kx.clone(), [0])
    torch.cuda.synchronize()
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for plane in ("k_tail", "v_tail"):
        got = cache[plane].cpu().numpy().view(np.uint16).reshape(T, d)
        assert np.array_equal(got, want), (plane, np.argwhere(got != want)[:4])
