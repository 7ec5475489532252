"""Pins for the oracle's chunked-prefill attention (reading R20: the chunk's
queries are the last n_q positions and attend causally to the cache as it
stands after the chunk was appended; prompt processing is the cost the
velog.io post "fix KV cache quantization outliers" reports in section
"compute cost and speed").

Each pin checks prefill_reference against something other than itself:
* one query: the decode reference (pinned in test_oracle_attention.py);
* without a tail: query i equals decode attention over the cache truncated
  to its own position (so an off-by-one in the causal limit fails);
* with every token in the tail: torch's scaled_dot_product_attention in
  float64 with an explicit bottom-right causal mask on bf16(H k), bf16(H v);
* different sequence lengths in one batch, and the causal structure: changing
  a token after position p leaves query p unchanged."""

import numpy as np
import torch

import workloads
from oracle import (OracleCache, decode_reference, prefill_reference, hadamard,
                    rotate_f32, bf16_round)


def _cache(B, Hkv, d, kb, vb, T, lens, seed, max_ctx=None):
    rng = np.random.default_rng(seed)
    n = max(lens)
    k = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((B, n, Hkv, d)).astype(np.float32)
    c = OracleCache(B, Hkv, d, kb, vb, T, max_ctx or n + 8)
    c.append(k, v, [0] * B, dtype="f32")
    return c, k, v


def test_one_query_is_decode():
    B, Hkv, Hq, d = 2, 2, 6, 64
    c, _, _ = _cache(B, Hkv, d, 8, 4, 16, [90, 90], 1)
    q = np.random.default_rng(2).standard_normal((B, Hq, d)).astype(np.float32)
    planes = c.physical()
    dec = decode_reference(planes, q, [90, 90], Hkv, d, 8, 4, 16)
    pre = prefill_reference(planes, q[:, None], [90, 90], Hkv, d, 8, 4, 16)
    assert np.array_equal(pre[:, 0], dec)


def test_no_tail_query_equals_truncated_decode():
    B, Hkv, Hq, d, n, n_q = 1, 2, 4, 64, 70, 9
    c, _, _ = _cache(B, Hkv, d, 4, 5, 0, [n], 3)
    planes = c.physical()
    q = np.random.default_rng(4).standard_normal((B, n_q, Hq, d)).astype(np.float32)
    pre = prefill_reference(planes, q, [n], Hkv, d, 4, 5, 0)
    for i in range(n_q):
        p = n - n_q + i
        dec = decode_reference(planes, q[:, i], [p + 1], Hkv, d, 4, 5, 0)
        assert np.allclose(pre[:, i], dec, rtol=1e-13, atol=1e-13), i


def test_all_tail_is_textbook_causal_attention():
    B, Hkv, Hq, d, n, n_q = 2, 2, 4, 64, 40, 12
    c, k, v = _cache(B, Hkv, d, 4, 4, 64, [n, n], 5, max_ctx=128)
    planes = c.physical()
    q = np.random.default_rng(6).standard_normal((B, n_q, Hq, d)).astype(np.float32)
    pre = prefill_reference(planes, q, [n, n], Hkv, d, 4, 4, 64)
    H = torch.tensor(hadamard(d))
    # query i (position n - n_q + i) may see key t iff t <= n - n_q + i
    mask = torch.arange(n)[None, :] <= (n - n_q + torch.arange(n_q))[:, None]
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            Kr = torch.tensor(bf16_round(rotate_f32(k[b, :, g])), dtype=torch.float64)
            Vr = torch.tensor(bf16_round(rotate_f32(v[b, :, g])), dtype=torch.float64)
            qr = torch.tensor(q[b, :, h], dtype=torch.float64) @ H.T
            o = torch.nn.functional.scaled_dot_product_attention(
                qr[None, None], Kr[None, None], Vr[None, None], attn_mask=mask[None, None])[0, 0]
            assert np.allclose(pre[b, :, h], (o @ H.T).numpy(), rtol=1e-12, atol=1e-12)


def test_ragged_batch_and_causality():
    B, Hkv, Hq, d, n_q = 2, 1, 2, 64, 5
    lens = [50, 33]
    c, k, v = _cache(B, Hkv, d, 8, 8, 0, lens, 7)
    # sequence 1 restarted at length 0 and appended 33 tokens
    rng = np.random.default_rng(8)
    c2 = OracleCache(B, Hkv, d, 8, 8, 0, 90)
    c2.append(k, v, [0, 0], dtype="f32")
    k1 = rng.standard_normal((B, 33, Hkv, d)).astype(np.float32)
    c2.append(k1, k1, [50, 0], dtype="f32")
    planes = c2.physical()
    q = rng.standard_normal((B, n_q, Hq, d)).astype(np.float32)
    pre = prefill_reference(planes, q, [83, 33], Hkv, d, 8, 8, 0)
    for b, n in ((0, 83), (1, 33)):
        for i in range(n_q):
            dec = decode_reference(planes, q[:, i], [n - n_q + i + 1] * B, Hkv, d, 8, 8, 0)
            assert np.allclose(pre[b, i], dec[b], rtol=1e-13, atol=1e-13)
    # a token after query 0's position changes queries 1.. but not query 0
    c3 = OracleCache(B, Hkv, d, 8, 8, 0, 90)
    c3.append(k, v, [0, 0], dtype="f32")
    k2 = k1.copy()
    k2[:, -1] += 3.0
    c3.append(k2, k1, [50, 0], dtype="f32")
    pre3 = prefill_reference(c3.physical(), q, [83, 33], Hkv, d, 8, 8, 0)
    assert np.array_equal(pre3[:, :n_q - 1], pre[:, :n_q - 1])
    assert not np.allclose(pre3[:, n_q - 1], pre[:, n_q - 1])
