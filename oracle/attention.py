"""Decode and chunked-prefill attention over the rotated quantized cache (oracle).

Source: velog.io post "fix KV cache quantization outliers", section
"Hadamard rotation": attention runs on the rotated Q and K (the Hadamard
matrix is orthogonal, so Q.K dot products and the scores are unchanged) and
the result is rotated back to the original space afterwards.  The bf16
precision tail (aitrends.kr article 92204, glossary "Precision Tail") holds
the newest tokens unquantized.

This is the plain definition in float64: dense H, scores, two-pass softmax,
weighted sum, dense inverse rotation.  No blocking, no online softmax.

Readings:
* R12 GQA: query head h uses KV head h // (Hq / Hkv).
* R13 The single query is the newest position; it attends to all n cached
      tokens (the current token is already appended), scaled by sm_scale.
* R14 The output is float32-valued, in the original (unrotated) space.
* R15 rotate_k off: neither q nor K is rotated; rotate_v off: V is not
      rotated and the output is not rotated back.
* R20 Chunked prefill (prompt processing, whose rotation cost the velog.io
      post reports in section "compute cost and speed"): the n_q queries of a
      chunk are the last n_q positions of the sequence, already appended;
      query i sits at position p = n - n_q + i and attends to positions
      0..p (causal), reading the cache as it stands after the whole chunk
      was appended (a token that left the tail during the chunk is read
      quantized).
"""

import numpy as np

from .rotation import rotation_matrix, unrotate_f32, hadamard_signs
from .blockquant import bf16_bits_to_f32
from .kvcache import dequantize_rows


def softmax_attention(q, K, V, sm_scale):
    """o = softmax(sm_scale * K q) V in float64 (two-pass, max subtracted)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = sm_scale * (K @ q)
    s = s - np.max(s)
    w = np.exp(s)
    w = w / np.sum(w)
    return w @ V


def dequantize_unit(planes, b, g, n, d, k_bits, v_bits, tail_len, k_min=False, v_min=False):
    """Rotated-space K_hat, V_hat (float64, [n][d]) of sequence b, KV head g.

    Positions below n - min(n, T) come from the code planes; the newest
    min(n, T) positions come from tail slot p mod T.  k_min / v_min select
    the scale-and-min blocks of reading R22."""
    T = int(tail_len)
    nt = min(n, T) if T > 0 else 0
    nq = n - nt
    out = []
    for p, bits, mf in (("k", k_bits, k_min), ("v", v_bits, v_min)):
        x = np.zeros((n, d), dtype=np.float64)
        if nq > 0:
            x[:nq] = dequantize_rows(planes[p + "_codes"][b, g],
                                     planes[p + "_scales"][b, g], d, bits, nq, p, mf)
        for pos in range(nq, n):
            x[pos] = bf16_bits_to_f32(planes[p + "_tail"][b, g, pos % T])
        out.append(x)
    return out[0], out[1]


def decode_reference(planes, q, lens, n_kv_heads, d, k_bits, v_bits,
                     tail_len, sm_scale=None, rotate_k=True, rotate_v=True,
                     heads=None, sign_seed=0, k_min=False, v_min=False):
    """Reference output [B][Hq][d] (float64) of decode attention.

    q: float values [B][Hq][d] (already widened from bf16 if needed).
    heads: optional iterable of (b, h) pairs to evaluate; others stay NaN.
    sign_seed: the randomized-sign rotation R = H diag(s) of reading R21
    (0: H); q is rotated by R and the output by R^T."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _ = q.shape
    G = Hq // n_kv_heads
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    H = rotation_matrix(d, sign_seed)
    out = np.full((B, Hq, d), np.nan)
    want = set(heads) if heads is not None else None
    cache = {}
    for b in range(B):
        for h in range(Hq):
            if want is not None and (b, h) not in want:
                continue
            g = h // G
            if (b, g) not in cache:
                cache[(b, g)] = dequantize_unit(planes, b, g, int(lens[b]), d,
                                                k_bits, v_bits, tail_len, k_min, v_min)
            K, V = cache[(b, g)]
            qr = H @ q[b, h] if rotate_k else q[b, h]
            o = softmax_attention(qr, K, V, sm_scale)
            out[b, h] = H.T @ o if rotate_v else o
    return out


def prefill_reference(planes, q, lens, n_kv_heads, d, k_bits, v_bits,
                      tail_len, sm_scale=None, rotate_k=True, rotate_v=True,
                      rows=None, sign_seed=0, k_min=False, v_min=False):
    """Reference output [B][n_q][Hq][d] (float64) of chunked prefill attention.

    q: float values [B][n_q][Hq][d], the queries of the last n_q positions of
    each sequence (R20); lens[b] >= n_q is the length after the chunk.
    rows: optional iterable of (b, i, h) triples to evaluate; others stay NaN.
    sign_seed: as for decode_reference."""
    q = np.asarray(q, dtype=np.float64)
    B, n_q, Hq, _ = q.shape
    G = Hq // n_kv_heads
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    H = rotation_matrix(d, sign_seed)
    out = np.full((B, n_q, Hq, d), np.nan)
    want = set(rows) if rows is not None else None
    cache = {}
    for b in range(B):
        n = int(lens[b])
        for i in range(n_q):
            p = n - n_q + i
            for h in range(Hq):
                if want is not None and (b, i, h) not in want:
                    continue
                g = h // G
                if (b, g) not in cache:
                    cache[(b, g)] = dequantize_unit(planes, b, g, n, d, k_bits, v_bits,
                                                    tail_len, k_min, v_min)
                K, V = cache[(b, g)]
                qr = H @ q[b, i, h] if rotate_k else q[b, i, h]
                o = softmax_attention(qr, K[:p + 1], V[:p + 1], sm_scale)
                out[b, i, h] = H.T @ o if rotate_v else o
    return out


def dequantize_reference(planes, which, b, t0, t1, n, n_kv_heads, d, bits,
                         tail_len, space, rotate=True, sign_seed=0, minf=False):
    """Dequantized positions [t0, t1) of sequence b (length n), all KV heads.

    space 0: rotated space (exact float32).  space 1: original space, i.e. the
    rotated value multiplied by H again in float32 with the fixed stage order
    (H is its own inverse) and then by the signs of R21, so the GPU must match
    bit for bit."""
    p = "k" if which == 0 else "v"
    T = int(tail_len)
    nt = min(n, T) if T > 0 else 0
    nq = n - nt
    out = np.zeros((t1 - t0, n_kv_heads, d), dtype=np.float32)
    for g in range(n_kv_heads):
        if nq > 0:
            rows = dequantize_rows(planes[p + "_codes"][b, g],
                                   planes[p + "_scales"][b, g], d, bits, nq, p, minf)
        for pos in range(t0, t1):
            if pos < nq:
                out[pos - t0, g] = rows[pos]
            else:
                out[pos - t0, g] = bf16_bits_to_f32(planes[p + "_tail"][b, g, pos % T])
    if space == 1:
        out = unrotate_f32(out, rotate, hadamard_signs(d, sign_seed))
    return out
