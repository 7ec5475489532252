"""Outlier-channel mixed precision (oracle, test infrastructure only).

Source: velog.io post "fix KV cache quantization outliers", section
"application and background": the TurboQuant work that the rotation patch
follows keeps only the outlier channels at 8 bits (mixed precision).  The
post gives no algorithm.  Section "the essence of the problem" says why it
helps: a few channels carry values far larger than the rest, and one scale
per block is then set by those extremes.

Reading R25 (the plainest scheme the post supports, written in this cache's
block formats):
* Each plane (K or V) of a KV head has a set O of outlier channels, given as
  a list of m distinct channel indices (m a multiple of 32; the caller picks
  them, for instance from calibration).
* A head vector x is split before rotation: x_O = x[O] (list order) and
  x_R = x with the channels of O set to 0.
* x_R takes the path of every other vector: y = rotation of x_R (readings
  R1-R4, R21, R23), bf16-rounded first when the plane has a precision tail
  (R5), then quantized in the plane's block format (R6-R10, R22).
* x_O stays in the original space and is quantized as 8-bit absmax blocks
  (the same rule at 8 bits, bf16-rounded first with a tail).
* Reconstruction in the original space: x_hat = R^T y_hat, plus the
  dequantized outlier values added at their channels (float32, one rounding).
* Attention splits the same way, which is exact algebra because R is
  orthogonal: q.x_hat = (R q).y_hat + q[O].x_O_hat, and the output is
  R^T (sum p v_R_hat) plus the outlier part scattered back to its channels.
"""

import numpy as np

from .rotation import rotate_f32, unrotate_f32, rotation_matrix
from .blockquant import (quantize_blocks, dequantize_blocks, quantize_blocks_min,
                         dequantize_blocks_min, bf16_round, BLOCK)


def _index(idx, d):
    idx = np.asarray(idx, dtype=np.int64).reshape(-1)
    if idx.size % BLOCK:
        raise ValueError("the outlier set holds a multiple of 32 channels")
    if idx.size and (idx.min() < 0 or idx.max() >= d or np.unique(idx).size != idx.size):
        raise ValueError("outlier channels must be distinct and in [0, d)")
    return idx


def split_outliers(x, idx):
    """(x_R, x_O): x with the channels idx set to zero, and x[..., idx]."""
    x = np.asarray(x)
    idx = _index(idx, x.shape[-1])
    rest = x.copy()
    rest[..., idx] = 0
    return rest, x[..., idx].copy()


def quantize_rows_outliers(x, idx, bits, rotate=True, signs=None, tail_round=False,
                           minf=False):
    """Quantize float32 head vectors x [..., d] with outlier set idx (R25).

    Returns a dict:
      rest_codes, rest_scales  the rotated rest in the plane's format
                               (scales: fp16 bits, or (s, m) pairs if minf)
      out_codes, out_scales    the outlier values as 8-bit absmax blocks
    tail_round: round both parts to bf16 before quantizing (a plane with a
    precision tail, reading R5)."""
    x = np.asarray(x, dtype=np.float32)
    rest, out = split_outliers(x, idx)
    y = rotate_f32(rest, rotate, signs)
    if tail_round:
        y = bf16_round(y)
        out = bf16_round(out)
    if minf:
        rc, rs = quantize_blocks_min(y, bits)
    else:
        rc, rs = quantize_blocks(y, bits)
    if out.shape[-1]:
        oc, os_ = quantize_blocks(out, 8)
    else:
        oc = np.zeros(out.shape, np.int8)
        os_ = np.zeros(out.shape[:-1] + (0,), np.uint16)
    return {"rest_codes": rc, "rest_scales": rs, "out_codes": oc, "out_scales": os_}


def dequantize_parts(parts, bits, minf=False):
    """(y_hat, x_O_hat): the rotated rest and the outlier values, float32."""
    if minf:
        y = dequantize_blocks_min(parts["rest_codes"], parts["rest_scales"], bits)
    else:
        y = dequantize_blocks(parts["rest_codes"], parts["rest_scales"])
    if parts["out_codes"].shape[-1]:
        o = dequantize_blocks(parts["out_codes"], parts["out_scales"])
    else:
        o = np.zeros(parts["out_codes"].shape, np.float32)
    return y, o


def reconstruct_f32(parts, idx, bits, rotate=True, signs=None, minf=False):
    """x_hat in the original space, float32: the rest rotated back (the same
    float32 transform as the append), then the outlier values added at their
    channels with one float32 add."""
    y, o = dequantize_parts(parts, bits, minf)
    x = unrotate_f32(y, rotate, signs)
    idx = _index(idx, x.shape[-1])
    x[..., idx] = (x[..., idx] + o).astype(np.float32)
    return x


def attention_outliers(q, k_parts, v_parts, k_idx, v_idx, k_bits, v_bits, sm_scale,
                       rotate_k=True, rotate_v=True, seed=0, k_min=False, v_min=False):
    """Single-query attention in float64 over n cached tokens stored with
    outlier sets (R25), in the split form:
      s_t = sm_scale * ((R q) . y_t + q[k_idx] . xo_t)
      out = R^T (sum_t p_t yv_t) + scatter_{v_idx}(sum_t p_t xov_t)
    q [d]; k_parts / v_parts as returned by quantize_rows_outliers for [n][d]."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    Rk = rotation_matrix(d, seed) if rotate_k else np.eye(d)
    Rv = rotation_matrix(d, seed) if rotate_v else np.eye(d)
    ky, ko = (a.astype(np.float64) for a in dequantize_parts(k_parts, k_bits, k_min))
    vy, vo = (a.astype(np.float64) for a in dequantize_parts(v_parts, v_bits, v_min))
    ki = _index(k_idx, d)
    vi = _index(v_idx, d)
    s = sm_scale * (ky @ (Rk @ q) + ko @ q[ki])
    s = s - np.max(s)
    p = np.exp(s)
    p = p / np.sum(p)
    out = Rv.T @ (p @ vy)
    out[vi] += p @ vo
    return out


# ---------------------------------------------------------------- the cache
# Planes of the outlier parts, in the device byte layout (reading R25 with
# the layouts of reading R11 at 32 channels):
#   k_out_codes  per (b, g): [cap][32] 8-bit two's-complement codes (rows)
#   v_out_codes  per (b, g): element-major 64-token tiles of the 32 outlier
#                channels at 8 bits (offset codes u = c + 128), the V-tile
#                layout of a 32-element head
#   k_out_scales, v_out_scales  per (b, g): [cap] fp16 bits (one 32-block)

class OutlierCache:
    """Cache with an outlier set of 32 channels per plane and KV head
    (reading R25), without a precision tail: the rest of every vector is
    stored by the plain rules (an OracleCache of the zeroed-outlier rest
    would hold the same planes), the outliers as one 8-bit absmax block in
    the original space.  k_idx, v_idx: int [Hkv][32] channel lists."""

    def __init__(self, batch, n_kv_heads, head_dim, k_bits, v_bits, max_ctx, k_idx, v_idx,
                 rotate_k=True, rotate_v=True, sign_seed=0, k_min=False, v_min=False):
        from .kvcache import OracleCache
        from .blockquant import TILE
        self.B, self.H, self.d = batch, n_kv_heads, head_dim
        self.idx = {"k": np.asarray(k_idx, np.int64).reshape(n_kv_heads, BLOCK),
                    "v": np.asarray(v_idx, np.int64).reshape(n_kv_heads, BLOCK)}
        for p in ("k", "v"):
            for g in range(n_kv_heads):
                _index(self.idx[p][g], head_dim)
        self.base = OracleCache(batch, n_kv_heads, head_dim, k_bits, v_bits, 0, max_ctx,
                                rotate_k, rotate_v, sign_seed, k_min, v_min)
        cap = self.base.cap
        self.out_codes = {p: np.zeros((batch, n_kv_heads, cap, BLOCK), np.int8) for p in ("k", "v")}
        self.out_scales = {p: np.zeros((batch, n_kv_heads, cap), np.uint16) for p in ("k", "v")}
        self.v_out_u = np.zeros((batch, n_kv_heads, cap, BLOCK), np.uint8)
        self.TILE = TILE

    def append(self, k_new, v_new, lens, dtype="bf16"):
        """Append n_new tokens per sequence ([B][n_new][Hkv][d]); lens are
        the lengths before.  Returns the new lengths."""
        from .kvcache import _widen
        lens = np.asarray(lens, dtype=np.int64)
        rests, outs = [], []
        for p, new in (("k", k_new), ("v", v_new)):
            x = _widen(new, dtype).astype(np.float32)            # [B][n][H][d]
            rest = x.copy()
            out = np.zeros(x.shape[:-1] + (BLOCK,), np.float32)
            for g in range(self.H):
                r, o = split_outliers(x[:, :, g, :], self.idx[p][g])
                rest[:, :, g, :] = r
                out[:, :, g, :] = o
            rests.append(rest)
            outs.append(out)
        # the rest takes the plain path (rotation, block format)
        new_lens = self.base.append(rests[0], rests[1], lens, dtype="f32")
        n_new = np.asarray(k_new).shape[1]
        for p, out in (("k", outs[0]), ("v", outs[1])):
            codes, scales = quantize_blocks(out, 8)               # [B][n][H][32], [B][n][H][1]
            for b in range(self.B):
                for i in range(n_new):
                    pos = int(lens[b]) + i
                    self.out_codes[p][b, :, pos, :] = codes[b, i]
                    self.out_scales[p][b, :, pos] = scales[b, i, :, 0]
                    if p == "v":
                        self.v_out_u[b, :, pos, :] = (codes[b, i].astype(np.int16) + 128).astype(np.uint8)
        return new_lens

    def physical(self):
        """The plain planes of the rest plus the four outlier planes."""
        from .blockquant import offset_codes_to_vtiles
        out = self.base.physical()
        cap = self.base.cap
        out["k_out_codes"] = self.out_codes["k"].view(np.uint8).reshape(self.B, self.H, cap * BLOCK).copy()
        vt = np.zeros((self.B, self.H, cap * BLOCK), np.uint8)
        for b in range(self.B):
            for g in range(self.H):
                vt[b, g] = offset_codes_to_vtiles(self.v_out_u[b, g], 8)
        out["v_out_codes"] = vt
        out["k_out_scales"] = self.out_scales["k"].copy()
        out["v_out_scales"] = self.out_scales["v"].copy()
        return out


def outlier_values(planes, p, b, g, n):
    """Dequantized outlier values [n][32] (float32) of plane p ("k"/"v") of
    sequence b, KV head g, read from the physical planes."""
    from .blockquant import vtiles_to_codes, TILE
    if p == "k":
        codes = planes["k_out_codes"][b, g].view(np.int8).reshape(-1, BLOCK)[:n]
    else:
        n_t = (n + TILE - 1) // TILE * TILE
        codes = vtiles_to_codes(planes["v_out_codes"][b, g], n_t, BLOCK, 8)[:n]
    scales = planes[p + "_out_scales"][b, g][:n].reshape(n, 1)
    return dequantize_blocks(codes, scales)


def decode_reference_outliers(planes, q, lens, n_kv_heads, d, k_bits, v_bits, k_idx, v_idx,
                              sm_scale=None, rotate_k=True, rotate_v=True, sign_seed=0,
                              k_min=False, v_min=False):
    """Decode attention [B][Hq][d] (float64) over a cache with outlier sets
    (reading R25, no precision tail), in the split form of
    attention_outliers, from the physical planes."""
    from .kvcache import dequantize_rows
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _ = q.shape
    G = Hq // n_kv_heads
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    Rk = rotation_matrix(d, sign_seed) if rotate_k else np.eye(d)
    Rv = rotation_matrix(d, sign_seed) if rotate_v else np.eye(d)
    ki = np.asarray(k_idx, np.int64).reshape(n_kv_heads, BLOCK)
    vi = np.asarray(v_idx, np.int64).reshape(n_kv_heads, BLOCK)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        n = int(lens[b])
        for g in range(n_kv_heads):
            ky = dequantize_rows(planes["k_codes"][b, g], planes["k_scales"][b, g], d, k_bits, n, "k",
                                 k_min).astype(np.float64)
            vy = dequantize_rows(planes["v_codes"][b, g], planes["v_scales"][b, g], d, v_bits, n, "v",
                                 v_min).astype(np.float64)
            ko = outlier_values(planes, "k", b, g, n).astype(np.float64)
            vo = outlier_values(planes, "v", b, g, n).astype(np.float64)
            for h in range(g * G, (g + 1) * G):
                s = sm_scale * (ky @ (Rk @ q[b, h]) + ko @ q[b, h][ki[g]])
                s = s - np.max(s)
                p = np.exp(s)
                p = p / np.sum(p)
                o = Rv.T @ (p @ vy)
                o[vi[g]] += p @ vo
                out[b, h] = o
    return out
