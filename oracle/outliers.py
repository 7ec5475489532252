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
