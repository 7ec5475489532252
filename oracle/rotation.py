"""Normalized Hadamard rotation (oracle, test infrastructure only).

Source: velog.io post "fix KV cache quantization outliers", section
"Hadamard rotation": Q, K and V are multiplied by a normalized Hadamard
matrix before K/V enter the cache, and the attention output is rotated back;
the matrix is orthogonal, so dot products (and hence attention scores) are
unchanged.  The section "application and background" enables the rotation
when head_dim is at least 64 and a multiple of 64.

Readings (the page does not fix these):
* R1  The matrix is Sylvester's construction in natural order with no random
      sign diagonal: H[i, j] = (-1)^popcount(i & j) / sqrt(d).
* R3  Normalization is one float32 multiply by fp32(1/sqrt(d)) applied after
      the unnormalized transform.
* R4  The float32 fast Walsh-Hadamard transform runs its stages in the order
      h = 1, 2, 4, ..., d/2 with butterflies (a + b, a - b); the order changes
      rounding, so it is fixed here and the GPU follows it.
* R21 Randomized-sign variant (a direction the velog.io post names in section
      "application and background", with no algorithm): R = H diag(s) with
      s_e = +-1 taken from SplitMix64 (Steele, Lea and Flood, "Fast splittable
      pseudorandom number generators", OOPSLA 2014) of the 64-bit counter
      seed * 2^32 + e: s_e = -1 iff the top bit of the output is set.  Seed 0
      is the plain matrix of R1.  A vector is rotated as H (s * x) and rotated
      back as s * (H y); sign flips are exact, so the float32 transform and
      its stage order are unchanged.
* R23 head_dim a multiple of 64 but not a power of two (the rule of section
      "application and background" admits it; no Sylvester matrix of that
      size exists): the rotation is block-diagonal, one normalized H_64 per
      consecutive group of 64 elements, each group transformed as in R3/R4
      with stages h = 1..32 and the factor fp32(1/8).
"""

import numpy as np


def hadamard(d):
    """Dense normalized Sylvester Hadamard matrix in float64 (plain definition).

    H[i, j] = (-1)^popcount(i & j) / sqrt(d); symmetric and orthogonal, so it
    is its own inverse (velog.io post, section "Hadamard rotation").
    """
    if d < 1 or d & (d - 1):
        raise ValueError("Sylvester Hadamard needs a power-of-two size")
    i = np.arange(d, dtype=np.int64)
    anded = i[:, None] & i[None, :]
    parity = np.zeros_like(anded)
    x = anded.copy()
    while np.any(x):
        parity ^= x & 1
        x >>= 1
    return np.where(parity == 1, -1.0, 1.0) / np.sqrt(float(d))


_M64 = (1 << 64) - 1


def splitmix64(x):
    """One SplitMix64 output for the 64-bit counter x (published mixing
    function: add the golden-gamma increment, then two xor-shift-multiply
    rounds and a final xor-shift)."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def hadamard_signs(d, seed):
    """The sign vector s (float64 +-1, length d) of reading R21, or None for
    seed 0 (no signs)."""
    if seed == 0:
        return None
    seed &= 0xFFFFFFFF
    return np.array([-1.0 if splitmix64((seed << 32) | e) >> 63 else 1.0 for e in range(d)])


def rotation_block(d):
    """Size of the Hadamard blocks the rotation of a d-vector uses: d itself
    for a power of two, 64 for other multiples of 64 (reading R23)."""
    if d >= 1 and d & (d - 1) == 0:
        return d
    if d % 64 == 0:
        return 64
    raise ValueError("the rotation needs a power of two or a multiple of 64")


def block_hadamard(d):
    """Dense float64 rotation matrix of reading R23: block-diagonal with
    normalized H_b blocks, b = rotation_block(d) (H_d itself when b = d)."""
    b = rotation_block(d)
    return np.kron(np.eye(d // b), hadamard(b))


def rotation_matrix(d, seed=0):
    """Dense R = H diag(s) in float64 (H alone for seed 0; H block-diagonal
    for a d that is not a power of two, reading R23)."""
    H = block_hadamard(d)
    s = hadamard_signs(d, seed)
    return H if s is None else H * s[None, :]


def rot_scale_f32(d):
    """fp32(1/sqrt(d)): the normalization constant of reading R3."""
    return np.float32(1.0 / np.sqrt(np.float64(d)))


def fwht_f32(x, block=None):
    """Unnormalized fast Walsh-Hadamard transform along the last axis, float32.

    Stage order h = 1, 2, ..., d/2 (reading R4); in each stage every index i
    with (i & h) == 0 pairs with i + h and becomes (x[i] + x[i+h],
    x[i] - x[i+h]), each rounded to float32.  No fused operations.
    The result equals sqrt(d) * H @ x up to float32 rounding.  With block,
    each consecutive group of block elements is transformed on its own
    (stages h < block; reading R23).
    """
    x = np.array(x, dtype=np.float32, copy=True)
    d = x.shape[-1]
    n = d if block is None else block
    if n < 1 or n & (n - 1) or d % n:
        raise ValueError("FWHT needs a power-of-two length")
    lead = x.shape[:-1]
    h = 1
    while h < n:
        v = x.reshape(lead + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        x = v.reshape(lead + (d,))
        h *= 2
    return x


def rotate_f32(x, enabled=True, signs=None):
    """y = fp32(1/sqrt(d)) * FWHT(s * x) in float32, or x unchanged if disabled.

    velog.io post, section "Hadamard rotation" (rotate before storing);
    readings R1, R3, R4, R21 (signs: a +-1 vector or None).  The per-plane
    switch follows the separate K and V disable variables named in section
    "application and background".
    """
    x = np.asarray(x, dtype=np.float32)
    if not enabled:
        return x.copy()
    if signs is not None:
        x = x * np.asarray(signs, dtype=np.float32)
    b = rotation_block(x.shape[-1])
    return fwht_f32(x, b) * rot_scale_f32(b)


def unrotate_f32(y, enabled=True, signs=None):
    """The inverse rotation in float32: s * (fp32(1/sqrt(d)) * FWHT(y)), or y
    unchanged if disabled (H is symmetric and orthogonal; R21)."""
    y = np.asarray(y, dtype=np.float32)
    if not enabled:
        return y.copy()
    b = rotation_block(y.shape[-1])
    out = fwht_f32(y, b) * rot_scale_f32(b)
    if signs is not None:
        out = out * np.asarray(signs, dtype=np.float32)
    return out
