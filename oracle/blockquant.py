"""32-element block quantization with one fp16 absmax scale (oracle, test only).

Sources:
* velog.io post "fix KV cache quantization outliers", section "the essence of
  the problem": the quantization scale is set by the few extreme values of a
  group, which is why outliers crush the small values (absmax scaling).
* aiwitness.kr post 1txlhxu, table "Qwen 3.6 27B Q5_K_S + 64k context KLD
  results": q4_0 / q5_0 / q6_0 / q8_0 caches cost 28.1 / 34.4 / 40.6 / 53.1 %
  of bf16, i.e. 4.5 / 5.5 / 6.5 / 8.5 bits per value = 32 codes plus one
  2-byte scale.
* aitrends.kr article 92204, glossary entry "Precision Tail": the newest
  tokens are kept in bf16.

The quantizer is an encoding, so every float32 operation is spelled out and
the GPU reproduces it bit for bit.  Readings (the pages do not fix these):
* R5  With a bf16 tail (T > 0) the rotated value is rounded to bf16 before it
      is quantized, so a token gets the same codes whether or not it passed
      through the tail.  With T = 0 the float32 value is quantized directly.
* R6  Symmetric codes c in [-qmax, qmax], qmax = 2^(b-1) - 1; no zero point.
* R7  scale = fp16_rne(min(absmax / qmax, 65504)), divide correctly rounded.
* R8  codes = clip(rint(x * r), -qmax, qmax) with r = 1 / fp32(scale)
      (one correctly rounded divide per block, one multiply per element),
      rint ties to even.
* R9  A block whose fp16 scale is 0 gets all-zero codes.
* R10 Code storage: 8-bit codes are two's-complement bytes.  4-bit codes are
      offset binary u = c + 8, two per byte, even element in the low nibble.
      5-bit codes are offset binary u = c + 16: the low four bits form a
      4-bit nibble plane (d/2 bytes, packed like 4-bit), followed by one
      little-endian 32-bit word per block holding bit 4 of each code; element
      w of the block (0..31) owns bit 8*((w%8)//2) + 2*(w//8) + (w%2).
      6-bit codes are offset binary u = c + 32: the same nibble plane, then
      two little-endian 32-bit words per block holding bits 4-5 of each code;
      element w owns the two bits from bit 8*((w%8)//2) + 4*((w//8)%2) +
      2*(w%2) of word w//16 (bit 4 of u first).
* R11 Memory layout of a K code plane: rows are padded to a multiple of 16
      bytes and grouped in tiles of 64 tokens; inside a tile, the 16-byte
      chunk c of the row of token l sits at byte (c*64 + l)*16.  Scale planes
      are plain [token][d/32] fp16.
* R11 V code planes keep the same codes but store each 64-token tile
      element-major, so that the eight codes of one element for eight
      consecutive tokens sit together: token t, element e of a tile belong to
      item ((t//32)*64 + 16*((t%32)//8) + e%16) * (d//16) + e//16, slot
      k = t%8 of that item.  4-bit: one little-endian 32-bit word per item,
      u = c + 8 of slot k in nibble 4*(k%2) + k//2.  8-bit: eight bytes per
      item, u = c + 128 in byte k.  5-bit: the 4-bit words of u & 15 for all
      items (32*d bytes per tile), then one byte per item whose bit
      4*(k%2) + k//2 is bit 4 of u.  6-bit: the 4-bit words of u & 15, then
      one little-endian 16-bit field per item whose bits 2n and 2n+1, with
      n = 4*(k%2) + k//2, are bits 4 and 5 of u.
* R22 Scale-and-min blocks q4_1 / q5_1 (the aiwitness.kr table's q5_1 rows, 37.5 %
      of bf16 = 5 bits plus two 2-byte values per 32; the aitrends.kr article
      names a q5_0-q4_1 pair): per block lo = min x, hi = max x, s =
      fp16_rne(min(fp32(hi - lo) / (2^b - 1), 65504)), m = fp16_rne(lo clamped
      to +-65504), r = 1 / fp32(s), u = clip(rint(fp32(fp32(x - m) * r)), 0,
      2^b - 1) (all 0 if s == 0); x_hat = fp32(u * s + m).  The scale plane
      holds the (s, m) pair of each block; the code planes hold u exactly
      where the symmetric formats hold c + 2^(b-1), so they are laid out by
      the same rules with c = u - 2^(b-1).
"""

import numpy as np

BLOCK = 32
QMAX = {4: 7, 5: 15, 6: 31, 8: 127}
TILE = 64
CHUNK = 16


def f32_to_bf16_bits(x):
    """Round float32 to bfloat16 with round-to-nearest-even; returns uint16 bits.

    NaN and infinity are outside the contract (reading R9)."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    b = b.astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen bfloat16 bits to float32 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_round(x):
    """float32 -> nearest bfloat16 value (ties to even), returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def quantize_blocks(xq, bits):
    """Quantize float32 rows of length d (a multiple of 32), block by block.

    Returns (codes, scales): codes int8 [..., d] in [-qmax, qmax]; scales
    uint16 [..., d/32] holding fp16 bit patterns.  Steps (readings R6-R9):
      a   = max |x| over the block                      (exact)
      s32 = a / qmax                                    (float32, IEEE divide)
      s16 = fp16_rne(min(s32, 65504))
      r   = 1 / float32(s16)                            (float32, IEEE divide)
      c   = clip(rint(float32(x * r)), -qmax, qmax)     (0 if s16 == 0)
    """
    if bits not in QMAX:
        raise ValueError("bits must be 4, 5, 6 or 8")
    qmax = np.float32(QMAX[bits])
    x = np.asarray(xq, dtype=np.float32)
    d = x.shape[-1]
    if d % BLOCK:
        raise ValueError("row length must be a multiple of 32")
    blocks = x.reshape(x.shape[:-1] + (d // BLOCK, BLOCK))
    a = np.max(np.abs(blocks), axis=-1)
    s32 = a / qmax
    s32 = np.minimum(s32, np.float32(65504.0))
    s16 = s32.astype(np.float16)
    s16f = s16.astype(np.float32)
    nz = s16f != 0
    r = np.where(nz, np.float32(1.0) / np.where(nz, s16f, np.float32(1.0)),
                 np.float32(0.0)).astype(np.float32)
    prod = (blocks * r[..., None]).astype(np.float32)
    c = np.clip(np.rint(prod), -qmax, qmax)
    c = np.where(nz[..., None], c, np.float32(0.0))
    codes = c.astype(np.int8).reshape(x.shape)
    return codes, s16.view(np.uint16)


def quantize_blocks_min(xq, bits):
    """Scale-and-min quantization of float32 rows (reading R22).

    Returns (codes, pairs): codes int8 [..., d] holding u - 2^(bits-1) (the
    storage convention of the symmetric formats); pairs uint16 [..., d/32, 2]
    holding the fp16 bits of (s, m)."""
    if bits not in (4, 5):
        raise ValueError("scale-and-min blocks are 4 or 5 bits")
    umax = np.float32((1 << bits) - 1)
    x = np.asarray(xq, dtype=np.float32)
    d = x.shape[-1]
    blocks = x.reshape(x.shape[:-1] + (d // BLOCK, BLOCK))
    lo = np.min(blocks, axis=-1)
    hi = np.max(blocks, axis=-1)
    s32 = (hi - lo).astype(np.float32) / umax
    s16 = np.minimum(s32, np.float32(65504.0)).astype(np.float16)
    m16 = np.clip(lo, np.float32(-65504.0), np.float32(65504.0)).astype(np.float16)
    sf = s16.astype(np.float32)
    mf = m16.astype(np.float32)
    nz = sf != 0
    r = np.where(nz, np.float32(1.0) / np.where(nz, sf, np.float32(1.0)),
                 np.float32(0.0)).astype(np.float32)
    t = ((blocks - mf[..., None]).astype(np.float32) * r[..., None]).astype(np.float32)
    u = np.clip(np.rint(t), np.float32(0), umax)
    u = np.where(nz[..., None], u, np.float32(0.0))
    codes = (u.astype(np.int16) - (1 << (bits - 1))).astype(np.int8).reshape(x.shape)
    pairs = np.stack([s16.view(np.uint16), m16.view(np.uint16)], axis=-1)
    return codes, pairs


def dequantize_blocks_min(codes, pairs, bits):
    """x_hat = fp32(u * s + m) with u = code + 2^(bits-1): u * s is exact
    (at most 5 + 11 significant bits), so the single rounding of the sum
    leaves one right answer (reading R22)."""
    u = np.asarray(codes, dtype=np.int16).astype(np.float32) + np.float32(1 << (bits - 1))
    d = u.shape[-1]
    pr = np.asarray(pairs, dtype=np.uint16).view(np.float16).astype(np.float32)
    s = pr[..., 0]
    m = pr[..., 1]
    out = u.reshape(u.shape[:-1] + (d // BLOCK, BLOCK)) * s[..., None] + m[..., None]
    return out.reshape(u.shape).astype(np.float32)


def dequantize_blocks(codes, scales_bits):
    """x_hat = float32(c) * float32(scale): exact in float32 (at most
    8 + 11 significant bits), so there is one right answer."""
    c = np.asarray(codes, dtype=np.int8).astype(np.float32)
    d = c.shape[-1]
    s = np.asarray(scales_bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    out = c.reshape(c.shape[:-1] + (d // BLOCK, BLOCK)) * s[..., None]
    return out.reshape(c.shape).astype(np.float32)


def row_bytes(d, bits):
    """Packed bytes of one head vector: d*bits/8 (reading R10)."""
    return d * bits // 8


def padded_row_bytes(d, bits):
    """Row bytes rounded up to the 16-byte chunk of the tiled layout (R11)."""
    r = row_bytes(d, bits)
    return (r + CHUNK - 1) // CHUNK * CHUNK


def _hibit_position(w):
    """Bit of the 5-bit high-bit word owned by element w of a block (R10)."""
    return 8 * ((w % 8) // 2) + 2 * (w // 8) + (w % 2)


def _hi2_position(w):
    """First bit of the 2-bit field of element w inside 6-bit high word w//16
    of its block (R10)."""
    return 8 * ((w % 8) // 2) + 4 * ((w // 8) % 2) + 2 * (w % 2)


def pack_rows(codes, bits):
    """Pack int8 codes [..., d] into uint8 rows [..., row_bytes] (reading R10)."""
    c = np.asarray(codes, dtype=np.int16)
    d = c.shape[-1]
    lead = c.shape[:-1]
    if bits == 8:
        return c.astype(np.int8).view(np.uint8).reshape(lead + (d,))
    if bits == 4:
        u = (c + 8).astype(np.uint8)
        return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)
    if bits == 5:
        u = (c + 16).astype(np.uint16)
        lo = (u & 15).astype(np.uint8)
        nib = (lo[..., 0::2] | (lo[..., 1::2] << 4)).astype(np.uint8)
        hb = ((u >> 4) & 1).astype(np.uint32)
        hb = hb.reshape(lead + (d // BLOCK, BLOCK))
        pos = np.array([_hibit_position(w) for w in range(BLOCK)], dtype=np.uint32)
        words = np.zeros(lead + (d // BLOCK,), dtype=np.uint32)
        for w in range(BLOCK):
            words |= hb[..., w] << pos[w]
        hi = words.astype("<u4").view(np.uint8).reshape(lead + (d // 8,))
        return np.concatenate([nib, hi], axis=-1)
    if bits == 6:
        u = (c + 32).astype(np.uint16)
        lo = (u & 15).astype(np.uint8)
        nib = (lo[..., 0::2] | (lo[..., 1::2] << 4)).astype(np.uint8)
        h2 = ((u >> 4) & 3).astype(np.uint32).reshape(lead + (d // BLOCK, BLOCK))
        words = np.zeros(lead + (d // BLOCK, 2), dtype=np.uint32)
        for w in range(BLOCK):
            words[..., w // 16] |= h2[..., w] << np.uint32(_hi2_position(w))
        hi = words.astype("<u4").view(np.uint8).reshape(lead + (d // 4,))
        return np.concatenate([nib, hi], axis=-1)
    raise ValueError("bits must be 4, 5, 6 or 8")


def unpack_rows(rows, bits, d):
    """Inverse of pack_rows: uint8 rows -> int8 codes [..., d]."""
    r = np.asarray(rows, dtype=np.uint8)
    lead = r.shape[:-1]
    if bits == 8:
        return r[..., :d].view(np.int8).copy()
    if bits == 4:
        b = r[..., : d // 2]
        u = np.empty(lead + (d,), dtype=np.int16)
        u[..., 0::2] = b & 15
        u[..., 1::2] = b >> 4
        return (u - 8).astype(np.int8)
    if bits == 5:
        b = r[..., : d // 2]
        lo = np.empty(lead + (d,), dtype=np.int16)
        lo[..., 0::2] = b & 15
        lo[..., 1::2] = b >> 4
        words = np.ascontiguousarray(r[..., d // 2: d // 2 + d // 8]).view("<u4")
        words = words.reshape(lead + (d // BLOCK,)).astype(np.uint32)
        hi = np.empty(lead + (d // BLOCK, BLOCK), dtype=np.int16)
        for w in range(BLOCK):
            hi[..., w] = (words >> np.uint32(_hibit_position(w))) & 1
        u = lo + 16 * hi.reshape(lead + (d,))
        return (u - 16).astype(np.int8)
    if bits == 6:
        b = r[..., : d // 2]
        lo = np.empty(lead + (d,), dtype=np.int16)
        lo[..., 0::2] = b & 15
        lo[..., 1::2] = b >> 4
        words = np.ascontiguousarray(r[..., d // 2: d // 2 + d // 4]).view("<u4")
        words = words.reshape(lead + (d // BLOCK, 2)).astype(np.uint32)
        hi = np.empty(lead + (d // BLOCK, BLOCK), dtype=np.int16)
        for w in range(BLOCK):
            hi[..., w] = (words[..., w // 16] >> np.uint32(_hi2_position(w))) & 3
        u = lo + 16 * hi.reshape(lead + (d,))
        return (u - 32).astype(np.int8)
    raise ValueError("bits must be 4, 5, 6 or 8")


def rows_to_tiled(rows, padded):
    """Logical rows [n][R] (n a multiple of 64) -> tiled plane bytes (R11).

    Byte (tile*64*padded) + (c*64 + l)*16 + k holds byte c*16 + k of the row of
    token tile*64 + l."""
    rows = np.asarray(rows, dtype=np.uint8)
    n, rlen = rows.shape
    if n % TILE:
        raise ValueError("token count must be a multiple of 64")
    full = np.zeros((n, padded), dtype=np.uint8)
    full[:, :rlen] = rows
    nch = padded // CHUNK
    t = full.reshape(n // TILE, TILE, nch, CHUNK).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(t).reshape(-1)


def tiled_to_rows(plane, n, padded, rlen):
    """Inverse of rows_to_tiled for the first n tokens (n a multiple of 64)."""
    plane = np.asarray(plane, dtype=np.uint8)
    nch = padded // CHUNK
    t = plane[: n * padded].reshape(n // TILE, nch, TILE, CHUNK).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(t).reshape(n, padded)[:, :rlen]


def v_tile_bytes(d, bits):
    """Bytes of one 64-token tile of a V code plane (reading R11)."""
    return TILE * d * bits // 8


def _v_item_index(d):
    """Token and element index arrays [2][64][d//16][8] of the V tile items
    (reading R11): item (j, lane, n), slot k holds token 32j + 8*(lane//16) + k
    and element 16n + lane % 16."""
    nn = d // 16
    j = np.arange(2)[:, None, None, None]
    lane = np.arange(64)[None, :, None, None]
    n = np.arange(nn)[None, None, :, None]
    k = np.arange(8)[None, None, None, :]
    t = 32 * j + 8 * (lane // 16) + k + 0 * n
    e = 16 * n + lane % 16 + 0 * k + 0 * j
    return t, e


# nibble (and high bit) position of slot k inside a 4-bit word / 5-bit byte
_V_NIBBLE = np.array([4 * (k % 2) + k // 2 for k in range(8)], dtype=np.uint32)


def codes_to_vtiles(codes, bits):
    """Int codes [n][d] (n a multiple of 64) -> V code plane bytes (R10, R11)."""
    c = np.asarray(codes, dtype=np.int16)
    return offset_codes_to_vtiles(c + (1 << (bits - 1)), bits)


def offset_codes_to_vtiles(u, bits):
    """Offset codes u = c + 2^(bits-1) [n][d] -> V code plane bytes.  Every
    stored code has u >= 1, so u = 0 marks a slot that was never written and
    becomes zero bits, as in a zero-filled plane."""
    u = np.asarray(u, dtype=np.int16)
    n, d = u.shape
    if n % TILE:
        raise ValueError("token count must be a multiple of 64")
    t, e = _v_item_index(d)
    u = u.reshape(n // TILE, TILE, d)
    items = u[:, t, e].astype(np.uint32)          # [tiles][2][64][d/16][8]
    nt = n // TILE
    if bits == 8:
        return items.astype(np.uint8).reshape(-1)
    if bits not in (4, 5, 6):
        raise ValueError("bits must be 4, 5, 6 or 8")
    words = np.zeros(items.shape[:-1], dtype=np.uint32)
    for k in range(8):
        words |= (items[..., k] & 15) << (4 * _V_NIBBLE[k])
    nib = words.astype("<u4").view(np.uint8).reshape(nt, -1)
    if bits == 4:
        return nib.reshape(-1)
    if bits == 6:
        h2 = np.zeros(items.shape[:-1], dtype=np.uint32)
        for k in range(8):
            h2 |= ((items[..., k] >> 4) & 3) << (2 * _V_NIBBLE[k])
        hib = h2.astype("<u2").view(np.uint8).reshape(nt, -1)
        return np.concatenate([nib, hib], axis=1).reshape(-1)
    hi = np.zeros(items.shape[:-1], dtype=np.uint32)
    for k in range(8):
        hi |= ((items[..., k] >> 4) & 1) << _V_NIBBLE[k]
    return np.concatenate([nib, hi.astype(np.uint8).reshape(nt, -1)], axis=1).reshape(-1)


def vtiles_to_codes(plane, n, d, bits):
    """Inverse of codes_to_vtiles for the first n tokens (n a multiple of 64)."""
    plane = np.asarray(plane, dtype=np.uint8)
    nt = n // TILE
    tb = v_tile_bytes(d, bits)
    tiles = plane[: nt * tb].reshape(nt, tb)
    shape = (nt, 2, 64, d // 16)
    if bits == 8:
        items = tiles.reshape(shape + (8,)).astype(np.int16)
    elif bits in (4, 5, 6):
        words = np.ascontiguousarray(tiles[:, : 32 * d]).view("<u4").reshape(shape).astype(np.uint32)
        items = np.stack([(words >> (4 * _V_NIBBLE[k])) & 15 for k in range(8)], axis=-1)
        if bits == 5:
            hi = tiles[:, 32 * d:].reshape(shape).astype(np.uint32)
            items = items | np.stack([((hi >> _V_NIBBLE[k]) & 1) << 4 for k in range(8)], axis=-1)
        if bits == 6:
            h2 = np.ascontiguousarray(tiles[:, 32 * d:]).view("<u2").reshape(shape).astype(np.uint32)
            items = items | np.stack([((h2 >> (2 * _V_NIBBLE[k])) & 3) << 4 for k in range(8)], axis=-1)
        items = items.astype(np.int16)
    else:
        raise ValueError("bits must be 4, 5, 6 or 8")
    t, e = _v_item_index(d)
    u = np.zeros((nt, TILE, d), dtype=np.int16)
    u[:, t, e] = items
    return (u.reshape(n, d) - (1 << (bits - 1))).astype(np.int8)
