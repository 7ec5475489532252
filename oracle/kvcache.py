"""Rotated, block-quantized KV cache with a bf16 precision tail (oracle).

Sources:
* velog.io post "fix KV cache quantization outliers", section "Hadamard
  rotation": K and V are rotated and then stored; only the store and the
  attention step change, the model file does not.  Section "the essence of
  the problem" names separate K and V cache types (--cache-type-k/-v).
* aitrends.kr article 92204, glossary entry "Precision Tail": the newest X
  tokens are kept in bf16 and the rest are stored low-bit.

Readings (the pages do not fix these):
* R5/R16  A tail token is stored as bf16(rotated value); when it leaves the
          tail it is quantized from that stored bf16 value, which is the same
          value a direct quantization uses when T > 0, so results do not
          depend on how appends are chunked.
* R11     The tail is a ring: position p lives in slot p mod T.  After an
          append that brings the length to n1, positions [n1 - T, n1) are in
          the tail and positions below n1 - T are quantized.
"""

import numpy as np

from .rotation import rotate_f32, hadamard_signs
from .blockquant import (
    BLOCK, TILE, quantize_blocks, dequantize_blocks, quantize_blocks_min,
    dequantize_blocks_min, pack_rows, unpack_rows,
    row_bytes, padded_row_bytes, rows_to_tiled, tiled_to_rows,
    offset_codes_to_vtiles, vtiles_to_codes, v_tile_bytes,
    f32_to_bf16_bits, bf16_bits_to_f32,
)


def _widen(x, dtype):
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError("dtype must be 'bf16' (uint16 bit patterns) or 'f32'")


class OracleCache:
    """Logical model of the cache for B sequences x Hkv KV heads.

    Rows are kept in logical order; physical() returns the planes in the
    tiled byte layout (reading R11) so they can be compared byte for byte.
    """

    def __init__(self, batch, n_kv_heads, head_dim, k_bits, v_bits,
                 tail_len, max_ctx, rotate_k=True, rotate_v=True, sign_seed=0,
                 k_min=False, v_min=False):
        self.B, self.H, self.d = batch, n_kv_heads, head_dim
        self.signs = hadamard_signs(head_dim, sign_seed)      # reading R21
        self.minf = {"k": bool(k_min), "v": bool(v_min)}      # reading R22
        self.bits = {"k": k_bits, "v": v_bits}
        self.rot = {"k": bool(rotate_k), "v": bool(rotate_v)}
        self.T = int(tail_len)
        self.max_ctx = int(max_ctx)
        self.cap = (self.max_ctx + TILE - 1) // TILE * TILE
        nb = head_dim // BLOCK
        self.rows, self.scales, self.tail = {}, {}, {}
        for p in ("k", "v"):
            self.rows[p] = np.zeros((batch, n_kv_heads, self.cap,
                                     row_bytes(head_dim, self.bits[p])), np.uint8)
        # V codes as offset codes u = c + 2^(bits-1) (u = 0: never written)
        self.v_u = np.zeros((batch, n_kv_heads, self.cap, head_dim), np.uint8)
        for p in ("k", "v"):
            # symmetric: one fp16 scale per block; scale-and-min: (s, m) pairs
            per = 2 if self.minf[p] else 1
            self.scales[p] = np.zeros((batch, n_kv_heads, self.cap, nb * per), np.uint16)
            self.tail[p] = np.zeros((batch, n_kv_heads, max(self.T, 0), head_dim), np.uint16)

    def append(self, k_new, v_new, lens, dtype="bf16"):
        """Append n_new tokens per sequence; k_new/v_new are [B][n_new][Hkv][d].

        lens[b] is the length before the append.  Returns the new lengths."""
        lens = np.asarray(lens, dtype=np.int64)
        n_new = np.asarray(k_new).shape[1]
        if np.any(lens + n_new > self.max_ctx):
            raise ValueError("append exceeds max_ctx")
        for p, new in (("k", k_new), ("v", v_new)):
            x = _widen(new, dtype)
            y = rotate_f32(x, self.rot[p], self.signs)      # [B][n][H][d]
            for b in range(self.B):
                self._append_one(p, b, y[b], int(lens[b]))
        return lens + n_new

    def _append_one(self, p, b, y, length):
        """y: [n_new][H][d] rotated float32 values for sequence b."""
        T, bits = self.T, self.bits[p]
        n_new = y.shape[0]
        n1 = length + n_new
        q_end = n1 - T if T > 0 else n1          # positions below q_end are quantized
        # 1. tokens leaving the tail: quantize their stored bf16 values
        if T > 0:
            for pp in range(max(0, length - T), min(length, q_end)):
                xq = bf16_bits_to_f32(self.tail[p][b, :, pp % T, :])    # [H][d]
                self._store_quantized(p, b, pp, xq, bits)
        # 2. new tokens: quantize directly, or write to the tail
        xq_all = bf16_bits_to_f32(f32_to_bf16_bits(y)) if T > 0 else y
        for i in range(n_new):
            pos = length + i
            if pos < q_end:
                self._store_quantized(p, b, pos, xq_all[i], bits)
            else:
                self.tail[p][b, :, pos % T, :] = f32_to_bf16_bits(y[i])

    def _store_quantized(self, p, b, pos, xq, bits):
        if self.minf[p]:
            codes, pairs = quantize_blocks_min(xq, bits)      # [H][d], [H][d/32][2]
            scales = pairs.reshape(pairs.shape[0], -1)
        else:
            codes, scales = quantize_blocks(xq, bits)         # [H][d], [H][d/32]
        self.rows[p][b, :, pos, :] = pack_rows(codes, bits)
        self.scales[p][b, :, pos, :] = scales
        if p == "v":
            self.v_u[b, :, pos, :] = codes.astype(np.int16) + (1 << (bits - 1))

    def physical(self):
        """Planes in the device byte layout (reading R11): K rows tiled in
        16-byte chunks, V codes in element-major tiles."""
        out = {}
        for p in ("k", "v"):
            bits = self.bits[p]
            if p == "k":
                pad = padded_row_bytes(self.d, bits)
                planes = np.zeros((self.B, self.H, self.cap * pad), np.uint8)
                for b in range(self.B):
                    for g in range(self.H):
                        planes[b, g] = rows_to_tiled(self.rows[p][b, g], pad)
            else:
                planes = np.zeros((self.B, self.H, self.cap // TILE * v_tile_bytes(self.d, bits)),
                                  np.uint8)
                for b in range(self.B):
                    for g in range(self.H):
                        planes[b, g] = offset_codes_to_vtiles(self.v_u[b, g], bits)
            out[p + "_codes"] = planes
            out[p + "_scales"] = self.scales[p].copy()
            out[p + "_tail"] = self.tail[p].copy()
        return out


def planes_to_rows(codes_plane, d, bits, n):
    """Physical K code plane of one (b, g) -> logical rows of the first n tokens."""
    pad = padded_row_bytes(d, bits)
    n_t = (n + TILE - 1) // TILE * TILE
    return tiled_to_rows(codes_plane, n_t, pad, row_bytes(d, bits))[:n]


def plane_codes(codes_plane, d, bits, n, which):
    """Int codes [n][d] of the first n tokens of one (b, g) plane; which is
    "k" (row layout) or "v" (element-major tiles)."""
    if which == "k":
        return unpack_rows(planes_to_rows(codes_plane, d, bits, n), bits, d)
    n_t = (n + TILE - 1) // TILE * TILE
    return vtiles_to_codes(codes_plane, n_t, d, bits)[:n]


def dequantize_rows(codes_plane, scales_plane, d, bits, n, which, minf=False):
    """Dequantized values (rotated space, float32) of quantized rows [0, n);
    minf selects the scale-and-min blocks of reading R22."""
    codes = plane_codes(codes_plane, d, bits, n, which)
    if minf:
        pairs = np.asarray(scales_plane[:n]).reshape(n, d // BLOCK, 2)
        return dequantize_blocks_min(codes, pairs, bits)
    return dequantize_blocks(codes, scales_plane[:n])


def pages_to_contiguous(pool, table, n_kv_heads, tile_size):
    """Gather one paged plane into the contiguous layout (reading R24).

    The pages fix no memory layout.  A paged cache keeps the 64-position
    tiles of its code and scale planes in a pool of pages shared by all
    sequences, one tile per KV head in each page, [page][g][tile]; the page
    table names the page of tile t of sequence b.  The contiguous layout
    orders the same tiles [b][g][t].

    pool:      array whose leading axis runs over pages * n_kv_heads tiles of
               tile_size elements each (any dtype; flattened).
    table:     int array [B][tiles]; an entry < 0 marks a tile that holds no
               positions, which comes back zero.
    Returns [B][n_kv_heads][tiles * tile_size] of pool's dtype.
    """
    table = np.asarray(table)
    B, tiles = table.shape
    flat = np.asarray(pool).reshape(-1)
    n_pages = flat.size // (n_kv_heads * tile_size)
    pages = flat[: n_pages * n_kv_heads * tile_size].reshape(n_pages, n_kv_heads, tile_size)
    out = np.zeros((B, n_kv_heads, tiles, tile_size), flat.dtype)
    for b in range(B):
        for t in range(tiles):
            page = int(table[b, t])
            if page >= 0:
                out[b, :, t, :] = pages[page]
    return out.reshape(B, n_kv_heads, tiles * tile_size)


def contiguous_to_pages(planes, table, n_pages, tile_size):
    """Scatter a contiguous plane [B][Hkv][tiles * tile_size] into a pool of
    n_pages pages (the inverse of pages_to_contiguous); pages no entry names
    stay zero.  Returns [n_pages][Hkv][tile_size]."""
    planes = np.asarray(planes)
    table = np.asarray(table)
    B, H = planes.shape[:2]
    tiles = table.shape[1]
    src = planes.reshape(B, H, tiles, tile_size)
    pool = np.zeros((n_pages, H, tile_size), planes.dtype)
    for b in range(B):
        for t in range(tiles):
            page = int(table[b, t])
            if page >= 0:
                pool[page] = src[b, :, t, :]
    return pool
