"""CPU oracle for rotated low-bit KV-cache quantization and decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this package.  The HIP library
never calls it, shares no code with it, and must fail loudly if it is missing
rather than fall back to anything here.

What the oracle computes, and where each step comes from:

* Rotation: each K/V head vector (and the query) is multiplied by the
  normalized Hadamard matrix; the attention result is rotated back afterwards.
  Source: velog.io post "fix KV cache quantization outliers", section
  "Hadamard rotation" (the paragraphs on the computation, on orthogonality
  preserving dot products, and on outlier spreading).
* Block quantization: 32-element blocks, one 2-byte scale each, 4/5/8-bit
  codes.  The byte cost is fixed by the cache-size column of the table
  "Qwen 3.6 27B Q5_K_S + 64k context KLD results" on aiwitness.kr post
  1txlhxu (q4_0 28.1 %, q5_0 34.4 %, q8_0 53.1 % of bf16).
* Precision tail: the newest tokens stay in bf16, the rest are quantized.
  Source: aitrends.kr article 92204, glossary entry "Precision Tail" and the
  detail section on tail length.
* Paged planes (pages_to_contiguous): a storage layout the pages do not
  describe (reading R24); the functions only move whole 64-position tiles.
* Outlier channels at 8 bits (oracle.outliers, reading R25): the mixed
  precision the velog.io post names in section "application and
  background".  The GPU path builds it for 32 channels, no precision tail,
  head_dim 128 and absmax blocks.

Everything the pages leave open (Hadamard ordering, fp32 association of the
transform, rounding of the scale, code encoding, memory layout) is a stated
reading; each reading is named where it is implemented.

Functions that have a plain mathematical definition (the Hadamard product,
softmax attention) are written as that definition in float64.  The quantizer
is an encoding, so it is written step by step in float32 with every rounding
spelled out, because the GPU must reproduce its bytes exactly.

Parity status: every function here is pinned by tests under tests/ against
properties the pages or mathematics fix (orthogonality, dot-product
preservation, brute-force argmin quantization, the page-3 byte counts, chunk
invariance, textbook attention).  The exact byte values of codes are pinned
only by this specification plus those invariants; the pages print no worked
example or test vector (parity unpinned against any external implementation).
"""

from .rotation import (hadamard, rot_scale_f32, fwht_f32, rotate_f32, unrotate_f32,
                       hadamard_signs, rotation_matrix, splitmix64, rotation_block,
                       block_hadamard)
from .blockquant import (
    QMAX, BLOCK, bf16_round, bf16_bits_to_f32, f32_to_bf16_bits,
    quantize_blocks, dequantize_blocks, quantize_blocks_min, dequantize_blocks_min,
    pack_rows, unpack_rows,
    row_bytes, padded_row_bytes, rows_to_tiled, tiled_to_rows,
)
from .kvcache import OracleCache, pages_to_contiguous, contiguous_to_pages
from .attention import (softmax_attention, decode_reference, dequantize_unit,
                        dequantize_reference, prefill_reference)

__all__ = [
    "hadamard", "rot_scale_f32", "fwht_f32", "rotate_f32", "unrotate_f32",
    "hadamard_signs", "rotation_matrix", "splitmix64", "rotation_block", "block_hadamard",
    "QMAX", "BLOCK", "bf16_round", "bf16_bits_to_f32", "f32_to_bf16_bits",
    "quantize_blocks", "dequantize_blocks", "quantize_blocks_min", "dequantize_blocks_min",
    "pack_rows", "unpack_rows",
    "row_bytes", "padded_row_bytes", "rows_to_tiled", "tiled_to_rows",
    "OracleCache", "softmax_attention", "decode_reference", "prefill_reference", "dequantize_unit",
    "dequantize_reference", "pages_to_contiguous", "contiguous_to_pages",
]
