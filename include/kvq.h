/*
 * kvq — rotated low-bit KV cache and single-query decode attention for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The method (sources are the three public pages this library is built from):
 *  - Each K/V head vector is multiplied by a normalized Hadamard matrix before
 *    it is stored, which spreads outlier channels; attention runs on rotated
 *    q and K (the matrix is orthogonal, so scores are unchanged) and the
 *    output is rotated back.  velog.io post "fix KV cache quantization
 *    outliers", section "Hadamard rotation".  Rotation is on by default when
 *    head_dim >= 64 and a multiple of 64, and can be switched off separately
 *    for K and V (same post, section "application and background").
 *  - Rotated vectors are stored as 32-element blocks: one fp16 absmax scale
 *    plus 4-, 5-, 6- or 8-bit codes, i.e. 4.5 / 5.5 / 6.5 / 8.5 bits per
 *    value, the q4_0 / q5_0 / q6_0 / q8_0 cache sizes (28.1 / 34.4 / 40.6 /
 *    53.1 % of bf16) in the table "Qwen 3.6 27B Q5_K_S + 64k context KLD
 *    results" of aiwitness.kr post 1txlhxu.  4- and 5-bit blocks may instead
 *    carry an fp16 scale and an fp16 minimum (q4_1 / q5_1; q5_1 is 37.5 % in
 *    the same table).  K and V pick their widths independently
 *    (--cache-type-k / --cache-type-v in the velog.io post).
 *  - An optional bf16 precision tail keeps the newest tokens unquantized
 *    (aitrends.kr article 92204, glossary entry "Precision Tail").
 *
 * Conventions shared by every call:
 *  - Ownership: the caller allocates and frees every device buffer; the
 *    library never allocates device memory and keeps no global state, so
 *    calls are re-entrant.  The one exception is the static workspace of
 *    kvq_decode_attention_static, a fixed device array the library holds on
 *    each GPU it runs on.  Host arrays (seq_len) are read during the call
 *    only.
 *  - Execution: all device work is queued on `stream` (a hipStream_t passed
 *    as void*; NULL is the default stream) and is asynchronous.
 *  - Errors: every argument is validated on the host before any device work
 *    is queued; a failed validation returns a negative status and queues
 *    nothing.  A failed kernel launch returns KVQ_ERR_HIP.  Errors raised by
 *    the device later surface from the HIP runtime on the caller's next
 *    synchronisation.
 *  - Device pointers must be 16-byte aligned (KVQ_ERR_ALIGN otherwise; the
 *    page table of a paged cache 4-byte aligned).  A paged cache without a
 *    page table is KVQ_ERR_INVALID, and so is a negative page_pool.
 *
 * Cache memory layout (all planes indexed by sequence b and KV head g,
 * cap = max_ctx rounded up to a multiple of 64 tokens):
 *  - K code plane (k_codes): per (b, g) a block of cap * R bytes, where
 *    R = head_dim * bits / 8 rounded up to a multiple of 16.  Tokens are
 *    grouped in tiles of 64; inside a tile, bytes [16c, 16c+16) of the row
 *    of token l live at byte (c * 64 + l) * 16.  Row encoding:
 *      8-bit  two's-complement code per element;
 *      4-bit  u = code + 8, element 2i in the low nibble of byte i,
 *             element 2i+1 in the high nibble;
 *      5-bit  u = code + 16: low nibbles packed as 4-bit (head_dim/2 bytes),
 *             then one little-endian 32-bit word per block holding bit 4 of
 *             each code; element w of the block owns bit
 *             8*((w%8)/2) + 2*(w/8) + (w%2);
 *      6-bit  u = code + 32: low nibbles as 4-bit, then two little-endian
 *             32-bit words per block holding bits 4-5 of each code; element
 *             w owns bits 8*((w%8)/2) + 4*((w/8)%2) + 2*(w%2) and the next
 *             one of word w/16.
 *    Row padding bytes are never read or written.
 *  - V code plane (v_codes): per (b, g) cap/64 tiles of 64*head_dim*bits/8
 *    bytes, element-major: token t (0..63 in its tile) and element e belong
 *    to item ((t/32)*64 + 16*((t%32)/8) + e%16)*(head_dim/16) + e/16, slot
 *    k = t%8, with offset codes u = code + 2^(bits-1):
 *      4-bit  one little-endian 32-bit word per item, slot k in nibble
 *             n(k) = 4*(k%2) + k/2;
 *      8-bit  eight bytes per item, slot k in byte k;
 *      5-bit  the 4-bit words of u & 15 for all items (32*head_dim bytes),
 *             then one byte per item whose bit n(k) is bit 4 of u;
 *      6-bit  the 4-bit words, then one little-endian 16-bit field per item
 *             whose bits 2n(k), 2n(k)+1 are bits 4, 5 of u.
 *  - scale planes (k_scales, v_scales): [b][g][cap][head_dim/32] fp16, or
 *    [b][g][cap][head_dim/32][2] fp16 (s, m) pairs for scale-and-min blocks.
 *    Attention reads the entries of positions past seq_len up to the end of
 *    their 64-token tile (weighting them by zero), so the scale planes must
 *    hold finite values there: zero them once when the cache is allocated.
 *  - tail planes (k_tail, v_tail): [b][g][tail_len][head_dim] bf16; position
 *    p of the newest tail_len positions lives in slot p % tail_len.  NULL is
 *    allowed when tail_len == 0.
 *  - paged caches (page_pool > 0): the K code, V code and scale planes are
 *    a pool of page_pool pages of KVQ_PAGE_TOKENS (64) positions shared by
 *    all sequences, each page holding one 64-token tile per KV head:
 *    [page][g][tile], with the tile formats above (K rows tiled in 16-byte
 *    chunks, V element-major, scales [64][head_dim/32]).  Positions
 *    64t .. 64t+63 of sequence b live in page page_table[b][t].  The
 *    contiguous layout is the same tile sequence ordered [b][g][t].  Tail
 *    planes are not paged.  The pages name no cache layout; paging lets
 *    sequences of very different lengths share one pool, as serving stacks
 *    do.
 *
 * Quantization of one block of 32 rotated values x (bf16-rounded first when
 * tail_len > 0, so that a token gets the same codes whether or not it passed
 * through the tail):
 *    a = max|x|;  s = fp16_rne(min(a / qmax, 65504));  r = 1 / float(s);
 *    code = clamp(rint(x * r), -qmax, qmax)   (all codes 0 if s == 0)
 * with qmax = 7 / 15 / 31 / 127, IEEE float32 arithmetic, no fused operations.
 *
 * Scale-and-min blocks (k_min / v_min; 4 or 5 bits, the q4_1 / q5_1 formats,
 * whose size the aiwitness.kr table prints: two fp16 values per 32 elements):
 *    lo = min x, hi = max x;  s = fp16_rne(min((hi - lo) / (2^bits - 1), 65504));
 *    m = fp16_rne(lo clamped to +-65504);  r = 1 / float(s);
 *    u = clamp(rint((x - m) * r), 0, 2^bits - 1)   (all u 0 if s == 0)
 *    x_hat = u * s + m
 * The code planes store u where the absmax formats store code + 2^(bits-1),
 * so their layouts are the same.
 * Outlier channels (kvq_config.outliers = 32; the velog.io post, section
 * "application and background", names the mixed precision that keeps only
 * the outlier channels at 8 bits): each K and V head vector x splits before
 * rotation into x_O = x[O] (the 32 listed channels, in list order) and the
 * rest x_R = x with those channels zeroed.  x_R is rotated and stored by the
 * rules above; x_O stays in the original space as one 8-bit absmax block
 * (code = clamp(rint(x_O * r)), one fp16 scale).  Planes per (b, g), tiled
 * by 64 positions like the others: K outlier codes [cap][32] two's-
 * complement bytes; V outlier codes in element-major tiles of the V layout
 * at 8 bits for a 32-element head (item ((t/32)*64 + 16*((t%32)/8) +
 * o%16)*2 + o/16, byte t%8, u = code + 128); one fp16 scale per position
 * in each scale plane.  Attention splits exactly: q.x = (R q).y_R + q[O].x_O,
 * and the output is R^T (sum p y_V) plus sum p x_V,O added at V's channels.
 * The rotation is y = fp32(1/sqrt(d)) * FWHT(x) with the float32 butterfly
 * stages applied in the order h = 1, 2, 4, ..., d/2.  head_dim 192, a
 * multiple of 64 that is not a power of two (the velog.io post's rule turns
 * the rotation on for it; no Sylvester matrix of that size exists), is
 * rotated block-diagonally: each group of 64 elements by itself, stages
 * h = 1..32, factor fp32(1/8).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = -1,      /* null pointer, bad size, bad enum value */
  KVQ_ERR_UNSUPPORTED = -2,  /* head_dim or bit width the library does not build */
  KVQ_ERR_CAPACITY = -3,     /* a sequence would exceed max_ctx */
  KVQ_ERR_ALIGN = -4,        /* a device pointer is not 16-byte aligned */
  KVQ_ERR_HIP = -5,          /* the HIP runtime reported an error */
  KVQ_ERR_WORKSPACE = -6,    /* decode workspace smaller than required */
  /* Range markers, never returned: they make every int32 a representable
   * value of the enum, so a caller passing an unknown value gets an error
   * status instead of undefined behaviour (the same in the enums below). */
  KVQ_STATUS_RANGE_MIN = -0x7FFFFFFF - 1, KVQ_STATUS_RANGE_MAX = 0x7FFFFFFF
} kvq_status;

typedef enum kvq_dtype {
  KVQ_BF16 = 0, KVQ_F32 = 1,
  KVQ_DTYPE_RANGE_MIN = -0x7FFFFFFF - 1, KVQ_DTYPE_RANGE_MAX = 0x7FFFFFFF
} kvq_dtype;

typedef enum kvq_plane {
  KVQ_K_CODES = 0, KVQ_K_SCALES = 1, KVQ_V_CODES = 2,
  KVQ_V_SCALES = 3, KVQ_K_TAIL = 4, KVQ_V_TAIL = 5,
  /* outlier channels (kvq_config.outliers > 0) */
  KVQ_K_OUT_CODES = 6, KVQ_K_OUT_SCALES = 7, KVQ_V_OUT_CODES = 8, KVQ_V_OUT_SCALES = 9,
  KVQ_PLANE_RANGE_MIN = -0x7FFFFFFF - 1, KVQ_PLANE_RANGE_MAX = 0x7FFFFFFF
} kvq_plane;

/* Largest batch a single call accepts (sequence lengths travel in the
 * kernel arguments). */
#define KVQ_MAX_BATCH 256

/* Positions per page of a paged cache (one tile of every tiled plane). */
#define KVQ_PAGE_TOKENS 64

typedef struct kvq_config {
  int32_t batch;       /* sequences, 1..KVQ_MAX_BATCH */
  int32_t n_kv_heads;  /* KV heads per sequence, >= 1 */
  int32_t head_dim;    /* 64, 128, 192 or 256 */
  int32_t k_bits;      /* 4, 5, 6 or 8 (q4_0, q5_0, q6_0, q8_0 blocks) */
  int32_t v_bits;      /* 4, 5, 6 or 8 */
  int32_t tail_len;    /* newest tokens kept in bf16, >= 0 */
  int32_t max_ctx;     /* capacity per sequence in tokens, >= 1 */
  int32_t rotate_k;    /* 1: rotate K (and q); 0: store K as is */
  int32_t rotate_v;    /* 1: rotate V and rotate the output back; 0: neither */
  uint32_t sign_seed;  /* 0: rotate by the Sylvester-Hadamard matrix H; else by
                        * H diag(s), s_e = -1 iff the top bit of SplitMix64 of
                        * the counter sign_seed * 2^32 + e is set (a random-sign
                        * variant, which the velog.io post names in section
                        * "application and background") */
  int32_t k_min;       /* 1: K uses scale-and-min blocks (q4_1 / q5_1; k_bits
                        * 4 or 5), 0: absmax blocks.  Byte cost per the
                        * aiwitness.kr table's q5_1 rows; see "Scale-and-min
                        * blocks" above */
  int32_t v_min;       /* the same for V */
  int32_t page_pool;   /* 0: contiguous planes, each (sequence, KV head)
                        * owns max_ctx rounded up to 64 positions; > 0: the
                        * code and scale planes are a pool of this many pages
                        * of 64 positions, mapped by kvq_cache.page_table */
  int32_t outliers;    /* 0, or 32: K and V each keep 32 caller-chosen
                        * outlier channels per KV head at 8 bits in the
                        * original space (see "Outlier channels" above);
                        * needs tail_len 0, head_dim 128 and absmax blocks */
} kvq_config;

typedef struct kvq_cache {
  void* k_codes;
  void* k_scales;
  void* v_codes;
  void* v_scales;
  void* k_tail;  /* may be NULL when tail_len == 0 */
  void* v_tail;  /* may be NULL when tail_len == 0 */
  /* Paged caches only (ignored when page_pool == 0): device int32
   * [batch][ceil(max_ctx / 64)], the page of each 64-position tile of each
   * sequence, 4-byte aligned, owned and filled by the caller.  Entries for
   * tiles a call writes or reads must name pages in [0, page_pool); a page
   * must not be written for two sequences.  The kernels never follow an
   * entry outside [0, page_pool): the append skips positions on such a page
   * and attention and read-back read page 0 in its place (results for those
   * positions are unspecified).  Entries past a sequence's last tile are
   * never read. */
  const int32_t* page_table;
  /* Outlier channels only (ignored when outliers == 0): the four outlier
   * planes (kvq_plane_bytes of KVQ_K_OUT_CODES .. KVQ_V_OUT_SCALES) and the
   * channel lists, device int32 [2][n_kv_heads][32] (K's lists, then V's),
   * each list 32 distinct channels in [0, head_dim), 4-byte aligned, owned
   * by the caller and fixed for the cache's life. */
  void* k_out_codes;
  void* k_out_scales;
  void* v_out_codes;
  void* v_out_scales;
  const int32_t* outlier_idx;
} kvq_cache;

/* Defaults: 4-bit K and V, no tail, rotation on iff head_dim >= 64 and
 * head_dim % 64 == 0 (velog.io post, section "application and background"),
 * sign_seed 0, absmax blocks (k_min = v_min = 0), contiguous planes
 * (page_pool = 0), no outlier channels (outliers = 0). */
kvq_config kvq_config_default(int32_t batch, int32_t n_kv_heads,
                              int32_t head_dim, int32_t max_ctx);

/* KVQ_OK if the configuration is one the library can run. */
kvq_status kvq_config_check(const kvq_config* cfg);

/* Bytes the caller must allocate for one cache plane; 0 for an invalid
 * configuration or plane (and for tail planes when tail_len == 0).  For a
 * paged cache the code and scale planes hold page_pool pages. */
size_t kvq_plane_bytes(const kvq_config* cfg, kvq_plane plane);

/* Device workspace kvq_decode_attention needs for n_q_heads query heads per
 * sequence; 0 for invalid arguments.  Depends only on the configuration. */
size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t n_q_heads);

/* Rotate, quantize and append n_new tokens to every sequence (velog.io post
 * "fix KV cache quantization outliers", section "Hadamard rotation": K and V
 * are rotated when they are stored; the block formats and their byte counts
 * follow the aiwitness.kr table "Qwen 3.6 27B Q5_K_S + 64k context KLD
 * results"; the tail follows aitrends.kr article 92204, glossary "Precision
 * Tail").
 *  k_new, v_new: device [batch][n_new][n_kv_heads][head_dim] of `dtype`.
 *  seq_len:      host [batch], each sequence's length BEFORE the append;
 *                positions seq_len[b] .. seq_len[b]+n_new-1 are written.
 *                The caller advances its lengths afterwards.
 * Positions below (new length - tail_len) are quantized; the newest tail_len
 * positions are written to the tail ring, and tokens that leave the tail are
 * quantized from their stored bf16 values in the same call.  n_new == 0 is a
 * no-op.  Errors: KVQ_ERR_CAPACITY if seq_len[b] + n_new > max_ctx;
 * KVQ_ERR_INVALID for null pointers, negative lengths or a bad dtype. */
kvq_status kvq_rotate_quantize_append(const kvq_config* cfg,
                                      const kvq_cache* cache,
                                      const void* k_new, const void* v_new,
                                      kvq_dtype dtype, int32_t n_new,
                                      const int32_t* seq_len, void* stream);

/* Single-query decode attention over the whole cache of every sequence
 * (velog.io post, section "Hadamard rotation": rotated q.K scores, softmax,
 * weighted sum of V, inverse rotation of the result).
 *  q:        device [batch][n_q_heads][head_dim] of `dtype`; query head h
 *            reads KV head h / (n_q_heads / n_kv_heads).
 *  sm_scale: multiplier of q.k before the softmax (1/sqrt(head_dim) is usual).
 *  seq_len:  host [batch], tokens cached per sequence, 1..max_ctx.
 *  out:      device [batch][n_q_heads][head_dim] float32, original space.
 *  workspace/workspace_bytes: device scratch of at least
 *            kvq_decode_workspace_bytes(cfg, n_q_heads) bytes
 *            (KVQ_ERR_WORKSPACE otherwise); contents need no initialisation.
 * The waves that share a (sequence, KV head) take its tiles dynamically, so
 * two calls on the same inputs agree to rounding (about 1e-4 relative), not
 * bit for bit.
 * Errors: KVQ_ERR_INVALID if n_q_heads is not a positive multiple of
 * n_kv_heads, a length is 0 or sm_scale is not finite; KVQ_ERR_CAPACITY if a
 * length exceeds max_ctx. */
kvq_status kvq_decode_attention(const kvq_config* cfg, const kvq_cache* cache,
                                const void* q, kvq_dtype dtype,
                                int32_t n_q_heads, float sm_scale,
                                const int32_t* seq_len, float* out,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/* One decode step: kvq_rotate_quantize_append of one token per sequence
 * followed by kvq_decode_attention over the cache with that token, in fewer
 * launches.  The token's K/V are appended exactly as the append call would
 * (the cache afterwards holds the same bytes), and attention sees the cache
 * as it stands after the append: the positions the append changes (the new
 * token and the position that becomes quantized) are attended to from the
 * values the append computes, the rest from the cache (velog.io post "fix
 * KV cache quantization outliers", section "Hadamard rotation": rotate and
 * store at append, rotated scores and weighted sum at attention; aitrends.kr
 * article 92204, glossary "Precision Tail").
 *  k_new, v_new: device [batch][1][n_kv_heads][head_dim] of kv_dtype.
 *  q:            device [batch][n_q_heads][head_dim] of q_dtype.
 *  seq_len:      host [batch], each sequence's length BEFORE the step (>= 0);
 *                attention covers seq_len[b] + 1 positions.  The caller
 *                advances its lengths afterwards.
 *  out, workspace, workspace_bytes, sm_scale: as kvq_decode_attention, with
 *                kvq_decode_workspace_bytes(cfg, n_q_heads) bytes enough.
 * Errors: those of the two calls it replaces (KVQ_ERR_CAPACITY if
 * seq_len[b] + 1 > max_ctx); nothing is queued on an error. */
kvq_status kvq_decode_step(const kvq_config* cfg, const kvq_cache* cache,
                           const void* k_new, const void* v_new, kvq_dtype kv_dtype,
                           const void* q, kvq_dtype q_dtype, int32_t n_q_heads,
                           float sm_scale, const int32_t* seq_len, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device workspace kvq_decode_attention_static uses. */
#define KVQ_STATIC_WORKSPACE_BYTES 33554432

/* kvq_decode_attention for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments, results and errors are those of
 * kvq_decode_attention without the workspace: the split partials go to a
 * static device buffer of KVQ_STATIC_WORKSPACE_BYTES that the library holds
 * on each GPU it runs on until the process ends.  The call allocates
 * nothing.  Returns KVQ_ERR_WORKSPACE, queueing nothing, when the call would
 * need more than that (the need grows with batch x query heads and is at
 * most kvq_decode_workspace_bytes(cfg, n_q_heads)); KVQ_ERR_HIP if the
 * buffer's device address cannot be obtained.  Every call on one GPU shares
 * the buffer, and it keeps the last call's partials: calls that overlap on
 * one GPU (on other streams or host threads) race and must be ordered by
 * the caller. */
kvq_status kvq_decode_attention_static(const kvq_config* cfg, const kvq_cache* cache,
                                       const void* q, kvq_dtype dtype,
                                       int32_t n_q_heads, float sm_scale,
                                       const int32_t* seq_len, float* out,
                                       void* stream);

/* Workspace bytes kvq_prefill_attention needs for n_q_heads query heads and
 * n_q queries per sequence at any length up to cfg->max_ctx; 0 if the
 * arguments are invalid. */
size_t kvq_prefill_workspace_bytes(const kvq_config* cfg, int32_t n_q_heads,
                                   int32_t n_q);

/* Chunked prefill (prompt processing) attention over the cache: the n_q
 * queries of each sequence are its last n_q positions, whose K/V a previous
 * kvq_rotate_quantize_append stored; query i sits at position
 * seq_len[b] - n_q + i and attends causally to positions 0..that position,
 * reading the cache as it stands (a position that left the bf16 tail during
 * the chunk is read quantized).  Per query the steps are those of
 * kvq_decode_attention (velog.io post "fix KV cache quantization outliers",
 * section "Hadamard rotation"; the post's section "compute cost and speed"
 * reports the rotation's cost on prompt processing).
 *  q:        device [batch][n_q][n_q_heads][head_dim] of `dtype`.
 *  n_q:      queries per sequence, 1 <= n_q <= seq_len[b] for every b.
 *  sm_scale: multiplier of q.k before the softmax.
 *  seq_len:  host [batch], tokens cached per sequence (the chunk included).
 *  out:      device [batch][n_q][n_q_heads][head_dim] float32, original space.
 *  workspace/workspace_bytes: device scratch of at least
 *            kvq_prefill_workspace_bytes(cfg, n_q_heads, n_q) bytes
 *            (KVQ_ERR_WORKSPACE otherwise), owned by the caller; contents
 *            need no initialisation.
 * Results are deterministic.  kvq_profile_decode_events instruments this
 * call's attention kernel too (the matrix-core kernel at head_dim 128 with
 * absmax blocks, the split kernel's prefill variant otherwise).
 * Errors: KVQ_ERR_INVALID if n_q_heads is not a positive multiple of
 * n_kv_heads, n_q < 1, a length is below n_q, sm_scale is not finite or the
 * rows of one KV head exceed 65535 blocks of 64; KVQ_ERR_CAPACITY if a length
 * exceeds max_ctx. */
kvq_status kvq_prefill_attention(const kvq_config* cfg, const kvq_cache* cache,
                                 const void* q, kvq_dtype dtype,
                                 int32_t n_q_heads, int32_t n_q, float sm_scale,
                                 const int32_t* seq_len, float* out,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Read back positions [t0, t1) of sequence b from the K (which = 0) or V
 * (which = 1) cache (velog.io post "fix KV cache quantization outliers",
 * section "Hadamard rotation": the normalized matrix is its own inverse, so
 * the stored values rotate back exactly in real arithmetic) as float32
 * [t1-t0][n_kv_heads][head_dim]: code * scale
 * for quantized positions, the stored bf16 value for tail positions.
 * space 0 returns the rotated values; space 1 rotates them back (the same
 * float32 transform as the append, since the matrix is its own inverse).
 * With outlier channels, space 0 returns the rotated rest y_R and space 1
 * the reconstruction: y_R rotated back, plus each outlier's dequantized
 * value added at its channel (one float32 add).
 * seq_len is the host length array; 0 <= t0 <= t1 <= seq_len[b]. */
kvq_status kvq_dequantize(const kvq_config* cfg, const kvq_cache* cache,
                          int32_t which, int32_t b, int32_t t0, int32_t t1,
                          const int32_t* seq_len, int32_t space, float* out,
                          void* stream);

/* Static text for a status code. */
const char* kvq_status_str(kvq_status status);

/* Instrumentation: when both are non-NULL, later kvq_decode_attention calls
 * on this host thread launch the split-K attention kernel with `before` and
 * `after` bound to it (hipExtLaunchKernel), so they take that kernel's own
 * start and end times on the call's stream.  Both are hipEvent_t created
 * with timing, passed as void*; the caller owns them.  NULL, NULL switches
 * this off. */
void kvq_profile_decode_events(void* before, void* after);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
