// Device helpers shared by the kvq kernels (gfx950, wave64).
//
// The rotation is the normalized Sylvester Hadamard transform (velog.io post
// "fix KV cache quantization outliers", section "Hadamard rotation"), applied
// as a float32 fast Walsh-Hadamard transform whose butterfly stages run in the
// order h = 1, 2, 4, ..., d/2 (optionally preceded, or on the way back followed,
// by the sign flips of a random-sign variant).  The quantizer and the transform must match the
// CPU reference bit for bit, so everything in this file is compiled with
// -ffp-contract=off and uses IEEE float32 with denormals preserved.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kTile = 64;     // tokens per tile of a code plane
constexpr int kChunk = 16;    // bytes per tiled chunk
constexpr int kBlock = 32;    // elements per quantization block

__host__ __device__ constexpr int row_bytes(int d, int bits) { return d * bits / 8; }
__host__ __device__ constexpr int padded_row_bytes(int d, int bits) {
  return (row_bytes(d, bits) + kChunk - 1) / kChunk * kChunk;
}
__host__ __device__ constexpr int qmax_of(int bits) { return (1 << (bits - 1)) - 1; }

// Size of the Hadamard blocks of the rotation: d for a power of two, else 64
// (head_dim 192: block-diagonal, one H_64 per group of 64 elements).
__host__ __device__ constexpr int rot_block(int d) { return (d & (d - 1)) == 0 ? d : 64; }

// Positions one 256-thread block covers at one lane per 32-element block: a
// multiple of 8 (V groups), so at head_dim 192 (6 lanes a row) 40 positions
// use 240 threads and the last 16 only join the cross-lane stages.
__host__ __device__ constexpr int rows_per_block(int d) { return 256 / (d / kBlock) / 8 * 8; }

// Byte offset of 16-byte chunk c of token p's row inside one (b, g) plane.
__host__ __device__ inline size_t chunk_offset(int p, int c, int rpad) {
  return (size_t)(p / kTile) * kTile * rpad + (size_t)(c * kTile + (p % kTile)) * kChunk;
}

// Where the 64-token tiles of the tiled planes (K codes, V codes, scales)
// live.  Contiguous caches keep the cap/64 tiles of each (sequence, KV head)
// together: tile t of (b, g) is slot (b*Hkv + g)*tiles + t.  Paged caches
// draw pages of 64 tokens from a pool shared by all sequences: tile t of
// sequence b is page ptab[b*tiles + t], whose slot for KV head g is
// page*Hkv + g.  A plane's tile of (b, g, t) starts at slot * (its tile bytes).
struct TileMap {
  const int32_t* ptab;   // [B][tiles] device page table; nullptr: contiguous
  int32_t n_pages;       // pool size in pages (paged caches)
  int32_t tiles;         // cap / 64: tiles per sequence, the table's row length
  int32_t Hkv;
};
// Slot of tile t of (b, g); -1 when the table entry lies outside
// [0, n_pages), which the kernels never follow.
__device__ inline long long tile_slot(const TileMap& m, int b, int g, int t) {
  if (!m.ptab) return ((long long)b * m.Hkv + g) * m.tiles + t;
  const int page = m.ptab[(size_t)b * m.tiles + t];
  return (unsigned)page < (unsigned)m.n_pages ? (long long)page * m.Hkv + g : -1LL;
}
// For reads: a bad entry reads page 0 instead, which stays inside the pool
// (results for those positions are then unspecified).
__device__ inline size_t tile_slot_read(const TileMap& m, int b, int g, int t) {
  const long long s = tile_slot(m, b, g, t);
  return s < 0 ? (size_t)g : (size_t)s;
}

// V code planes are stored element-major per 64-token tile, so that the
// codes of one element for eight consecutive tokens sit in one item (the
// shape of one lane's P.V matrix-core operand).  Token t (0..63) and element
// e of a tile belong to item v_item(d, t, e), slot t % 8:
//   4-bit: one 32-bit word per item, u = c + 8 of slot k in nibble v_nibble(k)
//   8-bit: eight bytes per item, u = c + 128 of slot k in byte k
//   5-bit: the 4-bit words of u & 15 for every item (32*d bytes), then one
//          byte per item whose bit v_nibble(k) is bit 4 of u.
//   6-bit: the 4-bit words of u & 15, then one 16-bit field per item whose
//          bits 2*v_nibble(k), +1 are bits 4, 5 of u.
__host__ __device__ constexpr int v_tile_bytes(int d, int bits) { return kTile * d * bits / 8; }
__host__ __device__ constexpr int v_item(int d, int t, int e) {
  return ((t / 32) * 64 + 16 * ((t % 32) / 8) + e % 16) * (d / 16) + e / 16;
}
__host__ __device__ constexpr int v_nibble(int k) { return 4 * (k % 2) + k / 2; }

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round-to-nearest-even to bfloat16 (finite inputs).
__device__ inline uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ inline float bf16_round(float x) { return __uint_as_float(f32_to_bf16_bits(x) << 16); }

// Value of lane (lane ^ M) within groups of 32 lanes.
template <int M>
__device__ inline float xor_lane(float v) {
  int i = __float_as_int(v);
  if constexpr (M == 1) {
    i = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    i = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
  } else {
    static_assert(M == 4 || M == 8 || M == 16, "xor within 32 lanes");
    i = __builtin_amdgcn_ds_swizzle(i, 0x1F | (M << 10));     // bit-mask mode, xor M
  }
  return __int_as_float(i);
}

// Butterfly stages h = 1..16 on the 32 consecutive elements a lane holds.
__device__ inline void fwht32_in_lane(float (&x)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float u = x[i], v = x[i + h];
        x[i] = u + v;
        x[i + h] = u - v;
      }
    }
  }
}

// One butterfly stage across lanes: element bit log2(32*M) lives in lane bit
// M.  The lane holding the lower index keeps a + b, the other b_low - a_high;
// adding the sign-flipped own value gives exactly those two results.
template <int M>
__device__ inline void fwht_cross_stage(float (&x)[32], int lane) {
  const uint32_t flip = (lane & M) ? 0x80000000u : 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float y = xor_lane<M>(x[i]);
    x[i] = y + __uint_as_float(__float_as_uint(x[i]) ^ flip);
  }
}

// The same stage in one instruction per element (lane distances 1 and 2):
// v_fmac_f32 with a DPP operand computes own + s * partner, s = +1 on the
// lower lane and -1 on the upper one, rounding once like the add.  The upper
// lane gets a_high - b_low, the negation of the butterfly's value, so the
// stored values carry a per-lane sign (the product of the stages' flips,
// shared by the partners of later stages), which the final multiply removes.
// Nonzero results are bit for bit those of the plain stage; an exact zero
// may come out with the other sign.  Only for values that go straight into
// an absmax quantizer, whose codes and scales do not see the sign of a zero.
// The compiler does not form this instruction from the intrinsics, so it is
// written out; a DPP operand must not be read within two wait states of the
// VALU write that produced it, hence the s_nop ahead of each group (inside a
// group every instruction reads a register written before the group).
#define KVQ_FMAC_DPP(PERM, I) "v_fmac_f32_dpp %" #I ", %" #I ", %16 " PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
#define KVQ_FMAC_DPP16(PERM)                                                             \
  "s_nop 1\n" KVQ_FMAC_DPP(PERM, 0) KVQ_FMAC_DPP(PERM, 1) KVQ_FMAC_DPP(PERM, 2)          \
  KVQ_FMAC_DPP(PERM, 3) KVQ_FMAC_DPP(PERM, 4) KVQ_FMAC_DPP(PERM, 5) KVQ_FMAC_DPP(PERM, 6) \
  KVQ_FMAC_DPP(PERM, 7) KVQ_FMAC_DPP(PERM, 8) KVQ_FMAC_DPP(PERM, 9)                      \
  KVQ_FMAC_DPP(PERM, 10) KVQ_FMAC_DPP(PERM, 11) KVQ_FMAC_DPP(PERM, 12)                   \
  KVQ_FMAC_DPP(PERM, 13) KVQ_FMAC_DPP(PERM, 14) KVQ_FMAC_DPP(PERM, 15)
template <int M>
__device__ inline void fwht_cross_stage_fma(float (&x)[32], int lane) {
  static_assert(M == 1 || M == 2, "DPP quad permutations");
  const float s = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int g = 0; g < 32; g += 16) {
    float* y = x + g;
    if constexpr (M == 1) {
      asm(KVQ_FMAC_DPP16("quad_perm:[1,0,3,2]")
          : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]),
            "+v"(y[6]), "+v"(y[7]), "+v"(y[8]), "+v"(y[9]), "+v"(y[10]), "+v"(y[11]),
            "+v"(y[12]), "+v"(y[13]), "+v"(y[14]), "+v"(y[15])
          : "v"(s));
    } else {
      asm(KVQ_FMAC_DPP16("quad_perm:[2,3,0,1]")
          : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]),
            "+v"(y[6]), "+v"(y[7]), "+v"(y[8]), "+v"(y[9]), "+v"(y[10]), "+v"(y[11]),
            "+v"(y[12]), "+v"(y[13]), "+v"(y[14]), "+v"(y[15])
          : "v"(s));
    }
  }
}
#undef KVQ_FMAC_DPP16
#undef KVQ_FMAC_DPP

// Full transform of a d-element row spread over d/32 consecutive lanes, each
// holding one 32-element block, followed by the normalization multiply.  At
// head_dim 192 each pair of lanes (one H_64 block) is transformed on its own.
template <int D>
__device__ inline void rotate_row(float (&x)[32], int lane, float cd) {
  constexpr int RB = rot_block(D);
  fwht32_in_lane(x);
  if constexpr (RB >= 64) fwht_cross_stage<1>(x, lane);
  if constexpr (RB >= 128) fwht_cross_stage<2>(x, lane);
  if constexpr (RB >= 256) fwht_cross_stage<4>(x, lane);
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = x[i] * cd;
}

// rotate_row for values that only feed an absmax quantizer: the cross-lane
// stages at lane distances 1 and 2 take one instruction per element, and the
// normalization multiply by +-fp32(1/sqrt(d)) removes their sign.  Equal to
// rotate_row except possibly for the sign of exact zeros.
template <int D>
__device__ inline void rotate_row_for_absmax(float (&x)[32], int lane, float cd) {
  constexpr int RB = rot_block(D);
  fwht32_in_lane(x);
  if constexpr (RB >= 64) fwht_cross_stage_fma<1>(x, lane);
  if constexpr (RB >= 128) fwht_cross_stage_fma<2>(x, lane);
  if constexpr (RB >= 256) fwht_cross_stage<4>(x, lane);
  const float c = (__builtin_popcount(lane & (RB >= 128 ? 3 : 1)) & 1) ? -cd : cd;
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = x[i] * c;
}

// Flip the sign of element i of a 32-element block where bit i of mask is
// set (the diagonal of the random-sign rotation H diag(s); exact).
__device__ inline void apply_signs(float (&x)[32], uint32_t mask) {
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = __uint_as_float(__float_as_uint(x[i]) ^ ((mask << (31 - i)) & 0x80000000u));
}

// Bit of the 5-bit high-bit word owned by element w (0..31) of a block.
__host__ __device__ constexpr int hibit_pos(int w) {
  return 8 * ((w % 8) / 2) + 2 * (w / 8) + (w % 2);
}
// First bit of element w's 2-bit field (bits 4, 5 of a 6-bit code) inside
// high word w / 16 of its block: the four fields of a group of 8 elements
// (w / 8) sit 8 bits apart, so one rotate aligns them with code bytes.
__host__ __device__ constexpr int hi2_pos(int w) {
  return 8 * ((w % 8) / 2) + 4 * ((w / 8) % 2) + 2 * (w % 2);
}

// Quantize one 32-element block: returns the fp16 scale bits; m[i] & 0xFF is
// the offset code c + 2^(BITS-1) of element i (higher bits are not zero).
// The code is clamp(x * r) rounded to nearest even: clamping to the integer
// bound first and then rounding equals rounding then clamping, and adding
// 1.5 * 2^23 + offset rounds |t| <= 127 to an integer in float32's last
// place (ties to even), leaving it in the low mantissa bits.
template <int BITS>
__device__ inline uint32_t quantize_block(const float (&x)[32], uint32_t (&m)[32]) {
  constexpr float qmax = (float)qmax_of(BITS);
  constexpr float kMagic = 12582912.0f + (float)(1 << (BITS - 1));
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(x[i]));
  float s32 = a / qmax;                  // correctly rounded divide
  s32 = fminf(s32, 65504.0f);
  const _Float16 s16 = (_Float16)s32;    // round to nearest even
  const float sf = (float)s16;
  const float r = sf != 0.f ? 1.0f / sf : 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float t = __builtin_amdgcn_fmed3f(x[i] * r, -qmax, qmax);
    m[i] = __float_as_uint(t + kMagic);
  }
  return (uint32_t)__builtin_bit_cast(uint16_t, s16);
}

// Scale-and-min quantization of one 32-element block (q4_1 / q5_1): returns
// the fp16 bits of the scale s (low half) and the minimum m (high half);
// m[i] & 0xFF is the level u in [0, 2^BITS - 1] of element i, which the code
// planes store where the symmetric formats store c + 2^(BITS-1).
//   s = fp16(min((hi - lo) / (2^BITS - 1), 65504)), m = fp16(lo clamped),
//   u = rint(clamp((x - m) * (1 / s), 0, 2^BITS - 1))   (0 when s == 0)
// rounded to nearest even by the same magic add as quantize_block.
template <int BITS>
__device__ inline uint32_t quantize_block_min(const float (&x)[32], uint32_t (&m)[32]) {
  constexpr float umax = (float)((1 << BITS) - 1);
  constexpr float kMagic = 12582912.0f;
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    lo = fminf(lo, x[i]);
    hi = fmaxf(hi, x[i]);
  }
  float s32 = (hi - lo) / umax;          // correctly rounded subtract and divide
  s32 = fminf(s32, 65504.0f);
  const _Float16 s16 = (_Float16)s32;
  const _Float16 m16 = (_Float16)fminf(fmaxf(lo, -65504.0f), 65504.0f);
  const float sf = (float)s16, mf = (float)m16;
  const float r = sf != 0.f ? 1.0f / sf : 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float t = __builtin_amdgcn_fmed3f((x[i] - mf) * r, 0.f, umax);
    m[i] = __float_as_uint(t + kMagic);
  }
  return (uint32_t)__builtin_bit_cast(uint16_t, s16) | ((uint32_t)__builtin_bit_cast(uint16_t, m16) << 16);
}

// Signed codes c of elements 32j..32j+31 of position p of one K tile (row
// layout, 16-byte chunks placed by chunk_offset).
template <int D, int BITS>
__device__ inline void load_codes(const uint8_t* plane, int p, int j, int (&c)[32]) {
  constexpr int RP = padded_row_bytes(D, BITS);
  if constexpr (BITS == 8) {
    const uint4 v0 = *reinterpret_cast<const uint4*>(plane + chunk_offset(p, 2 * j, RP));
    const uint4 v1 = *reinterpret_cast<const uint4*>(plane + chunk_offset(p, 2 * j + 1, RP));
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int e = 0; e < 32; ++e) c[e] = (int)(int8_t)((w[e / 4] >> (8 * (e % 4))) & 0xFF);
  } else {
    constexpr int OFF = 1 << (BITS - 1);
    const uint4 v = *reinterpret_cast<const uint4*>(plane + chunk_offset(p, j, RP));
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t hw = 0, hw2[2] = {0u, 0u};
    if constexpr (BITS == 5) {
      const int byte = D / 2 + 4 * j;
      hw = *reinterpret_cast<const uint32_t*>(plane + chunk_offset(p, byte / kChunk, RP) + byte % kChunk);
    }
    if constexpr (BITS == 6) {
      const int byte = D / 2 + 8 * j;
      const uint2 h = *reinterpret_cast<const uint2*>(plane + chunk_offset(p, byte / kChunk, RP) + byte % kChunk);
      hw2[0] = h.x;
      hw2[1] = h.y;
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      int u = (int)((w[e / 8] >> (4 * (e % 8))) & 15);
      if constexpr (BITS == 5) u |= (int)((hw >> hibit_pos(e)) & 1) << 4;
      if constexpr (BITS == 6) u |= (int)((hw2[e / 16] >> hi2_pos(e)) & 3) << 4;
      c[e] = u - OFF;
    }
  }
}

// Low bytes of a, b, c, d as one little-endian word.
__device__ inline uint32_t gather_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

}  // namespace kvq
