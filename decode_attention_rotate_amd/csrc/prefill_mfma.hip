// Chunked prefill on the matrix cores (head_dim 128, absmax blocks).
//
// A chunk's n_q queries attend causally to the cache (the chunked-prefill
// reading of the velog.io post "fix KV cache quantization outliers",
// section "compute cost and speed": the rotation costs prompt processing
// too).  Scores are taken on rotated vectors (section "Hadamard rotation":
// q is rotated like the keys, and the rotation is orthogonal).
//
// The decode kernel's layout (eight query rows per wave, everything else per
// 32-token step) leaves the per-token work of dequantizing and of the
// softmax spread over few rows.  Here a workgroup of eight waves owns 256
// rows of one KV head (32 per wave) and walks 64-position tiles:
//  * each tile is dequantized once into one of two LDS buffers, while the
//    products run on the other: waves 0-3 write K' = code * scale * 2^fk(p)
//    as fp16 hi + lo parts (fk per position keeps |K'| < 2^15; the pair
//    holds the 19-bit product exactly), waves 4-7 write V' = code * scale *
//    2^fv for one 32-element block each, as hi + lo parts stored transposed
//    (element-major).  fv is one power of two per block and workgroup that
//    only decreases; the accumulators of that block are rescaled exactly
//    when it does.  Codes become fp16 pairs by placing them under the
//    exponent of 1024 and subtracting 1024 + offset; the products with the
//    scale and their rounding remainders are packed fp16 operations;
//  * the K waves dequantize before their products and the V waves after
//    theirs, so the two waves sharing a SIMD tend to have one on the matrix
//    core while the other works on the vector unit; one barrier per tile;
//  * S^T = K' Q'^T on 32x32x16 f16 matrix-core steps, positions as the M
//    dimension and rows as N: three products per step (hi.hi, hi.lo,
//    lo.hi; the dropped lo.lo term is below 2^-22 of the score);
//  * each lane then holds 16 positions of one row per M tile, so the row's
//    softmax is in-lane work plus one exchange with the other half-wave,
//    and the fp16 probabilities are already in the lane layout of the B
//    operand of O^T += V'^T P^T (the K order of that product is chosen to
//    match the accumulator layout of the first one).  The probabilities are
//    split into fp16 hi + lo as well, so this product too is three f16
//    products (V hi.P hi, V lo.P hi, V hi.P lo): rows whose output nearly
//    cancels (a norm of a few percent of the values') magnify a 2^-12
//    rounding of P or V' thirty-fold, past a 1e-3 relative error.
// Queries are prepared once by prefill_q_kernel: q' = rotated q * sm_scale *
// log2(e), per row scaled by 2^fq into [2^14, 2^15) and split into fp16 hi +
// lo, with the elements of each 32-element block in the column order the K
// tiles use (the contraction does not depend on that order).  The partials
// (running maximum in log2 units, sum, unnormalized output in rotated space)
// are the split kernel's, merged by the same combine.
#include "common.hpp"
#include "kernels.hpp"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 hpair __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int PD = 128;                 // head_dim
constexpr int PR = kPrefillRows;        // rows per workgroup, 32 per wave
constexpr int kThreads = 512;
constexpr int KROW = PD + 8;            // halves per LDS row of K' (272 bytes)
constexpr int VROW = kTile + 8;         // halves per LDS row of V'^T (144 bytes)
constexpr int kNoScale = 1 << 20;       // "no nonzero value seen" for fk / fv
constexpr float kLog2eF = 1.44269504088896340736f;
constexpr float kLazy = 8.f;            // probabilities stay below 2^kLazy

__device__ inline int exponent_of(float x) {   // floor(log2(x)) for normal x > 0
  return (int)((__float_as_uint(x) >> 23) & 255u) - 127;
}
__device__ inline float pow2(int e) {          // 2^e, e clamped to [-100, 100]
  e = e < -100 ? -100 : (e > 100 ? 100 : e);
  return __uint_as_float((uint32_t)(e + 127) << 23);
}
__device__ inline float fp16_bits_to_f32(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); }

// Element of a 32-element K block held by column i of that block (in the K'
// tiles and in the prepared queries).  Codes of 4 to 6 bits are unpacked two
// at a time from nibbles 16 bits apart, elements k and k + 4 of each 8.
template <int KB>
__host__ __device__ constexpr int k_column_element(int i) {
  return KB == 8 ? i : 8 * (i / 8) + (i % 8) / 2 + 4 * (i % 2);
}

// ---------------------------------------------------------------- queries
// One row per four lanes (32 elements each), 64 rows per block.
template <int KB>
__global__ __launch_bounds__(256) void prefill_q_kernel(PrefillArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, j = tid & 3;
  const int g = blockIdx.y, b = blockIdx.z;
  const int r = blockIdx.x * 64 + (tid >> 2);
  const bool valid = r < a.n_q * a.G;
  float x[32];
  if (valid) {
    const int i = r / a.G, hq = g * a.G + r % a.G;
    const size_t off = (((size_t)b * a.n_q + i) * a.Hq + hq) * PD + 32 * j;
    if (a.q_dtype == KVQ_BF16) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + off);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = p[q];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[8 * q + 2 * k] = __uint_as_float(w[k] << 16);
          x[8 * q + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + off);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = p[q];
        x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = 0.f;
  }
  if (a.rotate_k) {   // every lane takes part in the cross-lane stages
    if (a.has_signs) apply_signs(x, a.signs[j]);
    rotate_row<PD>(x, lane, a.cd);
  }
  const float f = a.sm_scale * kLog2eF;
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    x[e] *= f;
    mx = fmaxf(mx, fabsf(x[e]));
  }
  mx = fmaxf(mx, xor_lane<1>(mx));
  mx = fmaxf(mx, xor_lane<2>(mx));
  const int fq = mx > 0.f ? 14 - exponent_of(mx) : 0;
  const float sc = pow2(fq);
  const size_t row = ((size_t)b * a.Hkv + g) * a.rows_pad + r;
  uint32_t hw[16], lw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float y0 = x[k_column_element<KB>(2 * i)] * sc, y1 = x[k_column_element<KB>(2 * i + 1)] * sc;
    const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1;
    const _Float16 l0 = (_Float16)(y0 - (float)h0), l1 = (_Float16)(y1 - (float)h1);
    hw[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    lw[i] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
  }
  uint4* dh = reinterpret_cast<uint4*>(a.q_hi + row * PD + 32 * j);
  uint4* dl = reinterpret_cast<uint4*>(a.q_lo + row * PD + 32 * j);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    dh[q] = make_uint4(hw[4 * q], hw[4 * q + 1], hw[4 * q + 2], hw[4 * q + 3]);
    dl[q] = make_uint4(lw[4 * q], lw[4 * q + 1], lw[4 * q + 2], lw[4 * q + 3]);
  }
  if (j == 0) a.q_w[row] = pow2(-fq);
}

// ---------------------------------------------------------------- attention
struct __align__(16) PrefillLds {
  _Float16 khi[2][kTile * KROW];   // K' hi, lo: [position][column]
  _Float16 klo[2][kTile * KROW];
  _Float16 vth[2][PD * VROW];      // V'^T hi, lo: [element][position]
  _Float16 vtl[2][PD * VROW];
  float ku[2][kTile];              // 2^-fk of each position
  int fv[2][4];                    // V exponent of each 32-element block
  uint16_t vsc[4][kTile];          // the V scales of one block, per V wave
};

// fp16 hi and lo parts of 2n floats as packed words: hi is y rounded
// toward zero (two per instruction), so y - hi has at most the 8-9
// significant bits a 19-bit value leaves and lo holds it exactly (inputs
// here have at most 19 significant bits and |y| < 2^15).
typedef __fp16 half2v __attribute__((ext_vector_type(2)));
template <int N>
__device__ inline void split_pairs(const float* y, uint32_t* hw, uint32_t* lw) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const half2v hh = __builtin_amdgcn_cvt_pkrtz(y[2 * i], y[2 * i + 1]);
    const half2v ll = __builtin_amdgcn_cvt_pkrtz(y[2 * i] - (float)hh[0], y[2 * i + 1] - (float)hh[1]);
    hw[i] = __builtin_bit_cast(uint32_t, hh);
    lw[i] = __builtin_bit_cast(uint32_t, ll);
  }
}

// Codes u (0..255) of a packed pair as fp16 1024 + u: c = that - (1024 +
// offset) is exact, and so are hi = fp16(c * s) and lo = fp16(c * s - hi)
// (fused): c * s has at most 19 significant bits.
__device__ inline void code_pair(uint32_t x, float off, hpair s, uint32_t& hw, uint32_t& lw) {
  const hpair c = __builtin_bit_cast(hpair, x) - hpair{(_Float16)off, (_Float16)off};
  const hpair hi = c * s;
  const hpair lo = __builtin_elementwise_fma(c, s, -hi);
  hw = __builtin_bit_cast(uint32_t, hi);
  lw = __builtin_bit_cast(uint32_t, lo);
}

// What a K wave's thread reads for one tile: the codes of one 32-element
// block of one position (and their high bits at 5 or 6 bits) and its scale.
struct KRaw {
  uint4 k0, k1;        // code chunks (k1: 8-bit codes only)
  uint2 hb;            // high-bit words (5- and 6-bit codes)
  uint32_t s;          // fp16 scale bits
};

template <int KB>
__device__ inline void load_k(const PrefillArgs& a, size_t slot, bool ok, int pl, int j, KRaw& r) {
  constexpr int RP = padded_row_bytes(PD, KB);
  r.k0 = r.k1 = make_uint4(0u, 0u, 0u, 0u);
  r.hb = make_uint2(0u, 0u);
  r.s = 0u;
  if (!ok) return;
  const uint8_t* kt = a.k_codes + slot * kTile * RP;
  if constexpr (KB == 8) {
    r.k0 = *reinterpret_cast<const uint4*>(kt + chunk_offset(pl, 2 * j, RP));
    r.k1 = *reinterpret_cast<const uint4*>(kt + chunk_offset(pl, 2 * j + 1, RP));
  } else {
    r.k0 = *reinterpret_cast<const uint4*>(kt + chunk_offset(pl, j, RP));
    if constexpr (KB == 5) {
      const int byte = PD / 2 + 4 * j;
      r.hb.x = *reinterpret_cast<const uint32_t*>(kt + chunk_offset(pl, byte / kChunk, RP) + byte % kChunk);
    }
    if constexpr (KB == 6) {
      const int byte = PD / 2 + 8 * j;
      r.hb = *reinterpret_cast<const uint2*>(kt + chunk_offset(pl, byte / kChunk, RP) + byte % kChunk);
    }
  }
  r.s = a.k_scales[(slot * kTile + pl) * 4 + j];
}

// Packed pairs 1024 + u of a block's codes in column order: pair i holds
// columns 2i, 2i + 1.
template <int KB>
__device__ inline void k_pairs(const KRaw& r, uint32_t (&x)[16]) {
  if constexpr (KB == 8) {   // signed bytes; u = c + 128
    const uint32_t w[8] = {r.k0.x, r.k0.y, r.k0.z, r.k0.w, r.k1.x, r.k1.y, r.k1.z, r.k1.w};
#pragma unroll
    for (int wi = 0; wi < 8; ++wi) {
      const uint32_t wx = w[wi] ^ 0x80808080u;
      x[2 * wi] = (wx & 0xFFu) | ((wx & 0xFF00u) << 8) | 0x64006400u;
      x[2 * wi + 1] = ((wx >> 16) & 0xFFu) | ((wx >> 8) & 0xFF0000u) | 0x64006400u;
    }
  } else {
    const uint32_t w[4] = {r.k0.x, r.k0.y, r.k0.z, r.k0.w};
    const uint32_t hw2[2] = {r.hb.x, r.hb.y};
#pragma unroll
    for (int wi = 0; wi < 4; ++wi)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e0 = 8 * wi + k, e1 = e0 + 4;
        uint32_t v = ((w[wi] >> (4 * k)) & 0x000F000Fu) | 0x64006400u;
        if constexpr (KB == 5)
          v |= (((hw2[0] >> hibit_pos(e0)) & 1u) << 4) | (((hw2[0] >> hibit_pos(e1)) & 1u) << 20);
        if constexpr (KB == 6)
          v |= (((hw2[e0 / 16] >> hi2_pos(e0)) & 3u) << 4) | (((hw2[e1 / 16] >> hi2_pos(e1)) & 3u) << 20);
        x[4 * wi + k] = v;
      }
  }
}

// K wave: position pl, block j of tile t into buffer bf.  Each group of
// eight columns is stored as soon as it is formed.
template <int KB>
__device__ inline void stage_k(const PrefillArgs& a, PrefillLds& sm, int bf, int t, int nq, int len,
                               size_t unit, const KRaw& r, int pl, int j) {
  constexpr float OFF = 1024.f + (float)(KB == 8 ? 128 : 1 << (KB - 1));
  const int p = t * kTile + pl;
  const bool quant = p < nq;
  int fkc = kNoScale;
  uint4 tw[4];   // the bf16 tail values of the block, as stored
#pragma unroll
  for (int q = 0; q < 4; ++q) tw[q] = make_uint4(0u, 0u, 0u, 0u);
  if (quant) {
    const float s = fp16_bits_to_f32(r.s);
    if (s > 0.f) fkc = 7 - exponent_of(s);   // |c| < 2^7: |x| < 2^(e+8)
  } else if (p < len) {
    const uint4* kr = reinterpret_cast<const uint4*>(a.k_tail + (unit * a.T + p % a.T) * PD + 32 * j);
    float km = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tw[q] = kr[q];
      const uint32_t w[4] = {tw[q].x, tw[q].y, tw[q].z, tw[q].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) km = fmaxf(km, fmaxf(fabsf(__uint_as_float(w[k] << 16)), fabsf(__uint_as_float(w[k] & 0xFFFF0000u))));
    }
    if (km > 0.f) fkc = 14 - exponent_of(km);
  }
  // one fk per position: the smallest of its four blocks' candidates
  fkc = min(fkc, __shfl_xor(fkc, 1));
  fkc = min(fkc, __shfl_xor(fkc, 2));
  const int fk = fkc == kNoScale ? 0 : fkc;
  uint4* dh = reinterpret_cast<uint4*>(&sm.khi[bf][pl * KROW + 32 * j]);
  uint4* dl = reinterpret_cast<uint4*>(&sm.klo[bf][pl * KROW + 32 * j]);
  if (quant) {
    const _Float16 s16 = (_Float16)__builtin_amdgcn_ldexph(__builtin_bit_cast(_Float16, (uint16_t)r.s), fk);
    uint32_t x[16];
    k_pairs<KB>(r, x);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) code_pair(x[4 * q + i], OFF, hpair{s16, s16}, hw[i], lw[i]);
      dh[q] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      dl[q] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  } else {   // tail (exact bf16 values) or past the sequence (zeros)
    const float sc = pow2(fk);
    const uint32_t tws[16] = {tw[0].x, tw[0].y, tw[0].z, tw[0].w, tw[1].x, tw[1].y, tw[1].z, tw[1].w,
                              tw[2].x, tw[2].y, tw[2].z, tw[2].w, tw[3].x, tw[3].y, tw[3].z, tw[3].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = k_column_element<KB>(8 * q + i);
        const uint32_t wv = tws[e / 2];
        y[i] = __uint_as_float(e % 2 ? wv & 0xFFFF0000u : wv << 16) * sc;
      }
      uint32_t hw[4], lw[4];
      split_pairs<4>(y, hw, lw);
      dh[q] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      dl[q] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  }
  if (j == 0) sm.ku[bf][pl] = pow2(-fk);
}

// What a V wave's lane reads for one tile of its block me: the items of
// elements 32 me + 16 c + eo + 8 k (k, c = 0, 1) for the eight positions
// 8 pg .. 8 pg + 7 (lane = 8 pg + eo), and the scale of position lane.
struct VRaw {
  uint4 w[2];          // per k: the 4-bit words of c = 0, 1 in .x, .y, or the 8 bytes of each in .xy, .zw
  uint32_t hb[2];      // per k: high bits of c = 0 (low byte or half), c = 1
  uint32_t s;          // fp16 scale bits
};

template <int VB>
__device__ inline void load_v(const PrefillArgs& a, size_t slot, bool ok_items, bool ok_scale, int me,
                              int lane, VRaw& r) {
  const int pg = lane >> 3, eo = lane & 7;
  const uint8_t* vt = a.v_codes + slot * (size_t)v_tile_bytes(PD, VB);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    r.w[k] = make_uint4(0u, 0u, 0u, 0u);
    r.hb[k] = 0u;
    if (ok_items) {
      // v_item of position 8 pg, element 32 me + eo + 8 k; c = 1 is the next item
      const int item = ((pg >> 2) * 64 + (pg & 3) * 16 + eo + 8 * k) * (PD / 16) + 2 * me;
      if constexpr (VB == 8) {
        r.w[k] = *reinterpret_cast<const uint4*>(vt + 8 * item);
      } else {
        const uint2 q = *reinterpret_cast<const uint2*>(vt + 4 * item);
        r.w[k].x = q.x;
        r.w[k].y = q.y;
        if constexpr (VB == 5) r.hb[k] = *reinterpret_cast<const uint16_t*>(vt + 32 * PD + item);
        if constexpr (VB == 6) r.hb[k] = *reinterpret_cast<const uint32_t*>(vt + 32 * PD + 2 * item);
      }
    }
  }
  r.s = ok_scale ? (uint32_t)a.v_scales[(slot * kTile + lane) * 4 + me] : 0u;
}

// Offset codes of the eight slots of a V item from its words (the V tile
// layout: nibble, byte or high bits of slot k).
template <int VB>
__device__ inline void decode_v(uint2 r, int (&u)[8]) {
  if constexpr (VB == 8) {
#pragma unroll
    for (int k = 0; k < 8; ++k) u[k] = (int)(((k < 4 ? r.x : r.y) >> (8 * (k % 4))) & 0xFFu);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int nb = v_nibble(k);
      int v = (int)((r.x >> (4 * nb)) & 15u);
      if constexpr (VB == 5) v |= (int)((r.y >> nb) & 1u) << 4;
      if constexpr (VB == 6) v |= (int)((r.y >> (2 * nb)) & 3u) << 4;
      u[k] = v;
    }
  }
}

// The codes word and high bits of element (k, c).
template <int VB>
__device__ inline uint2 v_item_words(const VRaw& r, int k, int c) {
  if constexpr (VB == 8) return c ? make_uint2(r.w[k].z, r.w[k].w) : make_uint2(r.w[k].x, r.w[k].y);
  const uint32_t word = c ? r.w[k].y : r.w[k].x;
  if constexpr (VB == 5) return make_uint2(word, (r.hb[k] >> (8 * c)) & 0xFFu);
  if constexpr (VB == 6) return make_uint2(word, (r.hb[k] >> (16 * c)) & 0xFFFFu);
  return make_uint2(word, 0u);
}

// Packed pairs 1024 + u of an item's slots 2i, 2i + 1 (positions in order).
template <int VB>
__device__ inline uint32_t v_pair(uint2 it, int i) {
  if constexpr (VB == 8) {
    const uint32_t ww = i < 2 ? it.x : it.y;
    const int sh = 16 * (i % 2);
    return ((ww >> sh) & 0xFFu) | (((ww >> (sh + 8)) & 0xFFu) << 16) | 0x64006400u;
  } else {
    uint32_t v = ((it.x >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
    if constexpr (VB == 5) v |= (((it.y >> i) & 1u) << 4) | (((it.y >> (i + 4)) & 1u) << 20);
    if constexpr (VB == 6) v |= (((it.y >> (2 * i)) & 3u) << 4) | (((it.y >> (2 * i + 8)) & 3u) << 20);
    return v;
  }
}

// V wave me: block me of tile t into buffer bf.  fv_run, the block's
// running exponent, is this wave's own.  Each element's eight positions are
// stored as soon as they are formed; tail values are read twice (for the
// exponent, then for the values) rather than held.
template <int VB>
__device__ inline void stage_v(const PrefillArgs& a, PrefillLds& sm, int bf, int t, int nq, int len,
                               size_t unit, const VRaw& r, int me, int lane, int& fv_run) {
  constexpr int OFFI = 1 << (VB - 1);
  constexpr float OFF = 1024.f + (float)OFFI;
  const int pg = lane >> 3, eo = lane & 7, t0p = 8 * pg;
  const int p0 = t * kTile + t0p;
  sm.vsc[me][lane] = (uint16_t)r.s;
  int fvc = kNoScale;
  {
    const float vs = fp16_bits_to_f32(r.s);
    if (t * kTile + lane < nq && vs > 0.f) fvc = 7 - exponent_of(vs);
  }
  const bool tail_tile = t * kTile + kTile > nq;   // the same for the whole wave
  auto tail_value = [&](int kc, int s) {
    const int e = 32 * me + 16 * (kc & 1) + eo + 8 * (kc >> 1);
    const int p = p0 + s;
    return (p >= nq && p < len) ? bf16_to_f32(a.v_tail[(unit * a.T + p % a.T) * PD + e]) : 0.f;
  };
  if (tail_tile) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float v = tail_value(kc, s);
        if (v != 0.f) fvc = min(fvc, 14 - exponent_of(fabsf(v)));
      }
  }
#pragma unroll
  for (int mk = 1; mk < 64; mk <<= 1) fvc = min(fvc, __shfl_xor(fvc, mk));
  fv_run = min(fv_run, fvc);
  const int vexp = fv_run == kNoScale ? 0 : fv_run;
  if (lane == 0) sm.fv[bf][me] = fv_run;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint4 sv = *reinterpret_cast<const uint4*>(&sm.vsc[me][t0p]);   // scales of positions t0p..t0p+7
  const uint32_t svw[4] = {sv.x, sv.y, sv.z, sv.w};
  if (!tail_tile) {
    hpair sp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const hpair s2 = __builtin_bit_cast(hpair, svw[i]);
      sp[i] = hpair{(_Float16)__builtin_amdgcn_ldexph(s2[0], vexp), (_Float16)__builtin_amdgcn_ldexph(s2[1], vexp)};
    }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int e = 32 * me + 16 * (kc & 1) + eo + 8 * (kc >> 1);
      const uint2 it = v_item_words<VB>(r, kc >> 1, kc & 1);
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) code_pair(v_pair<VB>(it, i), OFF, sp[i], hw[i], lw[i]);
      *reinterpret_cast<uint4*>(&sm.vth[bf][e * VROW + t0p]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(&sm.vtl[bf][e * VROW + t0p]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  } else {
    const float vm = pow2(vexp);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int e = 32 * me + 16 * (kc & 1) + eo + 8 * (kc >> 1);
      int u[8];
      decode_v<VB>(v_item_words<VB>(r, kc >> 1, kc & 1), u);
      float y[8];
#pragma unroll
      for (int s = 0; s < 8; ++s)
        y[s] = p0 + s < nq ? (float)(u[s] - OFFI) * (fp16_bits_to_f32(svw[s / 2] >> (16 * (s % 2))) * vm)
                           : tail_value(kc, s) * vm;
      uint32_t hw[4], lw[4];
      split_pairs<4>(y, hw, lw);
      *reinterpret_cast<uint4*>(&sm.vth[bf][e * VROW + t0p]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(&sm.vtl[bf][e * VROW + t0p]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  }
}

// fp16 hi (toward zero) and lo parts of two probabilities: lo = p - hi is
// formed by a mixed-precision fused multiply-add (fp16 hi, fp32 p) and
// rounded once to fp16; p - hi has at most 13 significant bits, so the pair
// is within 2^-22 of p.
__device__ inline void split_p(float p0, float p1, uint32_t& hw, uint32_t& lw) {
  hw = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p0, p1));
  uint32_t lo;
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(lo) : "v"(hw), "v"(p0));
  asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(lo) : "v"(hw), "v"(p1));
  lw = lo;
}

// max / sum of x over lanes l and l ^ 32
__device__ inline float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The state of one wave's 32 rows across the tiles of its split.
struct RowState {
  half8 qh[8], ql[8];   // query operands: B[k][n] = Q'[row n][column 16 ks + 8 h + slot]
  f32x16 o[4];          // O^T accumulators, one per 32-element block
  float m, l, w;
  int lim;
  int fv_seen[4];       // the V exponent each block's accumulators are in
};

// One tile from buffer bf: per 32 positions, S^T = K' Q'^T (M = positions,
// N = rows), the online softmax of row n, then O^T += V'^T P^T.
__device__ inline void tile_products(const PrefillLds& sm, int bf, int t, int n, int h, RowState& st) {
  // rescale a block's accumulators when its exponent went down
  {
    const int4 fvt = *reinterpret_cast<const int4*>(sm.fv[bf]);
    const int fn[4] = {__builtin_amdgcn_readfirstlane(fvt.x), __builtin_amdgcn_readfirstlane(fvt.y),
                       __builtin_amdgcn_readfirstlane(fvt.z), __builtin_amdgcn_readfirstlane(fvt.w)};
#pragma unroll
    for (int me = 0; me < 4; ++me) {
      if (st.fv_seen[me] != kNoScale && fn[me] < st.fv_seen[me]) st.o[me] *= pow2(fn[me] - st.fv_seen[me]);
      st.fv_seen[me] = fn[me];
    }
  }
  const _Float16* khi = sm.khi[bf];
  const _Float16* klo = sm.klo[bf];
  const _Float16* vth = sm.vth[bf];
  const _Float16* vtl = sm.vtl[bf];
  const float* ku = sm.ku[bf];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
    const _Float16* kh = khi + (32 * mt + n) * KROW + 8 * h;
    const _Float16* kl = klo + (32 * mt + n) * KROW + 8 * h;
    // let the scheduler interleave the operand reads with the products, so
    // later steps' LDS reads are in flight during earlier steps' products
    __builtin_amdgcn_iglp_opt(0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const half8 ah = *reinterpret_cast<const half8*>(kh + 16 * ks);
      const half8 al = *reinterpret_cast<const half8*>(kl + 16 * ks);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, st.qh[ks], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, st.qh[ks], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, st.ql[ks], sc, 0, 0, 0);
    }
    float tmax = -INFINITY;
    // causal masking only where some row of the wave stops inside these
    // 32 positions
    const bool masked = __any(t * kTile + 32 * mt + 31 > st.lim);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pos = 32 * mt + 8 * q + 4 * h;     // accumulator rows 4q..4q+3
      const float4 u4 = *reinterpret_cast<const float4*>(ku + pos);
      const float uu[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sc[4 * q + r] * uu[r];
        if (masked) v = t * kTile + pos + r <= st.lim ? v : -INFINITY;
        sc[4 * q + r] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = max_halves(tmax);
    // the reference maximum moves only when the row's maximum passes it by
    // more than kLazy, so probabilities stay below 2^kLazy and the
    // accumulators are rarely rescaled (the partials carry the reference)
    const float mrow = st.w * tmax;
    const float mn = mrow > st.m + kLazy ? mrow : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);   // arguments <= 0
    float ps = 0.f;
    half8 pbh[2], pbl[2];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[r], st.w, -mn));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[r + 1], st.w, -mn));
      ps += p0 + p1;
      uint32_t hw, lw;
      split_p(p0, p1, hw, lw);
      const hpair hh = __builtin_bit_cast(hpair, hw), ll = __builtin_bit_cast(hpair, lw);
      pbh[r / 8][r % 8] = hh[0];
      pbh[r / 8][r % 8 + 1] = hh[1];
      pbl[r / 8][r % 8] = ll[0];
      pbl[r / 8][r % 8 + 1] = ll[1];
    }
    st.l = st.l * alpha + ps;
    st.m = mn;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int me = 0; me < 4; ++me) st.o[me] *= alpha;
    }
    // K order of slot j of half h: 16 s' + 8 (j/4) + 4 h + j%4, the
    // accumulator rows of the scores
    __builtin_amdgcn_iglp_opt(0);
#pragma unroll
    for (int me = 0; me < 4; ++me) {
      const _Float16* vh = vth + (32 * me + n) * VROW + 32 * mt + 4 * h;
      const _Float16* vl = vtl + (32 * me + n) * VROW + 32 * mt + 4 * h;
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const half4 h0 = *reinterpret_cast<const half4*>(vh + 16 * sp);
        const half4 h1 = *reinterpret_cast<const half4*>(vh + 16 * sp + 8);
        const half4 l0 = *reinterpret_cast<const half4*>(vl + 16 * sp);
        const half4 l1 = *reinterpret_cast<const half4*>(vl + 16 * sp + 8);
        const half8 ah = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        const half8 al = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        st.o[me] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, pbh[sp], st.o[me], 0, 0, 0);
        st.o[me] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, pbh[sp], st.o[me], 0, 0, 0);
        st.o[me] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, pbl[sp], st.o[me], 0, 0, 0);
      }
    }
  }
}

// The tiles [t_begin, t_end) for a K wave (KW) or a V wave: the tile after
// the current one is dequantized into the other buffer, the K waves before
// their products and the V waves after them, and the one after that is
// loaded into registers.  Both kinds pass the same barriers.
template <int KB, int VB, bool KW>
__device__ inline void walk_tiles(const PrefillArgs& a, PrefillLds& sm, int b, int g, size_t unit, int nq,
                                  int len, int t_begin, int t_end, int n, int h, RowState& st) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int pl = (tid & 255) >> 2, j = tid & 3, me_s = (tid >> 6) & 3;
  int fv_run = kNoScale;   // V waves: the running exponent of their block
  KRaw kr;
  VRaw vr;
  auto load = [&](int t) {
    const size_t slot = tile_slot_read(a.map, b, g, t);
    if constexpr (KW) load_k<KB>(a, slot, t * kTile + pl < nq, pl, j, kr);
    else load_v<VB>(a, slot, t * kTile + 8 * (lane >> 3) < nq, t * kTile + lane < nq, me_s, lane, vr);
  };
  auto stage = [&](int t, int bf) {
    if constexpr (KW) stage_k<KB>(a, sm, bf, t, nq, len, unit, kr, pl, j);
    else stage_v<VB>(a, sm, bf, t, nq, len, unit, vr, me_s, lane, fv_run);
  };
  if (t_begin < t_end) {
    load(t_begin);
    stage(t_begin, 0);
    if (t_begin + 1 < t_end) load(t_begin + 1);
  }
  __syncthreads();
  for (int t = t_begin; t < t_end; ++t) {
    const int bf = (t - t_begin) & 1;
    if (KW && t + 1 < t_end) {
      stage(t + 1, bf ^ 1);
      if (t + 2 < t_end) load(t + 2);
    }
    tile_products(sm, bf, t, n, h, st);
    if (!KW && t + 1 < t_end) {
      stage(t + 1, bf ^ 1);
      if (t + 2 < t_end) load(t + 2);
    }
    __syncthreads();   // buffer bf ^ 1 is complete; every wave is done with bf
  }
}

template <int KB, int VB>
__global__ __launch_bounds__(kThreads) void prefill_mfma_kernel(PrefillArgs a) {
  __shared__ PrefillLds sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int split = blockIdx.x;
  const int g = blockIdx.y % a.Hkv, rb = blockIdx.y / a.Hkv;
  const int b = blockIdx.z;
  const int len = a.len[b];
  const int nrows = a.n_q * a.G;
  const int nq = len - (a.T > 0 ? min(len, a.T) : 0);   // quantized positions [0, nq)
  const size_t unit = (size_t)b * a.Hkv + g;

  // this lane's row (column n of the products) and its last visible position
  const int row = rb * PR + wave * 32 + n;
  const bool row_ok = row < nrows;
  // tiles holding a position some row of the block sees, split S ways
  const int last_row = min(rb * PR + PR, nrows) - 1;
  const int blim = len - a.n_q + last_row / a.G;
  const int ntiles = blim / kTile + 1;
  const int per = (ntiles + a.S - 1) / a.S;
  const int t_begin = split * per, t_end = min(ntiles, t_begin + per);

  RowState st;
  const size_t qrow = (unit * a.rows_pad + row) * PD;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    st.qh[ks] = *reinterpret_cast<const half8*>(a.q_hi + qrow + 16 * ks + 8 * h);
    st.ql[ks] = *reinterpret_cast<const half8*>(a.q_lo + qrow + 16 * ks + 8 * h);
  }
  st.w = a.q_w[unit * a.rows_pad + row];
  st.lim = row_ok ? len - a.n_q + row / a.G : -1;
  st.m = -1e30f;
  st.l = 0.f;
#pragma unroll
  for (int me = 0; me < 4; ++me) {
    st.fv_seen[me] = kNoScale;
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[me][r] = 0.f;
  }
  if (wave < 4) walk_tiles<KB, VB, true>(a, sm, b, g, unit, nq, len, t_begin, t_end, n, h, st);
  else walk_tiles<KB, VB, false>(a, sm, b, g, unit, nq, len, t_begin, t_end, n, h, st);

  // ---- partials: row (b, i, g*G + h') in the [B][n_q][Hq] order of the output
  const float l = st.l + __shfl_xor(st.l, 32);
  if (!row_ok) return;
  const size_t rv = ((size_t)b * a.n_q + row / a.G) * a.Hq + (size_t)g * a.G + row % a.G;
  if (h == 0) {
    a.part_ml[(rv * a.S + split) * 2] = st.m;
    a.part_ml[(rv * a.S + split) * 2 + 1] = l;
  }
  float* dst = a.part_acc + (rv * a.S + split) * PD;
#pragma unroll
  for (int me = 0; me < 4; ++me) {
    const float un = pow2(st.fv_seen[me] == kNoScale ? 0 : -st.fv_seen[me]);
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[32 * me + 8 * (r / 4) + 4 * h + r % 4] = st.o[me][r] * un;
  }
}

}  // namespace

hipError_t launch_prefill_q(const PrefillArgs& a, int kb, int B, hipStream_t s) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  const dim3 grid(a.rows_pad / 64, a.Hkv, B);
  if (kb == 8) hipLaunchKernelGGL(prefill_q_kernel<8>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(prefill_q_kernel<4>, grid, dim3(256), 0, s, a);   // 4, 5, 6: one column order
  return hipGetLastError();
}

template <int KB, int VB>
void launch_prefill_kv(const PrefillArgs& a, dim3 grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (t0 || t1)
    hipExtLaunchKernelGGL((prefill_mfma_kernel<KB, VB>), grid, dim3(kThreads), 0, s, t0, t1, 0, a);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<KB, VB>), grid, dim3(kThreads), 0, s, a);
}

template <int KB>
void launch_prefill_v(const PrefillArgs& a, int vb, dim3 grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  switch (vb) {
    case 4: launch_prefill_kv<KB, 4>(a, grid, s, t0, t1); break;
    case 5: launch_prefill_kv<KB, 5>(a, grid, s, t0, t1); break;
    case 6: launch_prefill_kv<KB, 6>(a, grid, s, t0, t1); break;
    default: launch_prefill_kv<KB, 8>(a, grid, s, t0, t1); break;
  }
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, int kb, int vb, int B, hipStream_t s,
                               hipEvent_t t0, hipEvent_t t1) {
  (void)hipGetLastError();
  const dim3 grid(a.S, a.n_rb * a.Hkv, B);
  switch (kb) {
    case 4: launch_prefill_v<4>(a, vb, grid, s, t0, t1); break;
    case 5: launch_prefill_v<5>(a, vb, grid, s, t0, t1); break;
    case 6: launch_prefill_v<6>(a, vb, grid, s, t0, t1); break;
    default: launch_prefill_v<8>(a, vb, grid, s, t0, t1); break;
  }
  return hipGetLastError();
}

}  // namespace kvq
