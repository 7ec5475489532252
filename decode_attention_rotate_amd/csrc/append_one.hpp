// One-token append (a decode step) as a device function of one wave, shared
// by the one-token append kernel and the fused decode step, with the
// storage helpers it needs.
//
// Each new K/V head vector is rotated by the normalized Hadamard matrix
// (velog.io post "fix KV cache quantization outliers", section "Hadamard
// rotation") and either quantized into 32-element blocks or, for the newest
// tail_len positions, stored in the bf16 precision tail (aitrends.kr article
// 92204, glossary "Precision Tail").
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace kvq {

// K codes of block j of position p, row layout (tiled 16-byte chunks), from
// the quantizer's words m (low byte: offset code u = c + 2^(BITS-1)).
template <int D, int BITS>
__device__ inline void store_k_row(const uint32_t (&m)[32], uint8_t* plane, int p, int j) {
  constexpr int RP = padded_row_bytes(D, BITS);
  if constexpr (BITS == 8) {
    // two's-complement bytes: u ^ 0x80 = c
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = gather_low_bytes(m[4 * k], m[4 * k + 1], m[4 * k + 2], m[4 * k + 3]) ^ 0x80808080u;
    *reinterpret_cast<uint4*>(plane + chunk_offset(p, 2 * j, RP)) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(plane + chunk_offset(p, 2 * j + 1, RP)) = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    // nibble pairs: element 2i low, 2i+1 high (u < 16 needs no mask)
    uint32_t pr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      pr[i] = BITS == 4 ? (m[2 * i + 1] << 4) | m[2 * i] : (m[2 * i + 1] << 4) | (m[2 * i] & 15u);
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = gather_low_bytes(pr[4 * k], pr[4 * k + 1], pr[4 * k + 2], pr[4 * k + 3]);
    *reinterpret_cast<uint4*>(plane + chunk_offset(p, j, RP)) = make_uint4(w[0], w[1], w[2], w[3]);
    if constexpr (BITS == 5) {
      uint32_t hw = 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) hw |= ((m[e] >> 4) & 1u) << hibit_pos(e);
      const int byte = D / 2 + 4 * j;
      *reinterpret_cast<uint32_t*>(plane + chunk_offset(p, byte / kChunk, RP) + byte % kChunk) = hw;
    }
    if constexpr (BITS == 6) {
      uint32_t hw[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 32; ++e) hw[e / 16] |= ((m[e] >> 4) & 3u) << hi2_pos(e);
      const int byte = D / 2 + 8 * j;
      *reinterpret_cast<uint2*>(plane + chunk_offset(p, byte / kChunk, RP) + byte % kChunk) = make_uint2(hw[0], hw[1]);
    }
  }
}

// Quantize one block with the symmetric rule, or with the scale-and-min
// rule when minf (4/5-bit only); the codes' low bytes are what the planes
// store (c + 2^(bits-1), or the level u), the result the scale (pair) bits.
template <int BITS>
__device__ inline uint32_t quantize_fmt(bool minf, const float (&x)[32], uint32_t (&c)[32]) {
  if constexpr (BITS == 4 || BITS == 5) {
    if (minf) return quantize_block_min<BITS>(x, c);
  }
  return quantize_block<BITS>(x, c);
}

template <int D>
__device__ inline uint32_t quantize_k(int bits, bool minf, const float (&x)[32], uint32_t (&c)[32],
                                      bool active, uint8_t* plane, int p, int j) {
  uint32_t s;
  if (bits == 4) {
    s = quantize_fmt<4>(minf, x, c);
    if (active) store_k_row<D, 4>(c, plane, p, j);
  } else if (bits == 5) {
    s = quantize_fmt<5>(minf, x, c);
    if (active) store_k_row<D, 5>(c, plane, p, j);
  } else if (bits == 6) {
    s = quantize_block<6>(x, c);
    if (active) store_k_row<D, 6>(c, plane, p, j);
  } else {
    s = quantize_block<8>(x, c);
    if (active) store_k_row<D, 8>(c, plane, p, j);
  }
  return s;
}

template <int D>
__device__ inline uint32_t quantize_any(int bits, bool minf, const float (&x)[32], uint32_t (&c)[32]) {
  if (bits == 4) return quantize_fmt<4>(minf, x, c);
  if (bits == 5) return quantize_fmt<5>(minf, x, c);
  if (bits == 6) return quantize_block<6>(x, c);
  return quantize_block<8>(x, c);
}

// Scale entry of block j of position l (0..63) of a tile: one fp16, or an
// (s, m) pair of fp16 (one 32-bit word) for scale-and-min blocks.  sc is the
// tile's first entry.
template <int D>
__device__ inline void store_scale(uint16_t* sc, bool minf, int l, int j, uint32_t s) {
  if (minf) reinterpret_cast<uint32_t*>(sc)[l * (D / kBlock) + j] = s;
  else sc[l * (D / kBlock) + j] = (uint16_t)s;
}
// First scale entry, K row tile and V tile of tile slot `slot` in plane pl.
template <int D, typename A>
__device__ inline uint16_t* scale_tile(const A& a, int pl, size_t slot) {
  return a.scales[pl] + slot * (size_t)kTile * (D / kBlock) * (a.minf[pl] ? 2 : 1);
}
template <int D, typename A>
__device__ inline uint8_t* k_tile(const A& a, size_t slot, int bits) {
  return a.codes[0] + slot * (size_t)kTile * padded_row_bytes(D, bits);
}
template <int D, typename A>
__device__ inline uint8_t* v_tile(const A& a, size_t slot, int bits) {
  return a.codes[1] + slot * (size_t)v_tile_bytes(D, bits);
}

// Outlier channels (a.outl == 32): the bits of block j's elements that are
// in the list of plane pl, KV head g.
template <typename A>
__device__ inline uint32_t outlier_mask(const A& a, int pl, int g, int j) {
  uint32_t m = 0;
  if (!a.outl) return 0u;
  const int32_t* li = a.out_idx + ((size_t)pl * a.Hkv + g) * kOutl;
#pragma unroll 8
  for (int o = 0; o < kOutl; ++o) {
    const int ch = li[o];   // an entry outside [0, D) masks nothing
    if (ch >= 0 && ch / kBlock == j) m |= 1u << (ch % kBlock);
  }
  return m;
}
__device__ inline void zero_masked(float (&x)[32], uint32_t m) {
#pragma unroll
  for (int e = 0; e < 32; ++e) x[e] = (m >> e) & 1u ? 0.f : x[e];
}

// Quantize and store the outlier block of one position of plane pl, KV
// head g: the 32 listed channels of the input row at src + row_off (bf16
// or float32 elements), one 8-bit absmax block.  slot, l: the position's
// tile slot and place in it.  K: bytes [l][32] of the tile, two's
// complement; V: the element-major 8-bit items of a 32-element head, offset
// codes.
template <int D, typename A>
__device__ inline void store_outlier_block(const A& a, int pl, int g, size_t slot, int l, const void* src,
                                           size_t row_off) {
  const int32_t* li = a.out_idx + ((size_t)pl * a.Hkv + g) * kOutl;
  float xo[32];
#pragma unroll
  for (int o = 0; o < kOutl; ++o) {
    const size_t i = row_off + (size_t)outlier_channel(li, o, D);
    xo[o] = a.dtype == KVQ_BF16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(src)[i] << 16)
                                : static_cast<const float*>(src)[i];
  }
  uint32_t c[32];
  const uint32_t s = quantize_block<8>(xo, c);   // offset codes u = c + 128
  uint8_t* tile = a.out_codes[pl] + slot * (kTile * kOutl);
  if (pl == 0) {
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = gather_low_bytes(c[4 * k], c[4 * k + 1], c[4 * k + 2], c[4 * k + 3]) ^ 0x80808080u;
    uint4* dst = reinterpret_cast<uint4*>(tile + l * kOutl);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
#pragma unroll
    for (int o = 0; o < kOutl; ++o) tile[8 * v_item(kOutl, l, o) + l % 8] = (uint8_t)(c[o] & 0xFFu);
  }
  a.out_scales[pl][slot * kTile + l] = (uint16_t)s;
}

// Positions [q0, q1) that become quantized and the first position of the
// tail after the append of sequence b.
struct AppendRange {
  int len, n1, q0, q1, t0;
};
__device__ inline AppendRange append_range(const AppendArgs& a, int b) {
  AppendRange r;
  r.len = a.len[b];
  r.n1 = r.len + a.n_new;
  const int T = a.T;
  r.q0 = T > 0 ? max(0, r.len - T) : r.len;
  r.q1 = T > 0 ? max(0, r.n1 - T) : r.n1;
  r.t0 = max(r.len, r.n1 - T);
  return r;
}

// Append one new token to plane pl of (sequence b, KV head g), by one whole
// wave (a decode step).  Lanes [0, LPR) hold the new token's blocks and
// rotate them; lanes [32, 32 + LPR) hold the row leaving the bf16 tail, when
// there is one.  The position that becomes quantized is the new token itself
// without a tail, the leaving row with one.  It runs in two phases so a
// caller can issue the loads of both planes (and its own) before waiting:
// append_one_load issues every global load (input row, ring row, the V
// items the quantized codes merge into) into an OneLoads; append_one_finish
// rotates, quantizes and stores.  The new row overwrites the ring slot the
// leaving row was read from: the quantizer has consumed that row by then.
// store: write the cache (false: only compute the values below).
// out_new (T > 0): the new token's values as the tail stores them, the
// plane's D floats; out_q: the dequantized values of the position that
// becomes quantized (code * scale, or level * scale + minimum), when there
// is one.  Either may be null.
// FAST: no tail and absmax blocks in both planes (see the bulk append).
// len: the sequence's length before the append.  KBS: K's width when the
// caller knows it at compile time (0: a.bits[0]).
struct OneLoads {
  uint4 rin[8], rring[4];
  uint32_t oldw[32], oldh[32];
};

struct OneLayout {
  int j, pq, len, T;
  bool new_lane, ring_lane, q_lane, has_q;
  size_t qs, unit;
};
template <int D>
__device__ inline OneLayout one_layout(const OneArgs& a, int g, int b, int len) {
  constexpr int LPR = D / kBlock;
  const int lane = threadIdx.x & 63;
  OneLayout o;
  o.j = (lane & 31) % LPR;   // block of lane l and of lane 32 + l
  o.T = a.T;
  o.len = len;
  const int q0 = o.T > 0 ? max(0, len - o.T) : len;
  const int q1 = o.T > 0 ? max(0, len + 1 - o.T) : len + 1;
  o.has_q = q1 > q0;
  o.new_lane = lane < LPR;
  o.ring_lane = o.T > 0 && o.has_q && lane >= 32 && lane < 32 + LPR;
  o.pq = q0;                                   // the quantized position
  // slot of pq's tile (-1: no quantized position, or a page outside the pool)
  const long long qslot = o.has_q ? tile_slot(a.map, b, g, o.pq / kTile) : -1LL;
  o.q_lane = qslot >= 0 && (o.T > 0 ? o.ring_lane : o.new_lane);
  o.qs = qslot >= 0 ? (size_t)qslot : 0;
  o.unit = (size_t)b * a.Hkv + g;
  return o;
}

template <int D, int VB>
__device__ inline void append_one_load(const OneArgs& a, int g, int b, int pl, int len, bool store,
                                       OneLoads& L) {
  const OneLayout o = one_layout<D>(a, g, b, len);
#pragma unroll
  for (int q = 0; q < 8; ++q) L.rin[q] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int q = 0; q < 4; ++q) L.rring[q] = make_uint4(0u, 0u, 0u, 0u);
  if (o.new_lane) {
    const size_t off = o.unit * D + (size_t)kBlock * o.j;
    if (a.dtype == KVQ_BF16) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src[pl]) + off);
#pragma unroll
      for (int q = 0; q < 4; ++q) L.rin[q] = src[q];
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(a.src[pl]) + off);
#pragma unroll
      for (int q = 0; q < 8; ++q) L.rin[q] = src[q];
    }
  }
  if (o.ring_lane) {
    const uint4* src = reinterpret_cast<const uint4*>(a.tail[pl] + (o.unit * o.T + o.pq % o.T) * D + kBlock * o.j);
#pragma unroll
    for (int q = 0; q < 4; ++q) L.rring[q] = src[q];
  }
  // V items of this lane's 32 elements at the quantized position
  if constexpr (VB != 8) {
    if (store && pl == 1 && o.q_lane) {
      const uint8_t* vtile = v_tile<D>(a, o.qs, VB);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int item = v_item(D, o.pq % kTile, kBlock * o.j + i);
        L.oldw[i] = reinterpret_cast<const uint32_t*>(vtile)[item];
        if constexpr (VB == 5) L.oldh[i] = vtile[32 * D + item];
        if constexpr (VB == 6) L.oldh[i] = reinterpret_cast<const uint16_t*>(vtile + 32 * D)[item];
      }
    }
  }
}

template <int D, int VB, bool FAST, int KBS = 0>
__device__ inline void append_one_finish(const OneArgs& a, int g, int b, int pl, int len, bool store,
                                         const OneLoads& L, float* out_new, float* out_q) {
  const int lane = threadIdx.x & 63;
  const OneLayout o = one_layout<D>(a, g, b, len);
  const int j = o.j, T = o.T, pq = o.pq;
  const size_t qs = o.qs;
  const int bits = pl == 0 ? (KBS ? KBS : a.bits[0]) : VB;   // V's width is the template's
  uint8_t* vtile = v_tile<D>(a, qs, VB);

  float x[32], y[32];
  auto widen_bf16 = [](const uint4 (&r)[8], float (&f)[32]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w[4] = {r[q].x, r[q].y, r[q].z, r[q].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f[q * 8 + 2 * k] = __uint_as_float(w[k] << 16);
        f[q * 8 + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
  };
  if (a.dtype == KVQ_BF16) {
    widen_bf16(L.rin, x);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      x[4 * q] = __uint_as_float(L.rin[q].x); x[4 * q + 1] = __uint_as_float(L.rin[q].y);
      x[4 * q + 2] = __uint_as_float(L.rin[q].z); x[4 * q + 3] = __uint_as_float(L.rin[q].w);
    }
  }
  {
    uint4 r8[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) { r8[q] = L.rring[q]; r8[q + 4] = make_uint4(0u, 0u, 0u, 0u); }
    widen_bf16(r8, y);
  }
  if (a.outl && o.new_lane) zero_masked(x, outlier_mask(a, pl, g, j));   // the rest only
  if (a.rotate[pl]) {                            // every lane takes part
    if (a.has_signs) apply_signs(x, a.signs[j]);
    if constexpr (FAST) rotate_row_for_absmax<D>(x, lane, a.cd);
    else rotate_row<D>(x, lane, a.cd);
  }
  // outlier channels (no tail: the new token is the quantized position)
  if (a.outl && store && lane == 0 && o.q_lane)
    store_outlier_block<D>(a, pl, g, qs, pq % kTile, a.src[pl], o.unit * D);
  if (out_new && T > 0 && o.new_lane) {
#pragma unroll
    for (int e = 0; e < 32; ++e) out_new[kBlock * j + e] = bf16_round(x[e]);
  }
  // the quantizer consumes the ring row here, before the new row's store
  // below overwrites its slot (program order; the wave waits for the load
  // before its first use)
  if (o.q_lane || (out_q && o.has_q && (T > 0 ? o.ring_lane : o.new_lane))) {
    float z[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) z[e] = T > 0 ? y[e] : x[e];
    const bool minf = a.minf[pl] != 0;
    uint16_t* scales = scale_tile<D>(a, pl, qs);
    uint32_t c[32];
    const uint32_t s = pl == 0 ? quantize_k<D>(bits, minf, z, c, store && o.q_lane, k_tile<D>(a, qs, bits),
                                               pq % kTile, j)
                               : quantize_fmt<VB>(minf, z, c);
    if (out_q) {
      // what a read of the cache gives: (u - 2^(bits-1)) * s, or u * s + m
      const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)(s & 0xFFFFu));
      const float mf = (float)__builtin_bit_cast(_Float16, (uint16_t)(s >> 16));
      const int off = minf ? 0 : 1 << (bits - 1);
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float lv = (float)((int)(c[e] & 0xFFu) - off) * sf;
        out_q[kBlock * j + e] = minf ? lv + mf : lv;
      }
    }
    if (store && o.q_lane) store_scale<D>(scales, minf, pq % kTile, j, s);
    if (store && o.q_lane && pl == 1) {
      const int k = pq % 8;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int item = v_item(D, pq % kTile, kBlock * j + i);
        const uint32_t u = c[i] & 0xFFu;   // offset code
        if constexpr (VB == 8) {
          vtile[8 * item + k] = (uint8_t)u;
        } else {
          const int nb = v_nibble(k);
          reinterpret_cast<uint32_t*>(vtile)[item] = (L.oldw[i] & ~(15u << (4 * nb))) | ((u & 15u) << (4 * nb));
          if constexpr (VB == 5)
            vtile[32 * D + item] = (uint8_t)((L.oldh[i] & ~(1u << nb)) | (((u >> 4) & 1u) << nb));
          if constexpr (VB == 6)
            reinterpret_cast<uint16_t*>(vtile + 32 * D)[item] =
                (uint16_t)((L.oldh[i] & ~(3u << (2 * nb))) | (((u >> 4) & 3u) << (2 * nb)));
        }
      }
    }
  }
  if (T == 0 || !store) return;
  if (o.new_lane) {
    uint4* dst = reinterpret_cast<uint4*>(a.tail[pl] + (o.unit * T + o.len % T) * D + kBlock * j);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = f32_to_bf16_bits(x[q * 8 + 2 * k]) | (f32_to_bf16_bits(x[q * 8 + 2 * k + 1]) << 16);
      dst[q] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

}  // namespace kvq
