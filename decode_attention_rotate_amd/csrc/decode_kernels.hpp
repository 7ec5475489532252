// Split-K single-query decode attention over the rotated block-quantized cache.
//
// Method (velog.io post "fix KV cache quantization outliers", section
// "Hadamard rotation"): scores are dot products of the rotated query with the
// rotated keys (the rotation is orthogonal, so they equal the unrotated
// scores), softmax, weighted sum of the rotated values; the combine kernel
// rotates the result back.  Newest tokens may sit unquantized in a bf16 tail
// (aitrends.kr article 92204, glossary "Precision Tail").
//
// One wave handles one (sequence b, KV head g, chunk of G query heads, split
// of the context) and streams every cache byte of its split exactly once.
// Each tile of 64 tokens runs in two layouts:
//  * Q.K, one token per lane.  K codes come in 16-byte chunks laid out so that
//    chunk c of the 64 tokens of a tile is 1 KB of contiguous memory.  The
//    query is held as a 16-bit fixed-point number split into two int8 planes
//    (high and low byte), read with scalar loads, so each group of four codes
//    costs two v_dot4_i32_i8 per head with no code conversion.  Offset-binary
//    4/5-bit codes are folded back to signed codes through a per-block
//    correction that initialises the accumulator.  Per block:
//      score += scale_k[j] * float(256 * dot(q_hi, u) + dot(q_lo, u) + corr_j)
//  * P.V, eight output elements per lane (D/8 lanes per token).  The softmax
//    weight of each token, already multiplied by the token's per-block V
//    scale and rounded to fp16, moves through LDS; two tokens' codes are
//    interleaved with v_perm into fp16 pairs (magic-number conversion, then an
//    exact subtraction of the bias) and v_dot2_f32_f16 accumulates both tokens
//    into a float32 accumulator in one instruction.
// The online softmax keeps one running maximum per head for the whole wave
// and rescales only when some lane's score exceeds it.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace kvq {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
using sgpr_i32 = const int32_t __attribute__((address_space(4)))*;
using sgpr_f32 = const float __attribute__((address_space(4)))*;

constexpr float kLog2e = 1.4426950408889634f;

// Relative cost of a 64-token tile: quantized codes vs bf16 tail rows.
constexpr int kCostQ = 2;
constexpr int kCostT = 5;

// Occupancy target of the split-K kernel (waves per SIMD); bounds the
// registers the scheduler may use.
#ifndef KVQ_SPLIT_WAVES_PER_EU
#define KVQ_SPLIT_WAVES_PER_EU 2
#endif

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

// Maximum / sum over the 64 lanes, result in every lane.
__device__ inline float wave_max(float v) {
  v = fmaxf(v, xor_lane<1>(v));
  v = fmaxf(v, xor_lane<2>(v));
  v = fmaxf(v, xor_lane<4>(v));
  v = fmaxf(v, xor_lane<8>(v));
  v = fmaxf(v, xor_lane<16>(v));
  const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  return fmaxf(lo, hi);
}
__device__ inline float wave_sum(float v) {
  v += xor_lane<1>(v);
  v += xor_lane<2>(v);
  v += xor_lane<4>(v);
  v += xor_lane<8>(v);
  v += xor_lane<16>(v);
  const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  return lo + hi;
}

// K codes of one token unpacked into D/4 dwords of byte-sized values in the
// order the prep kernel lays out the query bytes.
template <int D, int KB>
__device__ inline void unpack_k(const uint32_t* kw, uint32_t (&kb)[D / 4]) {
  if constexpr (KB == 8) {
#pragma unroll
    for (int w = 0; w < D / 4; ++w) kb[w] = kw[w];
  } else {
#pragma unroll
    for (int w = 0; w < D / 8; ++w) {
      uint32_t lo = kw[w] & 0x0F0F0F0Fu;
      uint32_t hi = (kw[w] >> 4) & 0x0F0F0F0Fu;
      if constexpr (KB == 5) {
        const uint32_t hw = kw[D / 8 + w / 4];
        const int gq = w % 4;
        const int sl = 4 - 2 * gq, sh = 3 - 2 * gq;
        const uint32_t tl = sl >= 0 ? (hw << sl) : (hw >> (-sl));
        const uint32_t th = sh >= 0 ? (hw << sh) : (hw >> (-sh));
        lo |= tl & 0x10101010u;
        hi |= th & 0x10101010u;
      }
      kb[2 * w] = lo;
      kb[2 * w + 1] = hi;
    }
  }
}

// Eight fp16 code pairs (token A in the low half, token B in the high half)
// for the eight elements a P.V lane owns.
template <int VB>
struct VTok;

// Byte k of token A in the low half and byte k of token B in the high half.
__device__ inline uint32_t pair_bytes(uint32_t b, uint32_t a, int k) {
  return __builtin_amdgcn_perm(b, a, (uint32_t)k | (0x0Cu << 8) | ((uint32_t)(4 + k) << 16) | (0x0Cu << 24));
}

// (x & mask) | magic as one v_and_or_b32; magic lives in a VGPR.
__device__ inline uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  return (x & mask) | magic;
}

template <>
struct VTok<4> {
  uint32_t n;  // 8 nibbles: element i in bits 4i..4i+3
  // Even elements become exact fp16 codes c; odd elements become 16*c
  // (nibble kept in mantissa bits 4..7), undone once when partials are stored.
  static constexpr bool kOddTimes16 = true;
  __device__ inline void pairs(const VTok& B, h2_t (&c)[8], uint32_t magic) const {
    const h2_t bias_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2_t bias_hi = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t p = pair_bytes(B.n, n, k);
      c[2 * k] = as_h2(and_or(p, 0x000F000Fu, magic)) + bias_lo;
      c[2 * k + 1] = as_h2(and_or(p, 0x00F000F0u, magic)) + bias_hi;
    }
  }
};

template <>
struct VTok<8> {
  uint32_t b0, b1;  // 8 signed bytes
  static constexpr bool kOddTimes16 = false;
  __device__ inline void pairs(const VTok& B, h2_t (&c)[8], uint32_t) const {
    const h2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c[k] = as_h2(pair_bytes(B.b0, b0, k) ^ 0x64806480u) + bias;
      c[4 + k] = as_h2(pair_bytes(B.b1, b1, k) ^ 0x64806480u) + bias;
    }
  }
};

template <>
struct VTok<5> {
  uint32_t n;   // 8 nibbles
  uint32_t hw;  // high-bit word of the block
  int gq;       // which 8-element group of the block this lane owns
  static constexpr bool kOddTimes16 = false;
  __device__ inline void pairs(const VTok& B, h2_t (&c)[8], uint32_t) const {
    const uint32_t x1 = __builtin_amdgcn_perm(B.n, n, 0x05040100u);
    const uint32_t x2 = __builtin_amdgcn_perm(B.n, n, 0x07060302u);
    const h2_t bias = {(_Float16)-1040.0f, (_Float16)-1040.0f};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t x = e < 4 ? x1 : x2;
      const uint32_t nib = (x >> (4 * (e % 4))) & 0x000F000Fu;
      const int i = e / 2, nb = e % 2;
      const uint32_t sel = (uint32_t)i | (0x0Cu << 8) | ((uint32_t)(4 + i) << 16) | (0x0Cu << 24);
      const uint32_t hb = __builtin_amdgcn_perm(B.hw, hw, sel);   // bit 2*gq+nb of each half
      const int sh = 4 - 2 * gq - nb;
      const uint32_t hbs = sh >= 0 ? (hb << sh) : (hb >> (-sh));
      c[e] = as_h2(nib | (hbs & 0x00100010u) | 0x64006400u) + bias;
    }
  }
};

template <int D, int KB, int VB>
struct TileRegs {
  static constexpr int NB = D / kBlock;
  static constexpr int NCK = padded_row_bytes(D, KB) / kChunk;
  static constexpr int TPS = D / 8;   // tokens per P.V slot in a tile
  uint4 kc[NCK];
  uint32_t ks[NB / 2];   // fp16 K scales of this lane's token
  uint32_t vs[NB / 2];   // fp16 V scales of this lane's token
  VTok<VB> v[TPS];
};

template <int D, int KB, int VB, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(KVQ_SPLIT_WAVES_PER_EU))) void decode_split_kernel(DecodeArgs a) {
  constexpr int NB = D / kBlock;
  constexpr int RKP = padded_row_bytes(D, KB);
  constexpr int RVP = padded_row_bytes(D, VB);
  constexpr int NCK = RKP / kChunk;
  constexpr int LPRV = D / 8;
  constexpr int NSLOT = 64 / LPRV;
  constexpr int TPS = 64 / NSLOT;
  constexpr int NPAIR = TPS / 2;
  constexpr int QPS = qp_stride(D);
  using Regs = TileRegs<D, KB, VB>;

  // per head: D/4 dwords of high query bytes, D/4 of low bytes, NB block
  // corrections, the fixed-point score multiplier; padded to 16 bytes
  constexpr int QCK = D / 2 + NB;
  constexpr int QLD = (QCK + 1 + 3) / 4 * 4;
  __shared__ __align__(16) uint32_t qlds[G][QLD];
  __shared__ __align__(16) uint32_t wlds[G][NB][32];
  __shared__ float plds[G][64];

  const int lane = threadIdx.x;
  const int split = blockIdx.x;
  const int g = blockIdx.y / a.n_gchunks;
  const int h0 = g * a.G + (blockIdx.y % a.n_gchunks) * G;
  const int b = blockIdx.z;
  const int n = a.len[b];
  const int T = a.T;
  const int nt = T > 0 ? min(n, T) : 0;
  const int nq = n - nt;
  // Work split by cost, not by token count: a 64-token tile of quantized
  // codes weighs kCostQ, a tile of bf16 tail tokens kCostT (it carries about
  // 2.5x the bytes).  Split s of S takes the cost interval [s*C/S, (s+1)*C/S)
  // of this sequence; boundaries fall on tile edges of each region.
  const int ctq = (nq + kTile - 1) / kTile;       // quantized tiles
  const int ctt = (nt + kTile - 1) / kTile;       // tail tiles
  const int64_t C = (int64_t)kCostQ * ctq + (int64_t)kCostT * ctt;
  const int64_t c0 = C * split / a.S, c1 = C * (split + 1) / a.S;
  auto q_tiles = [&](int64_t c) {
    const int64_t t = c / kCostQ;
    return (int)(t < ctq ? t : ctq);
  };
  auto t_tiles = [&](int64_t c) {
    const int64_t r = (c - (int64_t)kCostQ * ctq) / kCostT;
    return r <= 0 ? 0 : (int)(r < ctt ? r : ctt);
  };
  const int qa = q_tiles(c0) * kTile, qb = min(nq, q_tiles(c1) * kTile);
  const int ta = nq + t_tiles(c0) * kTile, tb = min(n, nq + t_tiles(c1) * kTile);
  const size_t unit = (size_t)b * a.Hkv + g;

  const uint8_t* kpl = a.k_codes + unit * (size_t)a.cap * RKP;
  const uint16_t* ksc = a.k_scales + unit * (size_t)a.cap * NB;
  const uint8_t* vpl = a.v_codes + unit * (size_t)a.cap * RVP;
  const uint16_t* vsc = a.v_scales + unit * (size_t)a.cap * NB;
  const uint8_t* qp0 = a.qp + ((size_t)b * a.Hq + h0) * QPS;

  const int slot = lane / LPRV;
  const int eg = lane % LPRV;
  const int jv = eg / 4;
  const int kq = lane / NSLOT;
  const int hidx = ((lane % NSLOT) * NPAIR + (kq >> 1)) * 2 + (kq & 1);

  for (int i = lane; i < G * (QCK + 1); i += 64) {
    const int h = i / (QCK + 1), k = i % (QCK + 1);
    qlds[h][k] = reinterpret_cast<const uint32_t*>(qp0 + (size_t)h * QPS)[k];
  }
  __syncthreads();

  float m[G], ls[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    ls[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  // Online-softmax step shared by the quantized and the tail loops:
  // x holds this lane's scores (log2 units, -inf for masked lanes).
  // Online-softmax step shared by the quantized and the tail loops:
  // x holds this lane's scores (log2 units, -inf for masked lanes).  The
  // running maxima only move when some lane exceeds them (a wave-uniform
  // branch); the rescale of the accumulators is applied unconditionally so
  // the common path carries no register shuffles.
  auto softmax_update = [&](float (&x)[G], float (&p)[G]) {
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) need |= x[h] > m[h];
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], wave_max(x[h]));
        const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
        m[h] = mn;
        ls[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      p[h] = __builtin_amdgcn_exp2f(x[h] - m[h]);
      ls[h] += p[h];
    }
  };

  // ------------------------------------------------ quantized positions
  if (qa < qb) {
    const int last = (qb - 1) / kTile * kTile;
    // per-lane byte offsets inside a tile; the tile base is uniform
    const uint32_t k_off = lane * kChunk;
    const uint32_t s_off = lane * NB * 2;
    uint32_t v_off, vh_off = 0;
    if constexpr (VB == 8) {
      v_off = ((eg / 2) * kTile + slot) * kChunk + (eg % 2) * 8;
    } else {
      v_off = ((eg / 4) * kTile + slot) * kChunk + (eg % 4) * 4;
      const int byte = D / 2 + 4 * jv;
      vh_off = ((byte / kChunk) * kTile + slot) * kChunk + byte % kChunk;
    }

    auto load_tile = [&](Regs& r, int t0) {
      const uint8_t* kt = kpl + (size_t)(t0 / kTile) * kTile * RKP;
#pragma unroll
      for (int c = 0; c < NCK; ++c)
        r.kc[c] = *reinterpret_cast<const uint4*>(kt + c * kTile * kChunk + k_off);
      const uint8_t* ks = reinterpret_cast<const uint8_t*>(ksc + (size_t)t0 * NB) + s_off;
      const uint8_t* vs = reinterpret_cast<const uint8_t*>(vsc + (size_t)t0 * NB) + s_off;
      if constexpr (NB == 2) {
        r.ks[0] = *reinterpret_cast<const uint32_t*>(ks);
        r.vs[0] = *reinterpret_cast<const uint32_t*>(vs);
      } else if constexpr (NB == 4) {
        const uint2 k2 = *reinterpret_cast<const uint2*>(ks);
        const uint2 v2 = *reinterpret_cast<const uint2*>(vs);
        r.ks[0] = k2.x; r.ks[1] = k2.y; r.vs[0] = v2.x; r.vs[1] = v2.y;
      } else {
        const uint4 k4 = *reinterpret_cast<const uint4*>(ks);
        const uint4 v4 = *reinterpret_cast<const uint4*>(vs);
        r.ks[0] = k4.x; r.ks[1] = k4.y; r.ks[2] = k4.z; r.ks[3] = k4.w;
        r.vs[0] = v4.x; r.vs[1] = v4.y; r.vs[2] = v4.z; r.vs[3] = v4.w;
      }
      const uint8_t* vt = vpl + (size_t)(t0 / kTile) * kTile * RVP;
#pragma unroll
      for (int k = 0; k < TPS; ++k) {
        const uint8_t* vk = vt + k * NSLOT * kChunk;
        if constexpr (VB == 4) {
          r.v[k].n = *reinterpret_cast<const uint32_t*>(vk + v_off);
        } else if constexpr (VB == 8) {
          const uint2 v = *reinterpret_cast<const uint2*>(vk + v_off);
          r.v[k].b0 = v.x; r.v[k].b1 = v.y;
        } else {
          r.v[k].n = *reinterpret_cast<const uint32_t*>(vk + v_off);
          r.v[k].hw = *reinterpret_cast<const uint32_t*>(vk + vh_off);
          r.v[k].gq = eg % 4;
        }
      }
    };

    auto compute_tile = [&](const Regs& r, int t0) {
      const bool valid = t0 + lane < qb;
      uint32_t kw[NCK * 4];
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        kw[4 * c] = r.kc[c].x; kw[4 * c + 1] = r.kc[c].y;
        kw[4 * c + 2] = r.kc[c].z; kw[4 * c + 3] = r.kc[c].w;
      }
      uint32_t kb[D / 4];
      unpack_k<D, KB>(kw, kb);
      float ksf[NB], vsf[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        ksf[j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(r.ks[j / 2] >> (16 * (j % 2))));
        vsf[j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(r.vs[j / 2] >> (16 * (j % 2))));
      }
      // Query bytes come from LDS (same address in every lane: a broadcast).
      // The read of block b is tied (empty asm on an opaque offset) to the
      // result of block b-2, so at most about three blocks of query bytes are
      // live: the reads run two blocks ahead of their use and cannot all be
      // hoisted to the top of the tile.
      int qz = 0;
      int ring[2] = {0, 0};
      float s[G];
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
      for (int bi = 0; bi < G * NB; ++bi) {
        const int h = bi / NB, j = bi % NB;
        asm volatile("" : "+s"(qz) : "v"(ring[bi % 2]));
        const uint32_t* qh = &qlds[h][0] + qz;
        const uint4 h0 = *reinterpret_cast<const uint4*>(qh + 8 * j);
        const uint4 h1 = *reinterpret_cast<const uint4*>(qh + 8 * j + 4);
        const uint4 l0 = *reinterpret_cast<const uint4*>(qh + D / 4 + 8 * j);
        const uint4 l1 = *reinterpret_cast<const uint4*>(qh + D / 4 + 8 * j + 4);
        const uint32_t qhi[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        const uint32_t qlo[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        int ahi = 0, alo = (int)qh[D / 2 + j];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          ahi = __builtin_amdgcn_sdot4((int)qhi[w], (int)kb[8 * j + w], ahi, false);
          alo = __builtin_amdgcn_sdot4((int)qlo[w], (int)kb[8 * j + w], alo, false);
        }
        const int dj = ahi * 256 + alo;
        ring[bi % 2] = dj;
        s[h] = __builtin_fmaf(ksf[j], (float)dj, s[h]);
      }
      float x[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float xv = s[h] * __uint_as_float(qlds[h][QCK + qz]);
        asm volatile("" : "+v"(xv));   // computed in every lane: a select, not a branch
        x[h] = valid ? xv : -INFINITY;
      }
      float p[G];
      softmax_update(x, p);
      __syncthreads();
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const float wv = valid ? p[h] * vsf[j] : 0.f;
          reinterpret_cast<_Float16*>(&wlds[h][j][0])[hidx] = (_Float16)wv;
        }
      }
      __syncthreads();
      uint32_t magic = 0x64006400u;
      asm volatile("" : "+v"(magic));
#pragma unroll
      for (int q2 = 0; q2 < NPAIR; q2 += 2) {
        u32x2 wq[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
          wq[h] = *reinterpret_cast<const u32x2*>(&wlds[h][jv][slot * NPAIR + q2]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          h2_t c[8];
          r.v[2 * (q2 + u)].pairs(r.v[2 * (q2 + u) + 1], c, magic);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const h2_t wp = as_h2(wq[h][u]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_amdgcn_fdot2(wp, c[e], acc[h][e], false);
          }
        }
      }
    };

    Regs ra, rb;
    load_tile(ra, qa);
    for (int t = qa; t < qb; t += 2 * kTile) {
      const int t1 = t + kTile;
      load_tile(rb, min(t1, last));
      compute_tile(ra, t);
      if (t1 >= qb) break;
      load_tile(ra, min(t1 + kTile, last));
      compute_tile(rb, t1);
    }
    if constexpr (VTok<VB>::kOddTimes16) {
      // odd elements were accumulated as 16*c (see VTok<4>); the tail loop
      // below accumulates plain values, so undo the factor before it runs
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 1; e < 8; e += 2) acc[h][e] *= 0.0625f;
      }
    }
  }

  // ------------------------------------------------ bf16 tail positions
  if (ta < tb) {
    const uint16_t* ktl = a.k_tail + unit * (size_t)T * D;
    const uint16_t* vtl = a.v_tail + unit * (size_t)T * D;
    for (int t0 = ta; t0 < tb; t0 += kTile) {
      const int t = t0 + lane;
      const bool valid = t < tb;
      const int sl = (valid ? t : t0) % T;
      const uint16_t* krow = ktl + (size_t)sl * D;
      const uint8_t* qbase = qp0;
      asm volatile("" : "+s"(qbase));
      float s[G];
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const uint4 kv = *reinterpret_cast<const uint4*>(krow + 8 * c);
        const uint32_t w4[4] = {kv.x, kv.y, kv.z, kv.w};
        float kf[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          kf[2 * k] = __uint_as_float(w4[k] << 16);
          kf[2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const sgpr_f32 qr = (sgpr_f32)(qbase + (size_t)h * QPS + 4 * D);
#pragma unroll
          for (int e = 0; e < 8; ++e) s[h] = __builtin_fmaf(qr[8 * c + e], kf[e], s[h]);
        }
      }
      float x[G], p[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float cs = *(sgpr_f32)(qbase + (size_t)h * QPS + 2 * D + D / 8 + 4);
        x[h] = valid ? s[h] * cs : -INFINITY;
      }
      softmax_update(x, p);
      __syncthreads();
#pragma unroll
      for (int h = 0; h < G; ++h) plds[h][lane] = p[h];
      __syncthreads();
#pragma unroll 4
      for (int k = 0; k < TPS; ++k) {
        const int tl = k * NSLOT + slot;
        const int tt = t0 + tl;
        const int sv = (tt < tb ? tt : t0) % T;
        const uint4 vv = *reinterpret_cast<const uint4*>(vtl + (size_t)sv * D + 8 * eg);
        const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
        float vf[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          vf[2 * q] = __uint_as_float(w4[q] << 16);
          vf[2 * q + 1] = __uint_as_float(w4[q] & 0xFFFF0000u);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ph = plds[h][tl];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(ph, vf[e], acc[h][e]);
        }
      }
    }
  }

  // ------------------------------------------------ partial results
#pragma unroll
  for (int h = 0; h < G; ++h) ls[h] = wave_sum(ls[h]);
#pragma unroll
  for (int s = LPRV; s < 64; s <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], s);
    }
  }
  const size_t row0 = ((size_t)b * a.Hq + h0) * a.S + split;
  if (lane < LPRV) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(a.part_acc + (row0 + (size_t)h * a.S) * D + 8 * eg);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      a.part_ml[(row0 + (size_t)h * a.S) * 2] = m[h];
      a.part_ml[(row0 + (size_t)h * a.S) * 2 + 1] = ls[h];
    }
  }
}

template <int D, int KB, int VB, int G>
hipError_t launch_decode_split(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  hipLaunchKernelGGL((decode_split_kernel<D, KB, VB, G>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
