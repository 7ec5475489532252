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

__device__ inline h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }
__device__ inline uint32_t as_u32(h2_t v) { return __builtin_bit_cast(uint32_t, v); }

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

template <>
struct VTok<4> {
  uint32_t n;  // 8 nibbles
  __device__ inline void pairs(const VTok& B, h2_t (&c)[8]) const {
    const uint32_t x1 = __builtin_amdgcn_perm(B.n, n, 0x05040100u);
    const uint32_t x2 = __builtin_amdgcn_perm(B.n, n, 0x07060302u);
    const h2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = as_h2(((x1 >> (4 * i)) & 0x000F000Fu) | 0x64006400u) + bias;
      c[4 + i] = as_h2(((x2 >> (4 * i)) & 0x000F000Fu) | 0x64006400u) + bias;
    }
  }
};

template <>
struct VTok<8> {
  uint32_t b0, b1;  // 8 signed bytes
  __device__ inline void pairs(const VTok& B, h2_t (&c)[8]) const {
    const h2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t sel = (uint32_t)i | (0x0Cu << 8) | ((uint32_t)(4 + i) << 16) | (0x0Cu << 24);
      c[i] = as_h2(__builtin_amdgcn_perm(B.b0, b0, sel) ^ 0x64806480u) + bias;
      c[4 + i] = as_h2(__builtin_amdgcn_perm(B.b1, b1, sel) ^ 0x64806480u) + bias;
    }
  }
};

template <>
struct VTok<5> {
  uint32_t n;   // 8 nibbles
  uint32_t hw;  // high-bit word of the block
  int gq;       // which 8-element group of the block this lane owns
  __device__ inline void pairs(const VTok& B, h2_t (&c)[8]) const {
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
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
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
  const int p0 = split * a.split_tokens;
  const int p1 = min(n, p0 + a.split_tokens);
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
  auto softmax_update = [&](float (&x)[G], float (&p)[G]) {
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) need |= x[h] > m[h];
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], wave_max(x[h]));
        const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
        ls[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
        m[h] = mn;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      p[h] = __builtin_amdgcn_exp2f(x[h] - m[h]);
      ls[h] += p[h];
    }
  };

  // ------------------------------------------------ quantized positions
  const int qa = p0, qb = min(p1, nq);
  if (qa < qb) {
    const int last = (qb - 1) / kTile * kTile;
    auto load_tile = [&](Regs& r, int t0) {
      const uint8_t* kt = kpl + (size_t)(t0 / kTile) * kTile * RKP;
#pragma unroll
      for (int c = 0; c < NCK; ++c)
        r.kc[c] = *reinterpret_cast<const uint4*>(kt + (size_t)(c * kTile + lane) * kChunk);
      const uint16_t* ks = ksc + (size_t)(t0 + lane) * NB;
      const uint16_t* vs = vsc + (size_t)(t0 + lane) * NB;
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
        const int t = k * NSLOT + slot;
        if constexpr (VB == 4) {
          r.v[k].n = *reinterpret_cast<const uint32_t*>(vt + (size_t)((eg / 4) * kTile + t) * kChunk + (eg % 4) * 4);
        } else if constexpr (VB == 8) {
          const uint2 v = *reinterpret_cast<const uint2*>(vt + (size_t)((eg / 2) * kTile + t) * kChunk + (eg % 2) * 8);
          r.v[k].b0 = v.x; r.v[k].b1 = v.y;
        } else {
          r.v[k].n = *reinterpret_cast<const uint32_t*>(vt + (size_t)((eg / 4) * kTile + t) * kChunk + (eg % 4) * 4);
          constexpr int hb0 = D / 2;
          const int byte = hb0 + 4 * jv;
          r.v[k].hw = *reinterpret_cast<const uint32_t*>(vt + (size_t)((byte / kChunk) * kTile + t) * kChunk + byte % kChunk);
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
      // scalar-load the fixed-point query for each head (kept out of the
      // loop-invariant set so it does not pin hundreds of SGPRs)
      const uint8_t* qbase = qp0;
      asm volatile("" : "+s"(qbase));
      float x[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint8_t* qh8 = qbase + (size_t)h * QPS;
        const sgpr_i32 qhi = (sgpr_i32)(qh8);
        const sgpr_i32 qlo = (sgpr_i32)(qh8 + D);
        const sgpr_i32 corr = (sgpr_i32)(qh8 + 2 * D);
        const float ck = *(sgpr_f32)(qh8 + 2 * D + D / 8);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          int ahi = 0, alo = corr[j];
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            ahi = __builtin_amdgcn_sdot4((int)qhi[8 * j + w], (int)kb[8 * j + w], ahi, false);
            alo = __builtin_amdgcn_sdot4((int)qlo[8 * j + w], (int)kb[8 * j + w], alo, false);
          }
          s = __builtin_fmaf(ksf[j], (float)(ahi * 256 + alo), s);
        }
        x[h] = valid ? s * ck : -INFINITY;
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
#pragma unroll
      for (int q4 = 0; q4 < NPAIR; q4 += 4) {
        uint4 wq[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
          wq[h] = *reinterpret_cast<const uint4*>(&wlds[h][jv][slot * NPAIR + q4]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          h2_t c[8];
          r.v[2 * (q4 + u)].pairs(r.v[2 * (q4 + u) + 1], c);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const uint32_t wsel = u == 0 ? wq[h].x : u == 1 ? wq[h].y : u == 2 ? wq[h].z : wq[h].w;
            const h2_t wp = as_h2(wsel);
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
  }

  // ------------------------------------------------ bf16 tail positions
  const int ta = max(p0, nq), tb = p1;
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
