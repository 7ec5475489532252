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
// softmax spread over few rows.  Here a workgroup owns 128 rows of one KV
// head (four waves of 32) and walks 64-position tiles:
//  * the tile is dequantized once into LDS: K' = code * scale * 2^fk(p) as
//    fp16 hi + lo parts (fk per position keeps |K'| < 2^15; the pair holds
//    the 19-bit product exactly), V' = code * scale * 2^fv likewise as hi +
//    lo, stored transposed (element-major), with fv one power of two per
//    workgroup that only decreases (the accumulators are rescaled exactly
//    when it does);
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
// lo.  The partials (running maximum in log2 units, sum, unnormalized output
// in rotated space) are the split kernel's, merged by the same combine.
#include "common.hpp"
#include "kernels.hpp"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int PD = 128;                 // head_dim
constexpr int PR = kPrefillRows;        // rows per workgroup, 32 per wave
constexpr int KROW = PD + 8;            // halves per LDS row of K' (272 bytes)
constexpr int VROW = kTile + 4;         // halves per LDS row of V'^T (136 bytes: the
                                        // 8-byte operand reads of 32 lanes hit 64 banks)
constexpr int kNoScale = 1 << 20;       // "no nonzero value seen" for fk / fv
constexpr float kLog2eF = 1.44269504088896340736f;

__device__ inline int exponent_of(float x) {   // floor(log2(x)) for normal x > 0
  return (int)((__float_as_uint(x) >> 23) & 255u) - 127;
}
__device__ inline float pow2(int e) {          // 2^e, e clamped to [-100, 100]
  e = e < -100 ? -100 : (e > 100 ? 100 : e);
  return __uint_as_float((uint32_t)(e + 127) << 23);
}
__device__ inline float fp16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// ---------------------------------------------------------------- queries
// One row per four lanes (32 elements each), 64 rows per block.
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
  for (int e = 0; e < 32; e += 2) {
    const float y0 = x[e] * sc, y1 = x[e + 1] * sc;
    const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1;
    const _Float16 l0 = (_Float16)(y0 - (float)h0), l1 = (_Float16)(y1 - (float)h1);
    hw[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    lw[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
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
// What one thread reads from the quantized planes for one tile: the codes
// of one 32-element K block of position tid / 4 (and its high bits at 5 or
// 6 bits), that block's K and V scales, and four V items.  Loaded one tile
// ahead, during the previous tile's products.
struct TileRaw {
  uint4 k0, k1;        // K code chunks (k1: 8-bit codes only)
  uint2 khb;           // K high-bit words (5- and 6-bit codes)
  uint32_t scales;     // K scale | V scale << 16 (fp16 bits)
  uint2 v[4];          // V items: the 4-bit word and the high bits, or 8 bytes
};

template <int KB, int VB>
__device__ inline void load_raw(const PrefillArgs& a, size_t slot, int t, int nq, TileRaw& r) {
  constexpr int RP = padded_row_bytes(PD, KB);
  const int tid = threadIdx.x, pl = tid >> 2, j = tid & 3;
  r.k0 = r.k1 = make_uint4(0u, 0u, 0u, 0u);
  r.khb = make_uint2(0u, 0u);
  r.scales = 0u;
  if (t * kTile + pl < nq) {
    const uint8_t* kt = a.k_codes + slot * kTile * RP;
    if constexpr (KB == 8) {
      r.k0 = *reinterpret_cast<const uint4*>(kt + chunk_offset(pl, 2 * j, RP));
      r.k1 = *reinterpret_cast<const uint4*>(kt + chunk_offset(pl, 2 * j + 1, RP));
    } else {
      r.k0 = *reinterpret_cast<const uint4*>(kt + chunk_offset(pl, j, RP));
      if constexpr (KB == 5) {
        const int byte = PD / 2 + 4 * j;
        r.khb.x = *reinterpret_cast<const uint32_t*>(kt + chunk_offset(pl, byte / kChunk, RP) + byte % kChunk);
      }
      if constexpr (KB == 6) {
        const int byte = PD / 2 + 8 * j;
        r.khb = *reinterpret_cast<const uint2*>(kt + chunk_offset(pl, byte / kChunk, RP) + byte % kChunk);
      }
    }
    const size_t si = (slot * kTile + pl) * 4 + j;
    r.scales = (uint32_t)a.k_scales[si] | ((uint32_t)a.v_scales[si] << 16);
  }
  const uint8_t* vtile = a.v_codes + slot * (size_t)v_tile_bytes(PD, VB);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int item = tid + 256 * k;
    const int R = item >> 3;
    const int t0p = 32 * (R >> 6) + 8 * ((R >> 4) & 3);
    r.v[k] = make_uint2(0u, 0u);
    if (t * kTile + t0p < nq) {
      if constexpr (VB == 8) {
        r.v[k] = reinterpret_cast<const uint2*>(vtile)[item];
      } else {
        r.v[k].x = reinterpret_cast<const uint32_t*>(vtile)[item];
        if constexpr (VB == 5) r.v[k].y = vtile[32 * PD + item];
        if constexpr (VB == 6) r.v[k].y = reinterpret_cast<const uint16_t*>(vtile + 32 * PD)[item];
      }
    }
  }
}

// Signed K codes of the thread's block from its raw words (the row layout
// of load_codes).
template <int KB>
__device__ inline void decode_k(const TileRaw& r, int (&c)[32]) {
  if constexpr (KB == 8) {
    const uint32_t w[8] = {r.k0.x, r.k0.y, r.k0.z, r.k0.w, r.k1.x, r.k1.y, r.k1.z, r.k1.w};
#pragma unroll
    for (int e = 0; e < 32; ++e) c[e] = (int)(int8_t)((w[e / 4] >> (8 * (e % 4))) & 0xFF);
  } else {
    constexpr int OFF = 1 << (KB - 1);
    const uint32_t w[4] = {r.k0.x, r.k0.y, r.k0.z, r.k0.w};
    const uint32_t hw2[2] = {r.khb.x, r.khb.y};
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      int u = (int)((w[e / 8] >> (4 * (e % 8))) & 15);
      if constexpr (KB == 5) u |= (int)((hw2[0] >> hibit_pos(e)) & 1) << 4;
      if constexpr (KB == 6) u |= (int)((hw2[e / 16] >> hi2_pos(e)) & 3) << 4;
      c[e] = u - OFF;
    }
  }
}

// Offset codes of the eight slots of a V item from its raw words.
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

// fp16 hi and lo parts of 2n floats as packed words: hi is y rounded
// toward zero (two per instruction), so y - hi has at most the 8-9
// significant bits a 19-bit value leaves and lo holds it exactly (inputs
// here have at most 19 significant bits and |y| < 2^15).
typedef __fp16 half2v __attribute__((ext_vector_type(2)));
template <int N>
__device__ inline void split_pairs(const float* y, uint32_t (&hw)[N], uint32_t (&lw)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const half2v hh = __builtin_amdgcn_cvt_pkrtz(y[2 * i], y[2 * i + 1]);
    const half2v ll = __builtin_amdgcn_cvt_pkrtz(y[2 * i] - (float)hh[0], y[2 * i + 1] - (float)hh[1]);
    hw[i] = __builtin_bit_cast(uint32_t, hh);
    lw[i] = __builtin_bit_cast(uint32_t, ll);
  }
}

template <int KB, int VB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_mfma_kernel(PrefillArgs a) {
  __shared__ __align__(16) _Float16 khi[kTile * KROW];
  __shared__ __align__(16) _Float16 klo[kTile * KROW];
  __shared__ __align__(16) _Float16 vth[PD * VROW];
  __shared__ __align__(16) _Float16 vtl[PD * VROW];
  __shared__ __align__(16) float ku[kTile];        // 2^-fk of each position
  __shared__ float vsr[kTile * 4];                 // V scales (position, block)
  __shared__ int red[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int split = blockIdx.x;
  const int g = blockIdx.y % a.Hkv, rb = blockIdx.y / a.Hkv;
  const int b = blockIdx.z;
  const int len = a.len[b];
  const int nrows = a.n_q * a.G;
  const int T = a.T;
  const int nq = len - (T > 0 ? min(len, T) : 0);   // quantized positions [0, nq)
  const size_t unit = (size_t)b * a.Hkv + g;

  // this lane's row (column n of the products) and its last visible position
  const int row = rb * PR + wave * 32 + n;
  const bool row_ok = row < nrows;
  const int lim = row_ok ? len - a.n_q + row / a.G : -1;
  // tiles holding a position some row of the block sees, split S ways
  const int last_row = min(rb * PR + PR, nrows) - 1;
  const int blim = len - a.n_q + last_row / a.G;
  const int ntiles = blim / kTile + 1;
  const int per = (ntiles + a.S - 1) / a.S;
  const int t_begin = split * per, t_end = min(ntiles, t_begin + per);

  // query operands: B[k][n] = Q'[row n][16 ks + 8 h + slot]
  half8 qh[8], ql[8];
  const size_t qrow = (unit * a.rows_pad + row) * PD;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qh[ks] = *reinterpret_cast<const half8*>(a.q_hi + qrow + 16 * ks + 8 * h);
    ql[ks] = *reinterpret_cast<const half8*>(a.q_lo + qrow + 16 * ks + 8 * h);
  }
  const float w = a.q_w[unit * a.rows_pad + row];

  float m = -1e30f, l = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int me = 0; me < 4; ++me)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[me][r] = 0.f;
  int fv_run = kNoScale;

  // V scales of tile t into vsr, and the wave's smallest V exponent
  // candidate into red: from the tile's raw words, after the previous
  // tile's products (its loads have arrived by then), so the two barriers
  // each tile has anyway publish them
  TileRaw raw;
  auto v_scales = [&](int t) {
    const int pl = tid >> 2, j = tid & 3;
    const int p = t * kTile + pl;
    int fvc = kNoScale;
    float vs = 0.f;
    if (p < nq) {
      vs = fp16_bits_to_f32((uint16_t)(raw.scales >> 16));
      if (vs > 0.f) fvc = 7 - exponent_of(vs);   // |c| < 2^7
    } else if (p < len) {
      const uint16_t* vr = a.v_tail + (unit * T + p % T) * PD + 32 * j;
      float vm = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) vm = fmaxf(vm, fabsf(bf16_to_f32(vr[e])));
      if (vm > 0.f) fvc = 14 - exponent_of(vm);
    }
    vsr[pl * 4 + j] = vs;
#pragma unroll
    for (int mk = 1; mk < 64; mk <<= 1) fvc = min(fvc, __shfl_xor(fvc, mk));
    if (lane == 0) red[wave] = fvc;
  };
  if (t_begin < t_end) {
    load_raw<KB, VB>(a, tile_slot_read(a.map, b, g, t_begin), t_begin, nq, raw);
    v_scales(t_begin);
  }
  __syncthreads();
  for (int t = t_begin; t < t_end; ++t) {
    const int fv_tile = min(min(red[0], red[1]), min(red[2], red[3]));
    const int fv_new = min(fv_run, fv_tile);
    if (fv_run != kNoScale && fv_new < fv_run) {
      const float f = pow2(fv_new - fv_run);   // exact power of two
#pragma unroll
      for (int me = 0; me < 4; ++me) o[me] *= f;
    }
    fv_run = fv_new;
    const float vmul = pow2(fv_run == kNoScale ? 0 : fv_run);
    // ---- stage K' (hi, lo); each thread one 32-element block of one
    // position
    {
      const int pl = tid >> 2, j = tid & 3;
      const int p = t * kTile + pl;
      int fkc = kNoScale;
      float x[32];
      if (p < nq) {
        int c[32];
        decode_k<KB>(raw, c);
        const float s = fp16_bits_to_f32((uint16_t)(raw.scales & 0xFFFFu));
        if (s > 0.f) fkc = 7 - exponent_of(s);   // |c| < 2^7: |x| < 2^(e+8)
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = (float)c[e] * s;
      } else if (p < len) {
        const uint16_t* kr = a.k_tail + (unit * T + p % T) * PD + 32 * j;
        float km = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          x[e] = bf16_to_f32(kr[e]);
          km = fmaxf(km, fabsf(x[e]));
        }
        if (km > 0.f) fkc = 14 - exponent_of(km);
      } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = 0.f;
      }
      // one fk per position: the smallest of its four blocks' candidates
      fkc = min(fkc, __shfl_xor(fkc, 1));
      fkc = min(fkc, __shfl_xor(fkc, 2));
      const int fk = fkc == kNoScale ? 0 : fkc;
      const float sc = pow2(fk);
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] *= sc;
#pragma unroll
      for (int q = 0; q < 2; ++q) {   // 16 elements at a time
        uint32_t hw[8], lw[8];
        split_pairs<8>(x + 16 * q, hw, lw);
        uint4* dh = reinterpret_cast<uint4*>(khi + pl * KROW + 32 * j + 16 * q);
        uint4* dl = reinterpret_cast<uint4*>(klo + pl * KROW + 32 * j + 16 * q);
        dh[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        dh[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        dl[0] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        dl[1] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
      }
      if (j == 0) ku[pl] = pow2(-fk);
    }
    // ---- stage V'^T (hi, lo): each thread four items (eight positions of
    // one element)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int item = tid + 256 * k;
      const int R = item >> 3;                 // item = R * (D/16) + e/16
      const int e = 16 * (item & 7) + (R & 15);
      const int t0p = 32 * (R >> 6) + 8 * ((R >> 4) & 3);
      const int p0 = t * kTile + t0p;
      constexpr int OFF = 1 << (VB - 1);
      int u[8];
      decode_v<VB>(raw.v[k], u);
      float v[8];
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) v[s2] = (float)(u[s2] - OFF) * (vsr[(t0p + s2) * 4 + (e >> 5)] * vmul);
      if (p0 + 7 >= nq) {   // the same for a wave: its items share t0p
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const int p = p0 + s2;
          if (p >= nq) v[s2] = p < len ? bf16_to_f32(a.v_tail[(unit * T + p % T) * PD + e]) * vmul : 0.f;
        }
      }
      uint32_t hw[4], lw[4];
      split_pairs<4>(v, hw, lw);
      uint2* dh = reinterpret_cast<uint2*>(vth + e * VROW + t0p);
      uint2* dl = reinterpret_cast<uint2*>(vtl + e * VROW + t0p);
      dh[0] = make_uint2(hw[0], hw[1]);
      dh[1] = make_uint2(hw[2], hw[3]);
      dl[0] = make_uint2(lw[0], lw[1]);
      dl[1] = make_uint2(lw[2], lw[3]);
    }
    __syncthreads();
    // the next tile's codes, in flight during this tile's products
    if (t + 1 < t_end) load_raw<KB, VB>(a, tile_slot_read(a.map, b, g, t + 1), t + 1, nq, raw);

    // ---- per 32 positions: S^T = K' Q'^T (M = positions, N = rows), the
    // online softmax of row n, then O^T += V'^T P^T
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 0.f;
      const _Float16* kh = khi + (32 * mt + n) * KROW + 8 * h;
      const _Float16* kl = klo + (32 * mt + n) * KROW + 8 * h;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const half8 ah = *reinterpret_cast<const half8*>(kh + 16 * ks);
        const half8 al = *reinterpret_cast<const half8*>(kl + 16 * ks);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, qh[ks], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, qh[ks], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, ql[ks], sc, 0, 0, 0);
      }
      float tmax = -INFINITY;
      // causal masking only where some row of the wave stops inside these
      // 32 positions
      const bool masked = __any(t * kTile + 32 * mt + 31 > lim);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pos = 32 * mt + 8 * q + 4 * h;     // accumulator rows 4q..4q+3
        const float4 u4 = *reinterpret_cast<const float4*>(ku + pos);
        const float uu[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = sc[4 * q + r] * uu[r];
          if (masked) v = t * kTile + pos + r <= lim ? v : -INFINITY;
          sc[4 * q + r] = v;
          tmax = fmaxf(tmax, v);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mn = fmaxf(m, w * tmax);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);   // arguments <= 0
      float ps = 0.f;
      half8 pbh[2], pbl[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(sc[r], w, -mn));
        const _Float16 ph = (_Float16)pe;
        ps += pe;
        pbh[r / 8][r % 8] = ph;
        pbl[r / 8][r % 8] = (_Float16)(pe - (float)ph);
      }
      l = l * alpha + ps;
      m = mn;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int me = 0; me < 4; ++me) o[me] *= alpha;
      }
      // K order of slot j of half h: 16 s' + 8 (j/4) + 4 h + j%4, the
      // accumulator rows of the scores
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
          o[me] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, pbh[sp], o[me], 0, 0, 0);
          o[me] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, pbh[sp], o[me], 0, 0, 0);
          o[me] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, pbl[sp], o[me], 0, 0, 0);
        }
      }
    }
    if (t + 1 < t_end) v_scales(t + 1);
    __syncthreads();   // every wave has read this tile's LDS and red; vsr, red are the next tile's
  }

  // ---- partials: row (b, i, g*G + h') in the [B][n_q][Hq] order of the output
  l += __shfl_xor(l, 32);
  if (!row_ok) return;
  const size_t rv = ((size_t)b * a.n_q + row / a.G) * a.Hq + (size_t)g * a.G + row % a.G;
  if (h == 0) {
    a.part_ml[(rv * a.S + split) * 2] = m;
    a.part_ml[(rv * a.S + split) * 2 + 1] = l;
  }
  const float un = pow2(fv_run == kNoScale ? 0 : -fv_run);
  float* dst = a.part_acc + (rv * a.S + split) * PD;
#pragma unroll
  for (int me = 0; me < 4; ++me)
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[32 * me + 8 * (r / 4) + 4 * h + r % 4] = o[me][r] * un;
}

}  // namespace

hipError_t launch_prefill_q(const PrefillArgs& a, int B, hipStream_t s) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  hipLaunchKernelGGL(prefill_q_kernel, dim3(a.rows_pad / 64, a.Hkv, B), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KB>
void launch_prefill_v(const PrefillArgs& a, int vb, dim3 grid, hipStream_t s) {
  switch (vb) {
    case 4: hipLaunchKernelGGL((prefill_mfma_kernel<KB, 4>), grid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL((prefill_mfma_kernel<KB, 5>), grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL((prefill_mfma_kernel<KB, 6>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((prefill_mfma_kernel<KB, 8>), grid, dim3(256), 0, s, a); break;
  }
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, int kb, int vb, int B, hipStream_t s) {
  (void)hipGetLastError();
  const dim3 grid(a.S, a.n_rb * a.Hkv, B);
  switch (kb) {
    case 4: launch_prefill_v<4>(a, vb, grid, s); break;
    case 5: launch_prefill_v<5>(a, vb, grid, s); break;
    case 6: launch_prefill_v<6>(a, vb, grid, s); break;
    default: launch_prefill_v<8>(a, vb, grid, s); break;
  }
  return hipGetLastError();
}

}  // namespace kvq
