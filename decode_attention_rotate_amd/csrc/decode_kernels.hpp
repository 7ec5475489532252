// Split-K single-query decode attention over the rotated block-quantized cache.
//
// Method (velog.io post "fix KV cache quantization outliers", section
// "Hadamard rotation"): scores are dot products of the rotated query with the
// rotated keys (the rotation is orthogonal, so they equal the unrotated
// scores), softmax, weighted sum of the rotated values; the combine kernel
// rotates the result back.  Newest tokens may sit unquantized in a bf16 tail
// (aitrends.kr article 92204, glossary "Precision Tail").
//
// Work unit: one (sequence b, KV head g, chunk of G <= 8 query heads); S
// waves share a unit and stream each of its cache bytes once.  Workgroups of
// 8 waves at d <= 128 (2 per SIMD), 4 at d = 256 (1 per SIMD, for registers),
// one per compute unit, take contiguous ranges
// of the unit's quantized tiles, and inside a workgroup each wave takes the
// next tile from an LDS counter, so waves the compute unit happens to serve
// less do less of the work.  Each wave keeps one online-softmax state in its
// own LDS rows and registers and writes one partial.  The
// G query heads share each K/V row, so both contractions of a step of 32
// tokens run on the matrix cores (16x16x32 MFMA; lane l owns A row l%16 and
// B column l%16, k-slots 8*(l/16)..+7, and output rows 4*(l/16)..+3):
//  * Q.K, v_mfma_i32_16x16x32_i8 per 16 tokens and 32-element block.  A rows
//    are the query of each head in 16-bit fixed point, split into a high-byte
//    row and a low-byte row; B columns are the int8 codes of 16 tokens, read
//    straight from the row layout (4/5-bit codes widened to bytes, their
//    offset folded in per block).  A lane gets the high and low sums of two
//    heads for one token, combines them exactly in int32 and applies the
//    token's fp16 block scale:
//      score += scale_k * float(256 * sum(q_hi * c) + sum(q_lo * c))
//  * Online softmax in log2 units, rescaling only when a running max grows.
//  * P.V, v_mfma_f32_16x16x32_f16 per 32 tokens and 16 output elements.  A
//    rows are the weights p * scale_v * 2^e of each head (rounded once to
//    fp16, moved from score layout to operand layout through LDS; 2^e keeps
//    the largest V scale near 2^11, so weights stay in fp16's normal range
//    for V of any size, and the accumulators are divided by it at the end);
//    B columns are
//    V codes of one element for 8 consecutive tokens, which the element-major
//    V tiles store together: nibbles / bytes become exact fp16 integers with
//    one v_and_or (or v_perm) per pair plus one packed fp16 add.
// bf16 tail tokens run the same steps on bf16 matrix products, with the
// float32 query and weights split into high and low bf16 parts, and share
// the online-softmax state of the quantized tokens.
// Scale-and-min blocks (x = u * s + m, levels u >= 0): Q.K takes the levels
// without an offset and adds m * sum(q) of the block, from per-block query
// sums made once; P.V takes the centred levels u - 2^(b-1) and each lane
// keeps sum(p * (m + 2^(b-1) * s)) per (head, block) beside the
// accumulators, rescaled with them, added to the output elements of that
// block at the end.
#pragma once

#include "append_one.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace kvq {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int i4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kStep = 32;   // tokens per step of the quantized loop

__device__ inline h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

// Orders this wave's LDS accesses around a point (each wave of the split
// kernel owns its LDS rows; no other wave waits).
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ inline uint32_t as_u32(h2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Larger of two scores; no NaN handling (scores are finite or -inf).
__device__ inline float fmax_fast(float a, float b) { return a > b ? a : b; }

// Rotation by N lanes inside each row of 16 lanes (DPP row_ror).
template <int N>
__device__ inline float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}
__device__ inline float row16_max(float v) {
  v = fmax_fast(v, row_ror<8>(v));
  v = fmax_fast(v, row_ror<4>(v));
  v = fmax_fast(v, row_ror<2>(v));
  return fmax_fast(v, row_ror<1>(v));
}
__device__ inline float row16_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  return v + row_ror<1>(v);
}

__device__ inline uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) { return (x & mask) | bits; }
__device__ inline uint32_t rotr(uint32_t x, uint32_t s) { return __builtin_amdgcn_alignbit(x, x, s); }
__device__ inline float half_of(uint32_t w, int hi) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(hi ? (w >> 16) : (w & 0xFFFFu)));
}
// In lanes 0..31, x of lane + 32 (one lane swap between the wave's halves;
// lanes 32..63 get their own x back)
__device__ inline float upper_half(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[1]);
}

// Cache bytes of one 32-token step held in registers.  KM / VM: K / V use
// scale-and-min blocks, whose scale planes hold an (s, m) fp16 pair per block.
template <int D, int KB, int VB, bool KM, bool VM, bool OUT = false>
struct StepRegs {
  static constexpr int NB = D / kBlock;
  static constexpr int NN = D / 16;
  static constexpr int NSW = (NB + 1) / 2;   // 32-bit words of fp16 scales per token
  static constexpr int KSW = KM ? NB : NSW;  // ... of K scales (pairs: one word a block)
  static constexpr int VSW = VM ? NB : NSW;
  u32x2 k8[KB == 8 ? 2 * NB : 1];            // [m][blk] 8 code bytes
  uint32_t k4[KB == 8 ? 1 : 2 * NB];         // [m][blk] 8 code nibbles
  uint32_t kh[KB == 5 || KB == 6 ? 2 * NB : 1];   // [m][blk] 5/6-bit high-bit word
  uint32_t ks[2][KSW], vs[2][VSW];           // [m] fp16 scales (pairs) of this lane's token
  u32x4 v[VB == 8 ? NN / 2 : NN / 4];        // V items (4 or 8 bytes each)
  uint32_t vh[VB == 5 ? NN / 4 : VB == 6 ? NN / 2 : 1];   // 5-bit bytes / 6-bit fields
  // outlier channels: K codes (bytes 8r..8r+7 of the lane's tokens), the
  // tokens' K and V outlier scales, the lane's two 8-bit V items
  u32x2 ko[OUT ? 2 : 1];
  uint32_t kos[OUT ? 2 : 1], vos[OUT ? 2 : 1];
  u32x4 vo;

  // scale of block j of token-row half m, and the minimum of a pair block
  __device__ float k_scale(int m, int j) const { return KM ? half_of(ks[m][j], 0) : half_of(ks[m][j / 2], j % 2); }
  __device__ float v_scale(int m, int j) const { return VM ? half_of(vs[m][j], 0) : half_of(vs[m][j / 2], j % 2); }
  __device__ float k_min(int m, int j) const { return half_of(ks[m][j], 1); }
  __device__ float v_min(int m, int j) const { return half_of(vs[m][j], 1); }
};

// Largest fp16 V scale (as its bit pattern; scales are >= 0, so bit patterns
// order like the values) of token-row half m of this lane.  Scale-and-min
// words hold (s, m) pairs with s in the low half.
template <int D, int KB, int VB, bool KM, bool VM, bool OUT>
__device__ inline uint32_t v_scale_max_bits(const StepRegs<D, KB, VB, KM, VM, OUT>& R, int m) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  constexpr int VSW = StepRegs<D, KB, VB, KM, VM, OUT>::VSW;
  u16x2 x = __builtin_bit_cast(u16x2, R.vs[m][0]);
#pragma unroll
  for (int w = 1; w < VSW; ++w) x = __builtin_elementwise_max(x, __builtin_bit_cast(u16x2, R.vs[m][w]));
  return VM ? (uint32_t)x[0] : (uint32_t)(x[0] > x[1] ? x[0] : x[1]);
}

// Loads of cache bytes.  Each byte is read once per call; with NT the loads
// are non-temporal (the hint lets the caches stream them past), which the
// part serves about a tenth faster than ordinary loads for this access
// pattern at two waves per SIMD (read-ceiling probes and the 64k decode
// kernel), but which made the one-wave-per-SIMD head_dim 256 kernel 2%
// slower, so those keep ordinary loads.
template <bool NT, typename T>
__device__ inline T ld_cache(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else return *reinterpret_cast<const T*>(p);
}

// Load NW consecutive 32-bit words with the widest loads their alignment
// allows: NW * 4 bytes per token, so 8-byte loads for even NW, 16-byte ones
// for multiples of 4 (head_dim 192 has NW = 3 or 6).
template <bool NT, int NW>
__device__ inline void load_words(const uint32_t* p, uint32_t (&w)[NW]) {
  if constexpr (NW % 4 != 0 && NW % 2 != 0) {
#pragma unroll
    for (int q = 0; q < NW; ++q) w[q] = ld_cache<NT, uint32_t>(p + q);
  } else if constexpr (NW % 4 != 0) {
#pragma unroll
    for (int q = 0; q < NW / 2; ++q) {
      const u32x2 x = ld_cache<NT, u32x2>(p + 2 * q);
      w[2 * q] = x[0]; w[2 * q + 1] = x[1];
    }
  } else {
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      const u32x4 x = ld_cache<NT, u32x4>(p + 4 * q);
#pragma unroll
      for (int k = 0; k < 4; ++k) w[4 * q + k] = x[k];
    }
  }
}

// B operand of Q.K for 16 tokens and one block: 8 int8 codes of this lane's
// token in the k-slot order of the query bytes (4/5/6-bit: elements
// 0,2,4,6,1,3,5,7 of the lane's group of 8, widened to bytes; the high bits
// come from one rotate of the block's high word).
template <int D, int KB, int VB, bool KM, bool VM, bool OUT>
__device__ inline long k_operand(const StepRegs<D, KB, VB, KM, VM, OUT>& R, int i, uint32_t rot_lo, uint32_t rot_hi) {
  if constexpr (KB == 8) {
    return __builtin_bit_cast(long, R.k8[i]);
  } else {
    const uint32_t x = R.k4[i];
    uint32_t lo = x & 0x0F0F0F0Fu;
    uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;
    if constexpr (KB == 5) {
      lo |= rotr(R.kh[i], rot_lo) & 0x10101010u;
      hi |= rotr(R.kh[i], rot_hi) & 0x10101010u;
    }
    if constexpr (KB == 6) {
      lo |= rotr(R.kh[i], rot_lo) & 0x30303030u;
      hi |= rotr(R.kh[i], rot_hi) & 0x30303030u;
    }
    return (long)(((uint64_t)hi << 32) | lo);
  }
}

// B operand of P.V for output elements 16*nb..+15: this lane's element for
// the 8 tokens of its k-slots, as exact fp16 codes (centred levels
// u - 2^(VB-1) for scale-and-min blocks).
// B operand of P.V from an 8-bit V item pair (items nb = 0, 1 of a u32x4):
// the 8 offset codes u of item nb as exact fp16 values u - 128.
__device__ inline h8_t v_operand8(const u32x4 q, int nb) {
  const uint32_t x0 = nb ? q[2] : q[0];
  const uint32_t x1 = nb ? q[3] : q[1];
  const uint32_t c64 = 0x64646464u;
  const h2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const h2_t d0 = as_h2(__builtin_amdgcn_perm(c64, x0, 0x04010400u)) + bias;
  const h2_t d1 = as_h2(__builtin_amdgcn_perm(c64, x0, 0x04030402u)) + bias;
  const h2_t d2 = as_h2(__builtin_amdgcn_perm(c64, x1, 0x04010400u)) + bias;
  const h2_t d3 = as_h2(__builtin_amdgcn_perm(c64, x1, 0x04030402u)) + bias;
  return h8_t{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
}

template <int D, int KB, int VB, bool KM, bool VM, bool OUT>
__device__ inline h8_t v_operand(const StepRegs<D, KB, VB, KM, VM, OUT>& R, int nb, uint32_t magic) {
  const h2_t one16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  if constexpr (VB == 8) {
    const u32x4 q = R.v[nb / 2];
    const uint32_t x0 = (nb % 2) ? q[2] : q[0];
    const uint32_t x1 = (nb % 2) ? q[3] : q[1];
    const uint32_t c64 = 0x64646464u;
    const h2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const h2_t d0 = as_h2(__builtin_amdgcn_perm(c64, x0, 0x04010400u)) + bias;
    const h2_t d1 = as_h2(__builtin_amdgcn_perm(c64, x0, 0x04030402u)) + bias;
    const h2_t d2 = as_h2(__builtin_amdgcn_perm(c64, x1, 0x04010400u)) + bias;
    const h2_t d3 = as_h2(__builtin_amdgcn_perm(c64, x1, 0x04030402u)) + bias;
    return h8_t{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
  } else {
    const uint32_t x = R.v[nb / 4][nb % 4];
    const uint32_t x8 = x >> 8;
    uint32_t w0 = and_or(x, 0x000F000Fu, magic);
    uint32_t w1 = and_or(x, 0x00F000F0u, magic);
    uint32_t w2 = and_or(x8, 0x000F000Fu, magic);
    uint32_t w3 = and_or(x8, 0x00F000F0u, magic);
    _Float16 b_lo, b_hi;
    if constexpr (VB == 6) {
      // slot fields 2n, 2n+1 of nibble position n go to bits 4-5 (low-nibble
      // halves, value 16 h) or 8-9 (high-nibble halves, value 256 h)
      const uint32_t h = (R.vh[nb / 2] >> (16 * (nb % 2))) & 0xFFFFu;
      const uint32_t y = (h << 4) | (h << 12);
      w0 |= y & 0x00300030u;
      w1 |= (y << 2) & 0x03000300u;
      w2 |= (y >> 4) & 0x00300030u;
      w3 |= (y >> 2) & 0x03000300u;
      b_lo = (_Float16)-1056.0f;
      b_hi = (_Float16)-96.0f;
    } else if constexpr (VB == 5) {
      const uint32_t hb = (R.vh[nb / 4] >> (8 * (nb % 4))) & 0xFFu;
      const uint32_t y = (hb << 4) | (hb << 16);
      w0 |= y & 0x00100010u;
      w1 |= (y << 3) & 0x01000100u;
      w2 |= (y >> 2) & 0x00100010u;
      w3 |= (y << 1) & 0x01000100u;
      b_lo = (_Float16)-1040.0f;
      b_hi = (_Float16)-80.0f;
    } else {
      b_lo = (_Float16)-1032.0f;
      b_hi = (_Float16)-72.0f;
    }
    const h2_t bl = {b_lo, b_lo}, bh = {b_hi, b_hi};
    const h2_t d0 = as_h2(w0) + bl;
    const h2_t d1 = __builtin_elementwise_fma(as_h2(w1), one16, bh);   // exact
    const h2_t d2 = as_h2(w2) + bl;
    const h2_t d3 = __builtin_elementwise_fma(as_h2(w3), one16, bh);
    return h8_t{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
  }
}

// PF = false: decode, one query per sequence; a wave's rows are the G <= 8
// query heads of one chunk of a KV head's group.
// PF = true: chunked prefill (G = 8): the rows of a KV head g are the pairs
// (query i, head h of g's group), numbered v = i * Gq + h, and the 8 waves of
// a workgroup own 8 consecutive rows each.  Row (i, h) sits at position
// n - n_q + i and sees positions up to there.  All waves of a workgroup walk
// the same tiles, so each cache byte comes from HBM once per workgroup (the
// other waves find it in L1 / L2).
// PGM: where tiles live.  kPageAny decides at run time between contiguous
// and paged planes; kPageFlat and kPagePaged fix it at compile time, for the
// variants whose register budget is too tight to carry both.
// OUT: outlier channels (32 per plane and KV head, 8-bit, original space;
// no tail): one more i8 product per 16 tokens adds q[O_K] . x_O to the
// scores, and two more f16 products accumulate the V outlier channels,
// which the combine adds at their channels.
template <int D, int KB, int VB, int G, bool PF, bool KM, bool VM, int PGM, bool OUT = false>
__global__ __launch_bounds__(64 * split_group_waves(D, KM || VM || PF))
__attribute__((amdgpu_waves_per_eu(split_waves_per_simd(D, KM || VM || PF),
                                   split_waves_per_simd(D, KM || VM || PF))))
void decode_split_kernel(DecodeArgs a) {
  static_assert(G >= 1 && G <= 8, "at most 8 query heads per wave");
  static_assert(!PF || G == 8, "prefill waves own 8 rows");
  constexpr int kGroupWaves = split_group_waves(D, KM || VM || PF);
  // non-temporal cache loads at two waves per SIMD (see ld_cache); not for
  // prefill, whose waves all read every tile of their workgroup's range and
  // find it in the caches after the first
  constexpr bool kNT = !PF && split_waves_per_simd(D, KM || VM || PF) >= 2;
  // tiles whose bytes a wave keeps in registers ahead of the one computing:
  // at one wave per SIMD (d = 256) the wave alone must cover the latency, so
  // it keeps two where four step buffers fit the 512 registers with at most
  // a few spilled (4-bit K, or 4-bit V with 5- or 8-bit K; decode only, a
  // prefill wave holds more state; contiguous planes only, a paged wave also
  // carries its page lookups and then spilled inside the loop).  The
  // one-wave d = 192 variants measured no faster with two.
  // The query as 24-bit fixed point (three bytes: two in the rows of the
  // Q.K product, the residual byte in a second product), in decode as in
  // prefill: with heavy-tailed data the scores grow large enough that the
  // 2^-16 relative step of a 16-bit query moved outputs by more than 1e-3
  // (measured up to 1.2e-3 on the GPU and 2.2e-3 in a CPU emulation at head
  // dims 64 to 256), against 1e-5 with 24 bits.  Its registers are those a
  // second tile ahead would take at one wave per SIMD.
  constexpr bool kQ24 = true;
  // Up to 4 heads per wave (decode) the hi / lo rows fill A rows 0..7 only,
  // and the residual bytes take the odd rows 8..15 of the same product
  // (kFold): no second product, and its registers free for a second tile.
  constexpr bool kFold = kQ24 && !PF && G <= 4;
  constexpr int kAhead =
      (!kQ24 || kFold) && split_waves_per_simd(D, KM || VM || PF) == 1 && D == 256 && !PF && !KM && !VM &&
              PGM != kPagePaged && (KB == 4 || (VB == 4 && KB != 6)) ? 2 : 1;
  constexpr int NB = D / kBlock;
  constexpr int NN = D / 16;
  constexpr int NSW = (NB + 1) / 2;
  constexpr int RKP = padded_row_bytes(D, KB);
  constexpr int VTB = v_tile_bytes(D, VB);
  // LDS weight rows of 32 tokens (+ pad), 16-bit: row 8*j + h holds head h's
  // weights for V block j; the tail keeps the low bf16 parts of its weights
  // in rows LOROW + h; row ZROW stays zero (A rows 8..15 of quantized steps
  // with absmax V).  Scale-and-min V, and prefill rows with either V
  // block kind (kLoW), keep the low fp16 parts of their weights in rows
  // LOQ + 8*j + h, as A rows 8..15 (see the weights below).
  constexpr bool kLoW = VM || PF;
  constexpr int WROW = 48;
  constexpr int LOROW = 8 * NB;
  constexpr int ZROW = 8 * NB + 8;
  constexpr int LOQ = 8 * NB + 9;
  constexpr int OROW = LOQ + (kLoW ? 8 * NB : 0);   // outlier weights of the 8 heads (OUT)
  using Regs = StepRegs<D, KB, VB, KM, VM, OUT>;
  static_assert(!OUT || (!PF && !KM && !VM), "outlier channels: decode with absmax blocks");

  __shared__ __align__(16) uint16_t wl_all[kGroupWaves][(8 * NB + 9 + (kLoW ? 8 * NB : 0) + (OUT ? 8 : 0)) * WROW];
  __shared__ __align__(16) float alds_all[kGroupWaves][16];
  __shared__ uint32_t tile_ctr;
  // fused step: new K, new V, quantized K, quantized V values; the two
  // positions' weights per head
  __shared__ __align__(16) float step_vals[PF ? 1 : 4 * D];
  __shared__ float step_w[2][8];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 15;
  const int r = lane >> 4;
  // this wave's partial slot
  const int split = PF ? (int)blockIdx.x : (int)blockIdx.x * kGroupWaves + wv;
  uint16_t* wl = wl_all[wv];
  float* alds = alds_all[wv];
  if (threadIdx.x == 0) tile_ctr = 0u;
  __syncthreads();
  const int g = PF ? (int)blockIdx.y / a.n_rb : (int)blockIdx.y / a.n_gchunks;
  const int h0 = g * a.G + (PF ? 0 : ((int)blockIdx.y % a.n_gchunks) * G);
  const int b = blockIdx.z;
  const int n = a.len[b];
  // rows of this wave (prefill): vbase .. vbase + 7 of the R rows of (b, g)
  const int R = PF ? a.n_q * a.G : G;
  const int vbase = PF ? (((int)blockIdx.y % a.n_rb) * kGroupWaves + wv) * 8 : 0;
  if (PF && vbase >= R) return;   // no barrier follows
  // row k of the wave: present?, index of its query / output vector among
  // the [B][n_q][Hq] (decode: [B][Hq]) ones, last position it sees
  auto row_ok = [&](int k) { return PF ? vbase + k < R : k < G; };
  auto row_vec = [&](int k) -> size_t {
    if constexpr (PF) {
      const int v = vbase + k, i = v / a.G;
      return ((size_t)b * a.n_q + i) * a.Hq + h0 + (v - i * a.G);
    } else {
      return (size_t)b * a.Hq + h0 + k;
    }
  };
  auto row_lim = [&](int k) { return PF ? n - a.n_q + (vbase + k) / a.G : n - 1; };
  // last position any row of the wave sees (rows are in position order)
  const int wlim = row_lim(min(7, R - 1 - vbase));
  const int T = a.T;
  const int nt = T > 0 ? min(n, T) : 0;
  const int nq = n - nt;
  // Fused decode step (decode only): this launch also appends the step's
  // token, so the positions the append changes, nq - 1 (the one that becomes
  // quantized, if any) and, with a tail, n - 1 (the new token), are attended
  // to from the values the append computes (below), not read from the
  // planes and the ring, which the append is writing meanwhile.
  const bool stp = !PF && a.step_on != 0;
  const int nqr = stp ? max(nq - 1, 0) : nq;   // quantized positions read from the planes
  const int ntr = stp && T > 0 ? n - 1 : n;    // tail positions [nq, ntr) read from the ring
  // Quantized tiles (decode): the unit's tiles are dealt round-robin to its
  // NG workgroups (tile t to workgroup t mod NG), and a workgroup's waves
  // pull its tiles, in order, one at a time from an LDS counter, so they
  // finish together however the compute unit schedules them.  At any time
  // the workgroups of a unit read neighbouring tiles: a compact window of
  // addresses, which HBM serves faster than far-apart ranges (read-ceiling
  // probes; dealing chunks of one tile measured a little faster than chunks
  // of a workgroup's size, and balances to one tile).  Prefill: workgroup
  // wg takes the contiguous range [ctq*wg/NG, ctq*(wg+1)/NG) and every wave
  // takes every tile of it, up to its rows' last position.  bf16 tail tiles
  // (few, each worth several quantized tiles) are dealt out round-robin:
  // tile k to workgroup k mod NG, wave (k / NG) mod kGroupWaves (prefill: to
  // every wave of workgroup k mod NG).
  const int ctq = (nqr + kTile - 1) / kTile;
  const int ctt = (ntr - nq + kTile - 1) / kTile;
  const int NG = (int)gridDim.x;
  const int wq0 = (int)((int64_t)ctq * blockIdx.x / NG), wq1 = (int)((int64_t)ctq * (blockIdx.x + 1) / NG);
  const int qend = PF ? wq1 : ctq;   // a grabbed tile at or past this ends the loop
  const size_t unit = (size_t)b * a.Hkv + g;

  for (int i = lane; i < WROW; i += 64) wl[ZROW * WROW + i] = 0;
  if (lane < 16) alds[lane] = 1.f;

  // this lane's score heads (Q.K output rows 4r..4r+3 = hi/lo of hA, hB)
  const int hA = 2 * r, hB = 2 * r + 1;
  const bool okA = row_ok(hA), okB = row_ok(hB);
  const int limA = row_lim(hA), limB = row_lim(hB);
  // running maxima start at -1e30 for present heads (a finite floor: a
  // prefill row may see no token of a whole split) and at 0 for absent ones,
  // so every masked score, whose value is -inf, gets weight exp2(-inf - m) = 0
  float mA = okA ? -1e30f : 0.f, mB = okB ? -1e30f : 0.f, lA = 0.f, lB = 0.f;
  f4_t acc[NN];
#pragma unroll
  for (int i = 0; i < NN; ++i) acc[i] = f4_t{0.f, 0.f, 0.f, 0.f};
  // V minima: this lane's share of sum(p * m) of heads hA, hB per V block
  float mvA[VM ? NB : 1], mvB[VM ? NB : 1];
#pragma unroll
  for (int j = 0; j < (VM ? NB : 1); ++j) mvA[j] = mvB[j] = 0.f;
  // V outlier channels: slots 16 nb + col of the heads' rows (OUT)
  f4_t acco[OUT ? 2 : 1];
#pragma unroll
  for (int i = 0; i < (OUT ? 2 : 1); ++i) acco[i] = f4_t{0.f, 0.f, 0.f, 0.f};
  // Weight factor of the quantized positions: their fp16 weights are
  // p * scale_v * 2^vfe, with 2^(11 - vfe) <= the largest V scale seen so far
  // < 2^(12 - vfe), so a weight never drops into fp16's subnormal range
  // however small V is (the result is the same for V and for V times a power
  // of two).  The accumulators carry the factor; a scale at or above vthr
  // (fp16 bits of 2^(15 - vfe)) raises it, and the accumulators are divided
  // by it at the end.  Powers of two: every rescale is exact.
  int vfe = 0;
  uint32_t vthr = 0u;   // the first step with a nonzero scale sets the factor

  // Query of this lane's A row in registers: row col < 2G is the wave's row
  // col/2; the lane holds elements 32j + 8r + i (j < NB, i < 8), rotated in
  // float32 with the butterfly stages in the order h = 1, 2, 4, ..., D/2
  // (h = 8, 16 exchange values with lanes 16 and 32 apart).  Lanes of absent
  // rows read row 0.
  auto load_query = [&](float (&f)[NB][8]) {
    const int qr = kFold && col >= 8 ? col - 8 : col;
    const int hq = qr < 2 * G && row_ok(qr / 2) ? qr / 2 : 0;
    const size_t off = row_vec(hq) * D + 8 * r;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (a.q_dtype == KVQ_BF16) {
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + off + kBlock * j);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f[j][2 * k] = __uint_as_float(w4[k] << 16);
          f[j][2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
        }
      } else {
        const float4* v = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + off + kBlock * j);
        const float4 x0 = v[0], x1 = v[1];
        f[j][0] = x0.x; f[j][1] = x0.y; f[j][2] = x0.z; f[j][3] = x0.w;
        f[j][4] = x1.x; f[j][5] = x1.y; f[j][6] = x1.z; f[j][7] = x1.w;
      }
    }
    if (!a.rotate_k) return;
    if (a.has_signs) {   // H diag(s): element 32j + 8r + i flips with bit 8r + i of word j
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const uint32_t m = a.signs[j] >> (8 * r);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          f[j][i] = __uint_as_float(__float_as_uint(f[j][i]) ^ ((m << (31 - i)) & 0x80000000u));
      }
    }
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if ((i & h) == 0) {
            const float u = f[j][i], v = f[j][i + h];
            f[j][i] = u + v;
            f[j][i + h] = u - v;
          }
        }
      }
    }
#pragma unroll
    for (int sh = 16; sh <= 32; sh <<= 1) {
      const uint32_t flip = (lane & sh) ? 0x80000000u : 0u;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float y = __shfl_xor(f[j][i], sh);
          f[j][i] = y + __uint_as_float(__float_as_uint(f[j][i]) ^ flip);
        }
      }
    }
    // stages across blocks, up to the rotation's block size (head_dim 192:
    // H_64 blocks, only the pairs j, j + 1)
#pragma unroll
    for (int h = 1; h < rot_block(D) / kBlock; h <<= 1) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if ((j & h) == 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float u = f[j][i], v = f[j + h][i];
            f[j][i] = u + v;
            f[j + h][i] = u - v;
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[j][i] = f[j][i] * a.cd;
    }
  };

  // Online softmax over this lane's scores (log2 units, -inf when masked).
  // The running maxima only move, and the accumulators are only rescaled,
  // when some score exceeds them (a wave-uniform branch); every weight stays
  // at most 1.
  // vtrig (wave-uniform): the accumulators also take the factor vratio, the
  // change of the V weight factor (one rescaling site for both).
  auto softmax = [&](const float (&xA)[2], const float (&xB)[2], float (&pA)[2], float (&pB)[2],
                     bool vtrig, float vratio) {
    const bool up = xA[0] > mA || xA[1] > mA || xB[0] > mB || xB[1] > mB;
    if (vtrig || __builtin_amdgcn_ballot_w64(up) != 0) {
      const float nA = fmax_fast(mA, row16_max(fmax_fast(xA[0], xA[1])));
      const float nB = fmax_fast(mB, row16_max(fmax_fast(xB[0], xB[1])));
      const float aA = nA > mA ? __builtin_amdgcn_exp2f(mA - nA) : 1.f;
      const float aB = nB > mB ? __builtin_amdgcn_exp2f(mB - nB) : 1.f;
      mA = nA;
      mB = nB;
      lA *= aA;
      lB *= aB;
      wave_sync();
      if (col == 0) {
        alds[hA] = aA;
        alds[hB] = aB;
        alds[8 + hA] = aA;
        alds[8 + hB] = aB;
      }
      wave_sync();
      const f4_t al = *reinterpret_cast<const f4_t*>(&alds[4 * r]) * vratio;
#pragma unroll
      for (int i = 0; i < NN; ++i) acc[i] *= al;
      if constexpr (OUT) {
        acco[0] *= al;
        acco[1] *= al;
      }
      if constexpr (VM) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          mvA[j] *= aA;
          mvB[j] *= aB;
        }
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      pA[m] = __builtin_amdgcn_exp2f(xA[m] - mA);
      pB[m] = __builtin_amdgcn_exp2f(xB[m] - mB);
    }
    lA += pA[0] + pA[1];
    lB += pB[0] + pB[1];
  };

  // ------------------------------------------------ fused step's positions
  // One wave per (b, g, head chunk) appends the step's token to the cache
  // (the first chunk stores it; every chunk needs its values) and attends
  // to the positions the append changes: position 0 below is the one that
  // becomes quantized (nq >= 1), position 1 the new token in the bf16 tail
  // (T > 0).  It runs before the wave's tiles (the workgroup's other waves
  // take more of them meanwhile), and issues every load it needs (both
  // planes' rows, the V items the new codes merge into, the query) before
  // it waits once.  The contributions take the V weight factor 2^vfe (1
  // here).  The ring slot the new token overwrites held the position that
  // leaves the tail, which no other wave reads in this launch.
  if constexpr (!PF) {
    if (stp && blockIdx.x == 0 && wv == 0) {
      float* sv = step_vals;
      const bool first = (int)blockIdx.y % a.n_gchunks == 0;
      OneLoads LK, LV;
      append_one_load<D, VB>(a.step, g, b, 0, n - 1, first, LK);
      append_one_load<D, VB>(a.step, g, b, 1, n - 1, first, LV);
      float f[NB][8];
      load_query(f);
      append_one_finish<D, VB, false, KB>(a.step, g, b, 0, n - 1, first, LK, sv, sv + 2 * D);
      append_one_finish<D, VB, false, KB>(a.step, g, b, 1, n - 1, first, LV, sv + D, sv + 3 * D);
      wave_sync();
      const bool has0 = nq >= 1, has1 = T > 0;
      float d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = kBlock * j + 8 * r + i;
          d0 = __builtin_fmaf(f[j][i], has0 ? sv[2 * D + e] : 0.f, d0);
          d1 = __builtin_fmaf(f[j][i], has1 ? sv[e] : 0.f, d1);
        }
      }
      d0 += __shfl_xor(d0, 16);
      d0 += __shfl_xor(d0, 32);
      d1 += __shfl_xor(d1, 16);
      d1 += __shfl_xor(d1, 32);
      // head h's score sits in lane 2h (column 2h, row group 0)
      const float cs = a.sm_scale * kLog2e;
      const float a0 = __shfl(d0 * cs, 4 * r), b0 = __shfl(d0 * cs, 4 * r + 2);
      const float a1 = __shfl(d1 * cs, 4 * r), b1 = __shfl(d1 * cs, 4 * r + 2);
      float xA[2], xB[2], pA[2], pB[2];
      xA[0] = col == 0 && has0 && okA ? a0 : -INFINITY;
      xA[1] = col == 0 && has1 && okA ? a1 : -INFINITY;
      xB[0] = col == 0 && has0 && okB ? b0 : -INFINITY;
      xB[1] = col == 0 && has1 && okB ? b1 : -INFINITY;
      softmax(xA, xB, pA, pB, false, 1.f);
      const float vfac = __uint_as_float((uint32_t)(127 + vfe) << 23);
      wave_sync();
      if (col == 0) {
        step_w[0][hA] = pA[0];
        step_w[0][hB] = pB[0];
        step_w[1][hA] = pA[1];
        step_w[1][hB] = pB[1];
      }
      wave_sync();
      if (r < 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float w0 = has0 ? step_w[0][4 * r + k] * vfac : 0.f;
          const float w1 = has1 ? step_w[1][4 * r + k] * vfac : 0.f;
#pragma unroll
          for (int i = 0; i < NN; ++i) {
            const int e = 16 * i + col;
            const float v0 = has0 ? sv[3 * D + e] : 0.f, v1 = has1 ? sv[D + e] : 0.f;
            acc[i][k] = __builtin_fmaf(w1, v1, __builtin_fmaf(w0, v0, acc[i][k]));
          }
        }
      }
    }
  }

  // ------------------------------------------------ bf16 tail positions
  // Same steps on bf16 rows with bf16 matrix products.  The float32 query
  // and the weights are each split into a high and a low bf16 part, so the
  // products carry about 16 significant bits: query parts are A rows 2h /
  // 2h+1 of Q.K, weight parts are A rows h / 8+h of P.V (rows 8..15 of the
  // accumulators are added to rows 0..7 at the end).  K rows come straight
  // from the ring; each lane gathers its element of 8 V rows.
  const int tk0 = (int)blockIdx.x + (PF ? 0 : NG * wv);
  if (tk0 < ctt) {
    const uint16_t* ktl = a.k_tail + unit * (size_t)T * D;
    const uint16_t* vtl = a.v_tail + unit * (size_t)T * D;
    bf8_t qt[NB];
    {
      float f[NB][8];
      load_query(f);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t hi = f32_to_bf16_bits(f[j][e]);
          const uint32_t lo = f32_to_bf16_bits(f[j][e] - __uint_as_float(hi << 16));
          qt[j][e] = __builtin_bit_cast(__bf16, (uint16_t)(col < 2 * G && row_ok(col / 2) ? ((col & 1) ? lo : hi) : 0u));
        }
      }
    }
    const float csA = okA ? a.sm_scale * kLog2e : 0.f;
    const float csB = okB ? a.sm_scale * kLog2e : 0.f;
    for (int kt = tk0; kt < ctt; kt += NG * (PF ? 1 : kGroupWaves)) {
    const int ta = nq + kt * kTile, tb = min(ntr, ta + kTile);
    if (PF && ta > wlim) break;
    for (int s0 = ta; s0 < tb && (!PF || s0 <= wlim); s0 += kStep) {
      f4_t d[2] = {f4_t{0.f, 0.f, 0.f, 0.f}, f4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int tok = s0 + 16 * m + col;
        const uint16_t* krow = ktl + (size_t)((tok < tb ? tok : ta) % T) * D + 8 * r;
#pragma unroll
        for (int j = 0; j < NB; ++j)
          d[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt[j], ld_cache<kNT, bf8_t>(krow + kBlock * j), d[m], 0, 0, 0);
      }
      bool vA[2], vB[2];
      float xA[2], xB[2], pA[2], pB[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int tok = s0 + 16 * m + col;
        vA[m] = tok < tb && (!PF || tok <= limA);
        vB[m] = tok < tb && (!PF || tok <= limB);
        float ya = (d[m][0] + d[m][1]) * csA, yb = (d[m][2] + d[m][3]) * csB;
        asm volatile("" : "+v"(ya), "+v"(yb));
        xA[m] = vA[m] && okA ? ya : -INFINITY;
        xB[m] = vB[m] && okB ? yb : -INFINITY;
      }
      softmax(xA, xB, pA, pB, false, 1.f);
      wave_sync();
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int t = 16 * m + col;
        const float wA = vA[m] ? pA[m] : 0.f;
        const float wB = vB[m] ? pB[m] : 0.f;
        const uint32_t hiA = f32_to_bf16_bits(wA), hiB = f32_to_bf16_bits(wB);
        wl[hA * WROW + t] = (uint16_t)hiA;
        wl[hB * WROW + t] = (uint16_t)hiB;
        wl[(LOROW + hA) * WROW + t] = (uint16_t)f32_to_bf16_bits(wA - __uint_as_float(hiA << 16));
        wl[(LOROW + hB) * WROW + t] = (uint16_t)f32_to_bf16_bits(wB - __uint_as_float(hiB << 16));
      }
      wave_sync();
      const int row = col < 8 ? col : LOROW + col - 8;
      const bf8_t wa = *reinterpret_cast<const bf8_t*>(&wl[row * WROW + 8 * r]);
      size_t voff[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int tok = s0 + 8 * r + k;
        voff[k] = (size_t)((tok < tb ? tok : ta) % T) * D + col;
      }
#pragma unroll
      for (int i = 0; i < NN; ++i) {
        bf8_t vb;
#pragma unroll
        for (int k = 0; k < 8; ++k) vb[k] = __builtin_bit_cast(__bf16, ld_cache<kNT, uint16_t>(vtl + voff[k] + 16 * i));
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, vb, acc[i], 0, 0, 0);
      }
    }
    }
  }

  // ------------------------------------------------ quantized positions
  if (PF ? wq0 < wq1 : (int)blockIdx.x < ctq) {
    constexpr int KSE = KM ? 2 * NB : NB;   // 16-bit scale entries per token
    constexpr int VSE = VM ? 2 * NB : NB;
    // A operand of Q.K: the rotated query in fixed point (step amax / 32639
    // per head), high bytes in even rows, low bytes in odd rows;
    // 4/5-bit codes widen to bytes in the order 0,2,4,6,1,3,5,7 of each group
    // of 8, so the query bytes follow that order.  Offset-binary codes need a
    // per-block correction -offset * sum(q_int), which seeds the low-byte rows
    // of the integer accumulators: cq[j] = {0, corr_hA, 0, corr_hB}.
    // The query extends to 24 bits (kQ24) by the residual byte
    // rint(256 * (q / step - q_int)).  Up to 4 heads (kFold) lanes of A rows
    // 8..15 hold the query of row - 8, and odd rows carry its residual bytes:
    // their sums land 32 lanes above the hi / lo sums of the same token, each
    // half sums its K-scaled blocks, and one lane swap adds the upper half's
    // sum / 256.  Otherwise (kQX) a second product per block takes the
    // residual bytes in the odd rows (so its sums land in the same lanes),
    // with its own offset correction (seeded, or two integers per block where
    // the main correction is).
    constexpr bool kQX = kQ24 && !kFold;
    constexpr bool kOffset = KB != 8 && !KM;   // offset-binary codes
    long qop[NB];
    long qres[kQX ? NB : 1];
    float ckA, ckB;
    // outlier channels: the unrotated query at K's channels in 16-bit fixed
    // point of its own step, and that step's score factor per head
    long qopo = 0;
    float ckoA = 0.f, ckoB = 0.f;
    // head_dim 256 keeps the correction as two integers per block, added to
    // the combined sums (exact), to free registers for issuing the two token
    // halves' products together
    constexpr bool kCorrInt = kOffset && D >= 192;
    i4_t cq[kOffset && !kCorrInt ? NB : 1];
    int ciA[kCorrInt ? NB : 1], ciB[kCorrInt ? NB : 1];
    int ci2A[kCorrInt && kQX ? NB : 1], ci2B[kCorrInt && kQX ? NB : 1];
    i4_t cq2[kQX && kOffset && !kCorrInt ? NB : 1];
    // K minima: sum of the fixed-point query over each block, heads hA, hB
    float bsA[KM ? NB : 1], bsB[KM ? NB : 1];
    // 5-bit K: bit 4 of the codes of this lane's group r sits at bits
    // 8i + 2r (even elements) and 8i + 2r + 1 (odd) of the block's word;
    // 6-bit K: bits 4-5 sit at 8i + 4(r%2) (even) and 8i + 4(r%2) + 2 (odd)
    // of the block's high word r/2; both rotate into bits 4(-5) of byte i
    const uint32_t rot_lo = KB == 6 ? (uint32_t)(4 * (r & 1) + 28) & 31u
                                    : (uint32_t)(2 * r + 28) & 31u;
    const uint32_t rot_hi = KB == 6 ? (uint32_t)(4 * (r & 1) + 30) & 31u
                                    : (uint32_t)(2 * r + 29) & 31u;
    uint32_t magic = 0x64006400u;
    asm volatile("" : "+v"(magic));

    // per-lane byte offsets inside a tile; the tile base is uniform
    const uint32_t k_off = KB == 8 ? (uint32_t)((((r >> 1) * kTile + col) * kChunk) + 8 * (r & 1))
                                   : (uint32_t)(col * kChunk + 4 * r);
    const uint32_t v_off = (uint32_t)(lane * NN * (VB == 8 ? 8 : 4));
    const uint32_t vh_off = (uint32_t)(32 * D + lane * NN);

    // Slot of position s0's tile in the contiguous or paged planes (see
    // tile_slot).  A paged cache's entry is read through the scalar cache
    // (the table is read-only while the kernel runs), so the lookup holds no
    // vector register and waits for no tile load; consecutive tiles share
    // its cache line.
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    // contiguous planes of this (b, g)
    const uint8_t* kpl = a.k_codes + unit * (size_t)a.cap * RKP;
    const uint16_t* ksc = a.k_scales + unit * (size_t)a.cap * KSE;
    const uint8_t* vpl = a.v_codes + unit * (size_t)(a.cap / kTile) * VTB;
    const uint16_t* vsc = a.v_scales + unit * (size_t)a.cap * VSE;
    auto load_step = [&](Regs& R, int s0) {
      if constexpr (OUT) {
        // outlier planes: [tile][64][32] K bytes, element-major V tiles of
        // 2 KiB, [tile][64] scales; the tile's slot as for the other planes
        size_t oslot = unit * (size_t)(a.cap / kTile) + s0 / kTile;
        if (PGM == kPagePaged || (PGM == kPageAny && a.map.ptab != nullptr)) {
          const int page = ((const __attribute__((address_space(4))) int32_t*)a.map.ptab)[(size_t)b * a.map.tiles +
                                                                                            s0 / kTile];
          oslot = (unsigned)page < (unsigned)a.map.n_pages ? (size_t)page * a.map.Hkv + g : (size_t)g;
        }
        const uint8_t* kot = a.out_codes[0] + oslot * (kTile * kOutl);
        const uint8_t* vot = a.out_codes[1] + oslot * (kTile * kOutl);
        const uint16_t* kos = a.out_scales[0] + oslot * kTile;
        const uint16_t* vos = a.out_scales[1] + oslot * kTile;
        const int l0 = s0 % kTile;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int l = l0 + 16 * m + col;
          R.ko[m] = ld_cache<kNT, u32x2>(kot + l * kOutl + 8 * r);
          R.kos[m] = ld_cache<kNT, uint16_t>(kos + l);
          R.vos[m] = ld_cache<kNT, uint16_t>(vos + l);
        }
        R.vo = ld_cache<kNT, u32x4>(vot + ((l0 / kStep) * 64 + lane) * 16);
      }
      const int j2 = (s0 / kStep) & 1;
      // s0's K and V tiles and its row of each scale plane
      const uint8_t* ktile = kpl + (size_t)(s0 / kTile) * kTile * RKP;
      const uint8_t* vt = vpl + (size_t)(s0 / kTile) * VTB;
      const uint16_t* ksrow = ksc;
      const uint16_t* vsrow = vsc;
      int srow = s0;   // scale row of s0 from ksrow / vsrow
      if (PGM == kPagePaged || (PGM == kPageAny && a.map.ptab != nullptr)) {
        const int page = ((const_i32*)a.map.ptab)[(size_t)b * a.map.tiles + s0 / kTile];
        const size_t slot =
            (unsigned)page < (unsigned)a.map.n_pages ? (size_t)page * a.map.Hkv + g : (size_t)g;
        ktile = a.k_codes + slot * (kTile * RKP);
        vt = a.v_codes + slot * VTB;
        ksrow = a.k_scales + slot * kTile * KSE;
        vsrow = a.v_scales + slot * kTile * VSE;
        srow = s0 % kTile;
      }
      const uint8_t* kt = ktile + j2 * kStep * kChunk;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if constexpr (KB == 8) {
            R.k8[m * NB + j] = ld_cache<kNT, u32x2>(kt + (2 * j * kTile + 16 * m) * kChunk + k_off);
          } else {
            R.k4[m * NB + j] = ld_cache<kNT, uint32_t>(kt + (j * kTile + 16 * m) * kChunk + k_off);
            if constexpr (KB == 5) {
              const int cb = D / 32 + j / 4;
              R.kh[m * NB + j] = ld_cache<kNT, uint32_t>(kt + (cb * kTile + 16 * m + col) * kChunk + 4 * (j % 4));
            }
            if constexpr (KB == 6) {
              const int cb = D / 32 + j / 2;
              R.kh[m * NB + j] = ld_cache<kNT, uint32_t>(kt + (cb * kTile + 16 * m + col) * kChunk + 8 * (j % 2) +
                                                     4 * (r >> 1));
            }
          }
        }
        const size_t tok = (size_t)srow + 16 * m + col;
        load_words<kNT>(reinterpret_cast<const uint32_t*>(ksrow + tok * KSE), R.ks[m]);
        load_words<kNT>(reinterpret_cast<const uint32_t*>(vsrow + tok * VSE), R.vs[m]);
      }
      const uint8_t* vj = vt + (size_t)j2 * 64 * NN * (VB == 8 ? 8 : 4) + v_off;
#pragma unroll
      for (int q = 0; q < (VB == 8 ? NN / 2 : NN / 4); ++q) R.v[q] = ld_cache<kNT, u32x4>(vj + 16 * q);
      if constexpr (VB == 5) {
        const uint8_t* hj = vt + (size_t)j2 * 64 * NN + vh_off;
#pragma unroll
        for (int q = 0; q < NN / 4; ++q) R.vh[q] = ld_cache<kNT, uint32_t>(hj + 4 * q);
      }
      if constexpr (VB == 6) {
        const uint8_t* hj = vt + 32 * D + (size_t)j2 * 64 * NN * 2 + (size_t)lane * NN * 2;
#pragma unroll
        for (int q = 0; q < NN / 2; ++q) R.vh[q] = ld_cache<kNT, uint32_t>(hj + 4 * q);
      }
    };

    auto compute_step = [&](const Regs& R, int s0) {
      // Q.K on the matrix cores: 2 x NB products of 16 tokens x 32 elements,
      // twice that where the residual bytes of the 24-bit query take a second
      // product (kQX: more than 4 heads, or prefill).  Up to head_dim 128 all of
      // them are issued before the first result is read, so their latencies
      // overlap instead of each product waiting out the last one's; the
      // registers allow it there except with scale-and-min blocks or 5- and
      // 6-bit K (their high-bit words), which then spilled.
      float sA[2] = {0.f, 0.f}, sB[2] = {0.f, 0.f};
      constexpr bool kIssueAll = NB <= 4 && !(kQX && (KM || VM || KB == 5 || KB == 6));
      // head_dim 256: the two token halves of one block together
      constexpr bool kIssuePair = !kIssueAll && D >= 192;
      // blocks per issued group above head_dim 128: two at 256 (one wave per
      // SIMD, registers for it once the correction is two integers), one at
      // 192 (two waves per SIMD)
      constexpr int kPairBlocks = D == 256 ? 2 : 1;
      i4_t dq[kIssueAll ? NB : kPairBlocks][2];
      i4_t dr[kQX ? (kIssueAll ? NB : (kIssuePair ? kPairBlocks : 1)) : 1][2];
      if constexpr (kIssueAll) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const long kop = k_operand<D, KB, VB, KM, VM>(R, m * NB + j, rot_lo, rot_hi);
            dq[j][m] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                qop[j], kop, kOffset && !kCorrInt ? cq[kOffset && !kCorrInt ? j : 0] : i4_t{0, 0, 0, 0}, 0, 0, 0);
            if constexpr (kQX)
              dr[j][m] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                  qres[j], kop, kOffset && !kCorrInt ? cq2[kOffset && !kCorrInt ? j : 0] : i4_t{0, 0, 0, 0}, 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          i4_t d;
          long kop = 0;
          if constexpr (kIssuePair) {
            if (m == 0 && j % kPairBlocks == 0) {
#pragma unroll
              for (int jj = j; jj < j + kPairBlocks; ++jj)
#pragma unroll
              for (int mm = 0; mm < 2; ++mm) {
                const long kp = k_operand<D, KB, VB, KM, VM>(R, mm * NB + jj, rot_lo, rot_hi);
                dq[jj % kPairBlocks][mm] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                    qop[jj], kp, kOffset && !kCorrInt ? cq[kOffset && !kCorrInt ? jj : 0] : i4_t{0, 0, 0, 0},
                    0, 0, 0);
                if constexpr (kQX)
                  dr[jj % kPairBlocks][mm] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                      qres[jj], kp, kOffset && !kCorrInt ? cq2[kOffset && !kCorrInt ? jj : 0] : i4_t{0, 0, 0, 0},
                      0, 0, 0);
              }
            }
            d = dq[j % kPairBlocks][m];
          } else if constexpr (kIssueAll) {
            d = dq[j][m];
          } else {
            kop = k_operand<D, KB, VB, KM, VM>(R, m * NB + j, rot_lo, rot_hi);
            d = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                qop[j], kop, kOffset && !kCorrInt ? cq[kOffset && !kCorrInt ? j : 0] : i4_t{0, 0, 0, 0}, 0, 0, 0);
          }
          int vA = (d[0] << 8) + d[1];
          int vB = (d[2] << 8) + d[3];
          if constexpr (kCorrInt) {
            vA += ciA[j];
            vB += ciB[j];
          }
          const float ks = R.k_scale(m, j);
          float fA = (float)vA, fB = (float)vB;
          if constexpr (kQX) {
            i4_t e;
            if constexpr (kIssueAll) {
              e = dr[j][m];
            } else if constexpr (kIssuePair) {
              e = dr[j % kPairBlocks][m];
            } else {
              e = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                  qres[j], kop, kOffset && !kCorrInt ? cq2[kOffset && !kCorrInt ? j : 0] : i4_t{0, 0, 0, 0}, 0, 0, 0);
            }
            int eA = e[1], eB = e[3];
            if constexpr (kCorrInt) {
              eA += ci2A[j];
              eB += ci2B[j];
            }
            fA = __builtin_fmaf((float)eA, 0.00390625f, fA);
            fB = __builtin_fmaf((float)eB, 0.00390625f, fB);
          }
          sA[m] = __builtin_fmaf(ks, fA, sA[m]);
          sB[m] = __builtin_fmaf(ks, fB, sB[m]);
          if constexpr (KM) {
            const float km = R.k_min(m, j);
            sA[m] = __builtin_fmaf(km, bsA[j], sA[m]);
            sB[m] = __builtin_fmaf(km, bsB[j], sB[m]);
          }
        }
      }
      if constexpr (kFold) {
        // lanes 0..31 add the residual sums of lanes 32..63 (same tokens,
        // same heads); the upper lanes hold no score head
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float uA = upper_half(sA[m]), uB = upper_half(sB[m]);
          sA[m] = __builtin_fmaf(uA, 0.00390625f, sA[m]);
          sB[m] = __builtin_fmaf(uB, 0.00390625f, sB[m]);
        }
      }
      float soA[2] = {0.f, 0.f}, soB[2] = {0.f, 0.f};
      if constexpr (OUT) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const i4_t e = __builtin_amdgcn_mfma_i32_16x16x32_i8(qopo, __builtin_bit_cast(long, R.ko[m]),
                                                               i4_t{0, 0, 0, 0}, 0, 0, 0);
          const float kso = half_of(R.kos[m], 0);
          soA[m] = kso * (float)((e[0] << 8) + e[1]);
          soB[m] = kso * (float)((e[2] << 8) + e[3]);
        }
      }
      float xA[2], xB[2], pA[2], pB[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int tok = s0 + 16 * m + col;
        const bool validA = tok < nqr && (!PF || tok <= limA);
        const bool validB = tok < nqr && (!PF || tok <= limB);
        float ya = sA[m] * ckA, yb = sB[m] * ckB;
        if constexpr (OUT) {
          ya = __builtin_fmaf(soA[m], ckoA, ya);
          yb = __builtin_fmaf(soB[m], ckoB, yb);
        }
        asm volatile("" : "+v"(ya), "+v"(yb));   // selects, not branches
        xA[m] = validA && okA ? ya : -INFINITY;
        xB[m] = validB && okB ? yb : -INFINITY;
      }
      // largest V scale of the step's positions (those past the quantized
      // range hold no data) against the weight factor's threshold; a new
      // factor rescales the accumulators with the softmax's rescaling
      bool vtrig = false;
      float vratio = 1.f;
      {
        uint32_t l0 = v_scale_max_bits<D, KB, VB, KM, VM>(R, 0);
        uint32_t l1 = v_scale_max_bits<D, KB, VB, KM, VM>(R, 1);
        if constexpr (OUT) {
          l0 = max(l0, R.vos[0] & 0xFFFFu);
          l1 = max(l1, R.vos[1] & 0xFFFFu);
        }
        l0 = s0 + col < nqr ? l0 : 0u;
        l1 = s0 + 16 + col < nqr ? l1 : 0u;
        const uint32_t lm = l0 > l1 ? l0 : l1;
        if (__builtin_amdgcn_ballot_w64(lm >= vthr) != 0) {
          const float mx = row16_max((float)__builtin_bit_cast(_Float16, (uint16_t)lm));
          const uint32_t mb = __builtin_amdgcn_readfirstlane(__float_as_uint(mx));
          if (mb != 0u) {
            const int e = (int)((mb >> 23) & 0xFFu) - 127;   // 2^e <= max < 2^(e+1), e >= -24
            const int nfe = 11 - e;
            vratio = __uint_as_float((uint32_t)(127 + nfe - vfe) << 23);
            vtrig = true;
            vfe = nfe;
            const int k = e + 4;   // threshold 2^(e + 4) in fp16 bits
            vthr = k > 15 ? 0x7C00u : (k >= -14 ? (uint32_t)(k + 15) << 10 : 1u << (k + 24));
          }
        }
      }
      softmax(xA, xB, pA, pB, vtrig, vratio);
      const float vf = __uint_as_float((uint32_t)(127 + vfe) << 23);
      // weights p * scale_v * 2^vfe in fp16 (0 for masked tokens and absent
      // heads), moved to the A-operand layout via LDS
      wave_sync();
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float vs = R.v_scale(m, j);
          const int t = 16 * m + col;
          const float fA = pA[m] * vf * vs, fB = pB[m] * vf * vs;
          const _Float16 wA = (_Float16)fA;
          const _Float16 wB = (_Float16)fB;
          wl[(8 * j + hA) * WROW + t] = __builtin_bit_cast(uint16_t, wA);
          wl[(8 * j + hB) * WROW + t] = __builtin_bit_cast(uint16_t, wB);
          if constexpr (kLoW) {
            // Scale-and-min blocks: a block whose range an outlier stretches
            // puts its ordinary elements far from the block's middle level,
            // so their centred levels are large against their values, and
            // the weight's fp16 rounding, common to the whole block, would
            // not cancel in a sum that nearly does.  Prefill rows: a row whose
            // output nearly cancels magnifies the weights' rounding (a
            // seeded sweep found 1.6e-3 at head_dim 64 with single fp16
            // weights).  The low fp16 part of each weight goes in A rows
            // 8..15 (otherwise zero), whose accumulator rows are added to
            // rows 0..7 at the end: about 22 significant bits for no extra
            // matrix products.
            wl[(LOQ + 8 * j + hA) * WROW + t] = __builtin_bit_cast(uint16_t, (_Float16)(fA - (float)wA));
            wl[(LOQ + 8 * j + hB) * WROW + t] = __builtin_bit_cast(uint16_t, (_Float16)(fB - (float)wB));
          }
        }
      }
      if constexpr (OUT) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float vso = half_of(R.vos[m], 0);
          const int t = 16 * m + col;
          wl[(OROW + hA) * WROW + t] = __builtin_bit_cast(uint16_t, (_Float16)(pA[m] * vf * vso));
          wl[(OROW + hB) * WROW + t] = __builtin_bit_cast(uint16_t, (_Float16)(pB[m] * vf * vso));
        }
      }
      if constexpr (VM) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          // x = u * s + m = (u - o) * s + (m + o * s): the matrix product
          // takes the centred levels u - o, so the rounding of its fp16
          // weights does not act on the block's offset, which goes here
          constexpr float o = (float)(1 << (VB - 1));
          const float v0 = __builtin_fmaf(o, R.v_scale(0, j), R.v_min(0, j));
          const float v1 = __builtin_fmaf(o, R.v_scale(1, j), R.v_min(1, j));
          mvA[j] = __builtin_fmaf(pA[1], v1, __builtin_fmaf(pA[0], v0, mvA[j]));
          mvB[j] = __builtin_fmaf(pB[1], v1, __builtin_fmaf(pB[0], v0, mvB[j]));
        }
      }
      wave_sync();
      // P.V on the matrix cores: NN products of 16 rows x 32 tokens x 16 elements
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int row = col < 8 ? 8 * j + col : (kLoW ? LOQ + 8 * j + col - 8 : ZROW);
        const h8_t wa = *reinterpret_cast<const h8_t*>(&wl[row * WROW + 8 * r]);
#pragma unroll
        for (int i = 2 * j; i < 2 * j + 2; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, v_operand<D, KB, VB, KM, VM>(R, i, magic), acc[i], 0, 0, 0);
      }
      if constexpr (OUT) {
        const int row = col < 8 ? OROW + col : ZROW;
        const h8_t wa = *reinterpret_cast<const h8_t*>(&wl[row * WROW + 8 * r]);
        acco[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, v_operand8(R.vo, 0), acco[0], 0, 0, 0);
        acco[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, v_operand8(R.vo, 1), acco[1], 0, 0, 0);
      }
    };

    // Tiles come from the workgroup's LDS counter, one tile ahead: the
    // second half of a tile and the first half of the next one load while
    // the half before computes.
    uint32_t pf_next = 0;
    auto grab_issue = [&]() {
      uint32_t v = 0;
      if constexpr (PF) {
        v = pf_next++;
      } else {
        if (lane == 0) v = atomicAdd(&tile_ctr, 1u);
      }
      return v;
    };
    auto grab_read = [&](uint32_t v) {
      const int c = (int)__builtin_amdgcn_readfirstlane(v);
      if constexpr (PF) {
        const int t = wq0 + c;
        return t * kTile > wlim ? wq1 : t;   // past the rows' last position
      } else {
        return c * NG + (int)blockIdx.x;
      }
    };
    // query operands, built while the first loads are in flight
    auto prep_query = [&]() {
      float f[NB][8];
      load_query(f);
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[j][i]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      if constexpr (OUT) {
        // q at K's outlier channels 8r..8r+7 of the list (original space)
        const int hq = col < 2 * G && row_ok(col / 2) ? col / 2 : 0;
        const size_t qoff = row_vec(hq) * D;
        const int32_t* kidx = a.out_idx + (size_t)g * kOutl + 8 * r;
        float fo[8];
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int ch = outlier_channel(kidx, i, D);
          fo[i] = a.q_dtype == KVQ_BF16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(a.q)[qoff + ch] << 16)
                                        : static_cast<const float*>(a.q)[qoff + ch];
          am = fmaxf(am, fabsf(fo[i]));
        }
        am = fmaxf(am, __shfl_xor(am, 16));
        am = fmaxf(am, __shfl_xor(am, 32));
        const float so = am > 0.f ? am / 32639.0f : 1.0f;
        const float io = 1.0f / so;
        uint64_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          int x = (int)rintf(fo[i] * io);
          x = x > 32639 ? 32639 : (x < -32639 ? -32639 : x);
          const int hi = (x + 128) >> 8;
          const int byte = (col & 1) ? x - 256 * hi : hi;
          w |= (uint64_t)(uint8_t)(int8_t)byte << (8 * i);
        }
        qopo = col < 2 * G && row_ok(col / 2) ? (long)w : 0;
        const float cko = so * a.sm_scale * kLog2e;
        ckoA = okA ? __shfl(cko, 4 * r) : 0.f;
        ckoB = okB ? __shfl(cko, 4 * r + 2) : 0.f;
      }
      const float step = amax > 0.f ? amax / 32639.0f : 1.0f;
      const float inv = 1.0f / step;
      const float ck = step * a.sm_scale * kLog2e;
      ckA = __shfl(ck, 4 * r);
      ckB = __shfl(ck, 4 * r + 2);
      ckA = okA ? ckA : 0.f;
      ckB = okB ? ckB : 0.f;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        int v[8], res[8];
        int bsum = 0, rsum = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float t = f[j][i] * inv;
          int x = (int)rintf(t);
          x = x > 32639 ? 32639 : (x < -32639 ? -32639 : x);
          v[i] = x;
          bsum += x;
          if constexpr (kQ24) {
            int y = (int)rintf((t - (float)x) * 256.0f);
            y = y > 127 ? 127 : (y < -127 ? -127 : y);
            res[i] = y;
            rsum += y;
          }
        }
        uint64_t w = 0, wr = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = KB == 8 ? i : (i < 4 ? 2 * i : 2 * (i - 4) + 1);
          const int hi = (v[e] + 128) >> 8;
          const int byte = (col & 1) ? v[e] - 256 * hi : hi;
          w |= (uint64_t)(uint8_t)(int8_t)byte << (8 * i);
          if constexpr (kQ24) wr |= (uint64_t)(uint8_t)(int8_t)res[e] << (8 * i);
        }
        const bool row_here = col < 2 * G && row_ok(col / 2);
        if constexpr (kFold) {
          const bool res_here = col >= 8 && (col & 1) && col - 8 < 2 * G && row_ok((col - 8) / 2);
          qop[j] = row_here ? (long)w : (res_here ? (long)wr : 0);
        } else {
          qop[j] = row_here ? (long)w : 0;
        }
        if constexpr (kQX) qres[j] = row_here && (col & 1) ? (long)wr : 0;
        if constexpr (KM) {
          bsum += __shfl_xor(bsum, 16);
          bsum += __shfl_xor(bsum, 32);
          float bf = (float)bsum;
          if constexpr (kQ24) {
            rsum += __shfl_xor(rsum, 16);
            rsum += __shfl_xor(rsum, 32);
            bf = __builtin_fmaf((float)rsum, 0.00390625f, bf);
          }
          bsA[j] = okA ? __shfl(bf, 4 * r) : 0.f;
          bsB[j] = okB ? __shfl(bf, 4 * r + 2) : 0.f;
        }
        if constexpr (kOffset) {
          bsum += __shfl_xor(bsum, 16);
          bsum += __shfl_xor(bsum, 32);
          int corr = -(1 << (KB - 1)) * bsum;
          bool cokA = okA, cokB = okB;
          if constexpr (kFold) {
            // rows 8..15: the residual bytes' correction, for heads 2r - 4, 2r - 3
            rsum += __shfl_xor(rsum, 16);
            rsum += __shfl_xor(rsum, 32);
            corr = col >= 8 ? -(1 << (KB - 1)) * rsum : corr;
            cokA = r >= 2 ? row_ok(hA - 4) : okA;
            cokB = r >= 2 ? row_ok(hB - 4) : okB;
          }
          const int cA = cokA ? __shfl(corr, 4 * r) : 0, cB = cokB ? __shfl(corr, 4 * r + 2) : 0;
          if constexpr (kCorrInt) {
            ciA[j] = cA;
            ciB[j] = cB;
          } else {
            cq[j] = i4_t{0, cA, 0, cB};
          }
          if constexpr (kQX) {
            rsum += __shfl_xor(rsum, 16);
            rsum += __shfl_xor(rsum, 32);
            const int corr2 = -(1 << (KB - 1)) * rsum;
            const int c2A = okA ? __shfl(corr2, 4 * r) : 0, c2B = okB ? __shfl(corr2, 4 * r + 2) : 0;
            if constexpr (kCorrInt) {
              ci2A[j] = c2A;
              ci2B[j] = c2B;
            } else {
              cq2[j] = i4_t{0, c2A, 0, c2B};
            }
          }
        }
      }
    };
    if constexpr (kAhead == 1) {
      int t_cur = grab_read(grab_issue());
      if (t_cur < qend) {
        int t_nxt = grab_read(grab_issue());
        Regs ra, rb;
        load_step(ra, t_cur * kTile);
        prep_query();
        while (true) {
          const uint32_t t_aft_v = grab_issue();
          load_step(rb, t_cur * kTile + kStep);
          compute_step(ra, t_cur * kTile);
          if (t_nxt < qend) load_step(ra, t_nxt * kTile);
          compute_step(rb, t_cur * kTile + kStep);
          const int t_aft = grab_read(t_aft_v);
          if (t_nxt >= qend) break;
          t_cur = t_nxt;
          t_nxt = t_aft;
        }
      }
    } else {
      // two tiles (four steps) in registers: while one step computes, the
      // next three are loaded or in flight
      int t0 = grab_read(grab_issue());
      if (t0 < qend) {
        int t1 = grab_read(grab_issue());
        Regs ra0, rb0, ra1, rb1;
        load_step(ra0, t0 * kTile);
        load_step(rb0, t0 * kTile + kStep);
        if (t1 < qend) {
          load_step(ra1, t1 * kTile);
          load_step(rb1, t1 * kTile + kStep);
        }
        prep_query();
        while (true) {
          const int t2 = grab_read(grab_issue());
          compute_step(ra0, t0 * kTile);
          if (t2 < qend) load_step(ra0, t2 * kTile);
          compute_step(rb0, t0 * kTile + kStep);
          if (t2 < qend) load_step(rb0, t2 * kTile + kStep);
          if (t1 >= qend) break;
          const int t3 = grab_read(grab_issue());
          compute_step(ra1, t1 * kTile);
          if (t3 < qend) load_step(ra1, t3 * kTile);
          compute_step(rb1, t1 * kTile + kStep);
          if (t3 < qend) load_step(rb1, t3 * kTile + kStep);
          if (t2 >= qend) break;
          t0 = t2;
          t1 = t3;
        }
      }
    }
  }

  // ------------------------------------------------ partial results
  // rows h and 8+h of the accumulators belong to head h
  lA = row16_sum(lA);
  lB = row16_sum(lB);
  {
    const float inv = __uint_as_float((uint32_t)(127 - vfe) << 23);   // exact
#pragma unroll
    for (int i = 0; i < NN; ++i) acc[i] *= inv;
  }
#pragma unroll
  for (int i = 0; i < NN; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[i][k] += __shfl_xor(acc[i][k], 32);
  }
  if constexpr (VM) {
    // head h's sum(p * m) of V block j (reduced over the row's 16 lanes) goes
    // to output elements 32j..32j+31 through this wave's LDS rows
    float* mvl = reinterpret_cast<float*>(wl);
    wave_sync();
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float sa = row16_sum(mvA[j]), sb = row16_sum(mvB[j]);
      if (col == 0) {
        mvl[hA * NB + j] = sa;
        mvl[hB * NB + j] = sb;
      }
    }
    wave_sync();
    if (r < 2) {
#pragma unroll
      for (int i = 0; i < NN; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i][k] += mvl[(4 * r + k) * NB + i / 2];
      }
    }
  }
  if (r < 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int h = 4 * r + k;
      if (row_ok(h)) {
        float* dst = a.part_acc + (row_vec(h) * a.S + split) * D + col;
#pragma unroll
        for (int i = 0; i < NN; ++i) dst[16 * i] = acc[i][k];
      }
    }
  }
  if constexpr (OUT) {
    const float inv = __uint_as_float((uint32_t)(127 - vfe) << 23);   // exact
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      acco[i] *= inv;
#pragma unroll
      for (int k = 0; k < 4; ++k) acco[i][k] += __shfl_xor(acco[i][k], 32);
    }
    if (r < 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int h = 4 * r + k;
        if (row_ok(h)) {
          float* dst = a.part_out + (row_vec(h) * a.S + split) * kOutl + col;
          dst[0] = acco[0][k];
          dst[16] = acco[1][k];
        }
      }
    }
  }
  if (col == 0) {
    if (okA) {
      a.part_ml[(row_vec(hA) * a.S + split) * 2] = mA;
      a.part_ml[(row_vec(hA) * a.S + split) * 2 + 1] = lA;
    }
    if (okB) {
      a.part_ml[(row_vec(hB) * a.S + split) * 2] = mB;
      a.part_ml[(row_vec(hB) * a.S + split) * 2 + 1] = lB;
    }
  }
}

template <int D, int KB, int VB, int G, bool PF = false, bool KM = false, bool VM = false,
          int PGM = kPageAny, bool OUT = false>
hipError_t launch_decode_split(const DecodeArgs& a, dim3 grid, hipStream_t s, hipEvent_t t0,
                               hipEvent_t t1) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  const dim3 block(64 * split_group_waves(D, KM || VM || PF));
  if (t0 || t1)
    hipExtLaunchKernelGGL((decode_split_kernel<D, KB, VB, G, PF, KM, VM, PGM, OUT>), grid, block, 0, s,
                          t0, t1, 0, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, KB, VB, G, PF, KM, VM, PGM, OUT>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
