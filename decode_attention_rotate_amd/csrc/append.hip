// Rotate-quantize-append kernels.
//
// Each new K/V head vector is rotated by the normalized Hadamard matrix
// (velog.io post "fix KV cache quantization outliers", section "Hadamard
// rotation") and either quantized into 32-element blocks with one fp16 absmax
// scale, or a scale and a minimum (byte cost per the aiwitness.kr table "Qwen
// 3.6 27B Q5_K_S + 64k context KLD results"), or, for the newest tail_len positions, stored in the
// bf16 precision tail (aitrends.kr article 92204, glossary "Precision Tail").
//
// An append of n_new tokens to a sequence of length len runs in two steps
// (two launches, or one block per (sequence, KV head, plane) with a barrier
// between the steps when n_new is small; one token per sequence has a kernel
// of its own, below):
//  1. quant: positions [q0, q1) become quantized, where q0/q1 are the first
//     non-tail position before/after the append (q0 = len, q1 = len + n_new
//     without a tail).  A position below len is read back from its tail slot
//     (it is leaving the tail), any other one is rotated from the input.
//     Work goes in groups of eight 8-aligned positions, because V codes of
//     eight consecutive tokens share one word of the element-major V tiles:
//     the group's codes meet in LDS and are packed there, merging with the
//     bytes of positions outside [q0, q1) that the group's words also hold.
//  2. tail: the newest min(n_new, T) positions are rotated and written to
//     their ring slots p % T.  This runs after (1), which has read every slot
//     it overwrites.
//
// Thread mapping: one lane per 32-element block, D/32 consecutive lanes per
// head vector, so a 256-thread block covers 256*32/D consecutive positions of
// one (sequence, KV head, plane).  The in-lane butterfly stages h = 1..16 run
// in registers, the remaining stages cross lanes with DPP / ds_swizzle, and
// the block absmax and the codes never leave the lane.
#include "append_one.hpp"

namespace kvq {
namespace {

__device__ inline void load_row_block(const void* src, int dtype, size_t elem_off, float (&x)[32]) {
  if (dtype == KVQ_BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + elem_off);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = p[q];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[q * 8 + 2 * k] = __uint_as_float(w[k] << 16);
        x[q * 8 + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + elem_off);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 v = p[q];
      x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
    }
  }
}

__device__ inline void load_bf16_block(const uint16_t* row, float (&x)[32]) {
  const uint4* src = reinterpret_cast<const uint4*>(row);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = src[q];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[q * 8 + 2 * k] = __uint_as_float(w[k] << 16);
      x[q * 8 + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
}

// Merge the slots of one V item whose bit is set in `mask` into memory.
// u holds the offset codes of slots 0..7 in bytes 0..7.
template <int D, int BITS>
__device__ inline void store_v_item(uint8_t* tile, int item, uint64_t u, uint32_t mask) {
  if constexpr (BITS == 8) {
    uint64_t* dst = reinterpret_cast<uint64_t*>(tile) + item;
    if (mask != 0xFFu) {
      uint64_t keep = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (!(mask & (1u << k))) keep |= (uint64_t)0xFF << (8 * k);
      u = (u & ~keep) | (*dst & keep);
    }
    *dst = u;
  } else if (BITS == 4 && mask == 0xFFu) {
    // a whole group: gather the even slots' and the odd slots' bytes, fold
    // each byte pair into one byte (slot codes < 16), and take bytes 0 and 2
    // of both: nibbles 0-3 = slots 0, 2, 4, 6 and nibbles 4-7 = slots 1, 3,
    // 5, 7, the order v_nibble gives
    const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
    const uint32_t ev = __builtin_amdgcn_perm(hi, lo, 0x06040200u);   // b0 b2 b4 b6
    const uint32_t od = __builtin_amdgcn_perm(hi, lo, 0x07050301u);   // b1 b3 b5 b7
    const uint32_t fe = ev | __builtin_amdgcn_alignbit(ev, ev, 4);
    const uint32_t fo = od | __builtin_amdgcn_alignbit(od, od, 4);
    reinterpret_cast<uint32_t*>(tile)[item] = __builtin_amdgcn_perm(fo, fe, 0x06040200u);
  } else {
    uint32_t w = 0, hi = 0, keep = 0, keep_hi = 0;
    constexpr int HB = BITS == 6 ? 2 : 1;          // high bits per slot
    constexpr uint32_t HM = BITS == 6 ? 3u : 1u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t v = (uint32_t)(u >> (8 * k)) & 0xFFu;
      w |= (v & 15u) << (4 * v_nibble(k));
      hi |= ((v >> 4) & HM) << (HB * v_nibble(k));
      if (!(mask & (1u << k))) {
        keep |= 15u << (4 * v_nibble(k));
        keep_hi |= HM << (HB * v_nibble(k));
      }
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile) + item;
    if (keep) w = (w & ~keep) | (*dst & keep);
    *dst = w;
    if constexpr (BITS == 5) {
      uint8_t* dh = tile + 32 * D + item;
      if (keep_hi) hi = (hi & ~keep_hi) | (*dh & keep_hi);
      *dh = (uint8_t)hi;
    }
    if constexpr (BITS == 6) {
      uint16_t* dh = reinterpret_cast<uint16_t*>(tile + 32 * D) + item;
      if (keep_hi) hi = (hi & ~keep_hi) | (*dh & keep_hi);
      *dh = (uint16_t)hi;
    }
  }
}

// Quantize the positions of block bx of [q0 & ~7, q1) (RPB per block) for
// plane pl of (b, g).  Called by all 256 threads; contains barriers.
// FAST: both planes use absmax blocks, whose codes and scales do not see the
// sign of a zero, so the rotation may take its one-instruction cross-lane
// stages (rotate_row_for_absmax); scale-and-min blocks see it in their
// minimum.
template <int D, bool FAST>
__device__ void quant_part(const AppendArgs& a, int bx, int g, int b, int pl, uint8_t* vlds) {
  constexpr int LPR = D / kBlock;
  constexpr int RPB = rows_per_block(D);   // positions per block, a multiple of 8
  constexpr int NGRP = RPB / 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = tid % LPR;
  const AppendRange rg = append_range(a, b);
  const int len = rg.len, q0 = rg.q0, q1 = rg.q1;
  const int T = a.T;
  const int blk0 = (q0 & ~7) + bx * RPB;
  if (blk0 >= q1) return;                       // uniform over the block
  const int rho = tid / LPR;
  const int p = blk0 + rho;
  const bool active = rho < RPB && p >= q0 && p < q1;
  const bool from_ring = active && p < len;     // leaving the tail (T > 0)
  const int Hkv = a.Hkv;
  const size_t unit = (size_t)b * Hkv + g;
  // slot of p's tile; positions on a page outside the pool are not stored
  const long long slot = active ? tile_slot(a.map, b, g, p / kTile) : -1LL;
  const bool store = slot >= 0;

  float x[32];
  if (active && !from_ring) {
    const size_t off = ((size_t)(b * (size_t)a.n_new + (p - len)) * Hkv + g) * D + (size_t)kBlock * j;
    load_row_block(a.src[pl], a.dtype, off, x);
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = 0.f;
  }
  // outlier channels: the rest of the vector is rotated and quantized, the
  // listed channels are stored apart (no tail with outliers)
  if (a.outl) {
    zero_masked(x, outlier_mask(a, pl, g, j));
    if (active && store && j == 0) {
      const size_t roff = ((size_t)(b * (size_t)a.n_new + (p - len)) * Hkv + g) * D;
      store_outlier_block<D>(a, pl, g, (size_t)slot, p % kTile, a.src[pl], roff);
    }
  }
  // every lane takes part in the cross-lane stages
  if (a.rotate[pl]) {
    if (a.has_signs) apply_signs(x, a.signs[j]);
    if constexpr (FAST) rotate_row_for_absmax<D>(x, lane, a.cd);
    else rotate_row<D>(x, lane, a.cd);
  }
  if (T > 0) {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = bf16_round(x[e]);
  }
  if (from_ring) load_bf16_block(a.tail[pl] + (unit * T + p % T) * D + kBlock * j, x);

  const int bits = a.bits[pl];
  const bool minf = a.minf[pl] != 0;
  const size_t st = store ? (size_t)slot : 0;
  uint16_t* scales = scale_tile<D>(a, pl, st);
  uint32_t c[32];
  if (pl == 0) {
    const uint32_t s = quantize_k<D>(bits, minf, x, c, store, k_tile<D>(a, st, bits), p % kTile, j);
    if (store) store_scale<D>(scales, minf, p % kTile, j, s);
    return;
  }

  // V: codes of the block's positions meet in LDS as bytes [group][e][slot]
  const uint32_t s = quantize_any<D>(bits, minf, x, c);
  if (store) store_scale<D>(scales, minf, p % kTile, j, s);
  if (active) {
    uint8_t* dst = vlds + ((rho / 8) * D + kBlock * j) * 8 + rho % 8;
#pragma unroll
    for (int e = 0; e < 32; ++e) dst[8 * e] = (uint8_t)c[e];   // offset code
  }
  __syncthreads();

  constexpr int NN = D / 16;
  for (int it = tid; it < NGRP * D; it += 256) {
    const int grp = it / D, idx = it % D;
    const int e = 16 * (idx % NN) + idx / NN;   // consecutive threads: consecutive items
    const int p0 = blk0 + 8 * grp;
    uint32_t mask = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (p0 + k >= q0 && p0 + k < q1) mask |= 1u << k;
    if (!mask) continue;
    const long long vslot = tile_slot(a.map, b, g, p0 / kTile);
    if (vslot < 0) continue;
    const uint64_t u = *reinterpret_cast<const uint64_t*>(vlds + (grp * D + e) * 8);
    uint8_t* tile = v_tile<D>(a, (size_t)vslot, bits);
    const int item = v_item(D, p0 % kTile, e);
    if (bits == 4) store_v_item<D, 4>(tile, item, u, mask);
    else if (bits == 5) store_v_item<D, 5>(tile, item, u, mask);
    else if (bits == 6) store_v_item<D, 6>(tile, item, u, mask);
    else store_v_item<D, 8>(tile, item, u, mask);
  }
}

// Rotate the new positions of block bx of [t0, n1) and write them to their
// tail slots (plane pl of (b, g)).
template <int D>
__device__ void tail_part(const AppendArgs& a, int bx, int g, int b, int pl) {
  constexpr int LPR = D / kBlock;
  constexpr int RPB = rows_per_block(D);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = tid % LPR;
  const AppendRange rg = append_range(a, b);
  const int len = rg.len, n1 = rg.n1;
  const int T = a.T;
  const int p = rg.t0 + bx * RPB + tid / LPR;
  const bool active = tid / LPR < RPB && p < n1;
  const int Hkv = a.Hkv;

  float x[32];
  if (active) {
    const size_t off = ((size_t)(b * (size_t)a.n_new + (p - len)) * Hkv + g) * D + (size_t)kBlock * j;
    load_row_block(a.src[pl], a.dtype, off, x);
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = 0.f;
  }
  if (a.rotate[pl]) {
    if (a.has_signs) apply_signs(x, a.signs[j]);
    rotate_row<D>(x, lane, a.cd);
  }
  if (!active) return;
  const size_t unit = (size_t)b * Hkv + g;
  uint4* dst = reinterpret_cast<uint4*>(a.tail[pl] + (unit * T + p % T) * D + kBlock * j);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = f32_to_bf16_bits(x[q * 8 + 2 * k]) | (f32_to_bf16_bits(x[q * 8 + 2 * k + 1]) << 16);
    dst[q] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int D, bool FAST>
__global__ __launch_bounds__(256) void append_quant_kernel(AppendArgs a) {
  __shared__ __align__(16) uint8_t vlds[256 * kBlock];
  quant_part<D, FAST>(a, blockIdx.x, blockIdx.y, blockIdx.z >> 1, blockIdx.z & 1, vlds);
}

// Bulk quantization at head_dim 128 with absmax blocks in both planes, bf16
// inputs and no outlier channels (the common shape of a long prompt's
// append): the same arithmetic as quant_part, with the code widths fixed at
// compile time and the work in tile-aligned passes.  A block takes up to
// kBulkPasses 64-position tiles of one (sequence, KV head, plane); each pass
// is one tile, one position per four lanes, and loads the next pass's rows
// before its own arithmetic.  Whether a tile is stored, and which of its
// eight-position groups are whole, is the same for every lane, so the V
// items' masks and tile slots are scalar work.
constexpr int kBulkPasses = 4;

template <int KB, int VB>
__global__ __launch_bounds__(256) void append_bulk_kernel(AppendArgs a) {
  constexpr int D = 128, LPR = D / kBlock, NN = D / 16;
  static_assert(rows_per_block(D) == kTile, "one tile per pass");
  __shared__ __align__(16) uint8_t vlds[2][8 * D * 8];   // [pass & 1][group][e][slot]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = tid % LPR;
  const int rho = tid / LPR;                             // position within the tile
  const int g = blockIdx.y, b = blockIdx.z >> 1, pl = blockIdx.z & 1;
  const AppendRange rg = append_range(a, b);
  const int len = rg.len, q0 = rg.q0, q1 = rg.q1;
  const int T = a.T;
  const int Hkv = a.Hkv;
  const int t_first = q0 / kTile + (int)blockIdx.x * kBulkPasses;
  const int t_end = min((q1 + kTile - 1) / kTile, t_first + kBulkPasses);
  if (q1 <= q0 || t_first >= t_end) return;             // uniform
  const size_t unit = (size_t)b * Hkv + g;
  const uint16_t* src = static_cast<const uint16_t*>(a.src[pl]);
  // everything read from memory but the rows before the loop: the page
  // table and the sign masks
  long long slots[kBulkPasses];
#pragma unroll
  for (int k = 0; k < kBulkPasses; ++k) slots[k] = t_first + k < t_end ? tile_slot(a.map, b, g, t_first + k) : -1LL;
  const bool signs = a.rotate[pl] && a.has_signs;
  const uint32_t sgn = signs ? a.signs[j] : 0u;

  // Raw bf16 words of this lane's block of position t * 64 + rho.  A row
  // that is not an input row of this append (outside [len, len + n_new):
  // a tail row, or past the range) reads input row 0 or n_new - 1 instead,
  // whose values are never stored, so every load is unconditional and the
  // next pass's loads stay in flight during this pass.
  auto load = [&](int t, uint4 (&r)[4]) {
    const int ip = min(max(t * kTile + rho - len, 0), a.n_new - 1);
    const uint4* q = reinterpret_cast<const uint4*>(
        src + ((size_t)(b * (size_t)a.n_new + ip) * Hkv + g) * D + (size_t)kBlock * j);
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = q[k];
  };
  uint4 cur[4], nxt[4];
  load(t_first, cur);
#pragma unroll 1
  for (int k = 0; k < kBulkPasses; ++k) {
    const int t = t_first + k;
    if (t >= t_end) break;                               // uniform
    load(t + 1, nxt);
    const int p = t * kTile + rho;
    const bool active = p >= q0 && p < q1;
    const bool from_ring = active && p < len;           // leaving the tail (T > 0)
    long long kslot = slots[0];
#pragma unroll
    for (int i = 1; i < kBulkPasses; ++i) kslot = k == i ? slots[i] : kslot;
    float x[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w[4] = {cur[q].x, cur[q].y, cur[q].z, cur[q].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[q * 8 + 2 * i] = __uint_as_float(w[i] << 16);
        x[q * 8 + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
    if (a.rotate[pl]) {
      if (signs) {
        // a fresh copy per pass: the 32 bit masks derived from it are not
        // kept live across the unrolled passes
        uint32_t sk = sgn;
        asm volatile("" : "+v"(sk));
        apply_signs(x, sk);
      }
      rotate_row_for_absmax<D>(x, lane, a.cd);
    }
    if (T > 0) {
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] = bf16_round(x[e]);
      if (from_ring) load_bf16_block(a.tail[pl] + (unit * T + p % T) * D + kBlock * j, x);
    }
    const long long slot = kslot;                        // the same for the whole pass
    const bool store = slot >= 0;
    const size_t st = store ? (size_t)slot : 0;
    uint16_t* scales = a.scales[pl] + st * (size_t)kTile * LPR;
    uint32_t c[32];
    if (pl == 0) {
      const uint32_t s = quantize_block<KB>(x, c);
      if (store && active) {
        store_k_row<D, KB>(c, a.codes[0] + st * (size_t)kTile * padded_row_bytes(D, KB), rho, j);
        scales[rho * LPR + j] = (uint16_t)s;
      }
    } else {
      const uint32_t s = quantize_block<VB>(x, c);
      if (store && active) scales[rho * LPR + j] = (uint16_t)s;
      uint8_t* buf = vlds[k & 1];
      if (active) {
        uint8_t* dst = buf + ((rho / 8) * D + kBlock * j) * 8 + rho % 8;
#pragma unroll
        for (int e = 0; e < 32; ++e) dst[8 * e] = (uint8_t)c[e];   // offset code
      }
      // the buffer of pass k was last read in pass k - 2, before the
      // barrier of pass k - 1
      __syncthreads();
      if (store) {
        uint8_t* tile = a.codes[1] + st * (size_t)v_tile_bytes(D, VB);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int it = tid + 256 * i;
          const int grp = __builtin_amdgcn_readfirstlane(it / D);   // the same for a wave
          const int idx = it % D;
          const int e = 16 * (idx % NN) + idx / NN;
          const int p0 = t * kTile + 8 * grp;
          const int lo = max(q0 - p0, 0), hi = min(q1 - p0, 8);
          if (lo >= hi) continue;
          const uint32_t mask = (0xFFu >> (8 - hi)) & (0xFFu << lo);
          const uint64_t u = *reinterpret_cast<const uint64_t*>(buf + (grp * D + e) * 8);
          store_v_item<D, VB>(tile, v_item(D, 8 * grp, e), u, mask);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
  }
}

template <int D>
__global__ __launch_bounds__(256) void append_tail_kernel(AppendArgs a) {
  tail_part<D>(a, blockIdx.x, blockIdx.y, blockIdx.z >> 1, blockIdx.z & 1);
}

// Appends small enough for one block per (b, g, plane): quantize, then (after
// a barrier, so every displaced slot has been read) write the tail.
template <int D, bool FAST>
__global__ __launch_bounds__(256) void append_small_kernel(AppendArgs a) {
  __shared__ __align__(16) uint8_t vlds[256 * kBlock];
  const int g = blockIdx.y, b = blockIdx.z >> 1, pl = blockIdx.z & 1;
  quant_part<D, FAST>(a, 0, g, b, pl, vlds);
  __syncthreads();
  if (a.T > 0) tail_part<D>(a, 0, g, b, pl);
}

// One new token per sequence (a decode step), one wave per (b, g, plane):
// append_one_load and append_one_finish, shared with the fused decode step.
template <int D, int VB, bool FAST>
__global__ __launch_bounds__(64) void append_one_kernel(AppendArgs a) {
  const OneArgs o = one_args(a);
  OneLoads L;
  append_one_load<D, VB>(o, blockIdx.x, blockIdx.y, blockIdx.z, a.len[blockIdx.y], true, L);
  append_one_finish<D, VB, FAST>(o, blockIdx.x, blockIdx.y, blockIdx.z, a.len[blockIdx.y], true, L, nullptr,
                                 nullptr);
}

template <int KB>
void launch_bulk_k(const AppendArgs& a, dim3 grid, hipStream_t s) {
  switch (a.bits[1]) {
    case 4: hipLaunchKernelGGL((append_bulk_kernel<KB, 4>), grid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL((append_bulk_kernel<KB, 5>), grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL((append_bulk_kernel<KB, 6>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((append_bulk_kernel<KB, 8>), grid, dim3(256), 0, s, a); break;
  }
}
// Grid of append_bulk_kernel: enough blocks of kBulkPasses tiles for the
// sequence whose quantized range spans the most tiles.
void launch_bulk(const AppendArgs& a, int B, hipStream_t s) {
  int tiles = 0;
  for (int b = 0; b < B; ++b) {
    const int len = a.len[b], n1 = len + a.n_new;
    const int q0 = a.T > 0 ? max(0, len - a.T) : len;
    const int q1 = a.T > 0 ? max(0, n1 - a.T) : n1;
    if (q1 > q0) tiles = max(tiles, (q1 + kTile - 1) / kTile - q0 / kTile);
  }
  const dim3 grid((tiles + kBulkPasses - 1) / kBulkPasses, a.Hkv, 2 * B);
  switch (a.bits[0]) {
    case 4: launch_bulk_k<4>(a, grid, s); break;
    case 5: launch_bulk_k<5>(a, grid, s); break;
    case 6: launch_bulk_k<6>(a, grid, s); break;
    default: launch_bulk_k<8>(a, grid, s); break;
  }
}

template <int D>
hipError_t launch_append_d(const AppendArgs& a, int B, hipStream_t s) {
  constexpr int RPB = rows_per_block(D);
  const bool absmax = !a.minf[0] && !a.minf[1];
  if (a.n_new == 1) {
    const dim3 grid(a.Hkv, B, 2), block(64);
    if (absmax && a.T == 0) {
      switch (a.bits[1]) {
        case 4: hipLaunchKernelGGL((append_one_kernel<D, 4, true>), grid, block, 0, s, a); break;
        case 5: hipLaunchKernelGGL((append_one_kernel<D, 5, true>), grid, block, 0, s, a); break;
        case 6: hipLaunchKernelGGL((append_one_kernel<D, 6, true>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((append_one_kernel<D, 8, true>), grid, block, 0, s, a); break;
      }
    } else {
      switch (a.bits[1]) {
        case 4: hipLaunchKernelGGL((append_one_kernel<D, 4, false>), grid, block, 0, s, a); break;
        case 5: hipLaunchKernelGGL((append_one_kernel<D, 5, false>), grid, block, 0, s, a); break;
        case 6: hipLaunchKernelGGL((append_one_kernel<D, 6, false>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((append_one_kernel<D, 8, false>), grid, block, 0, s, a); break;
      }
    }
    return hipGetLastError();
  }
  if (a.n_new <= RPB - 7) {
    // [q0 & ~7, q1) spans at most n_new + 7 positions and the tail at most n_new
    if (absmax) hipLaunchKernelGGL((append_small_kernel<D, true>), dim3(1, a.Hkv, 2 * B), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((append_small_kernel<D, false>), dim3(1, a.Hkv, 2 * B), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  int quant_blocks = 0;
  for (int b = 0; b < B; ++b) {
    const int len = a.len[b], n1 = len + a.n_new;
    const int q0 = a.T > 0 ? max(0, len - a.T) : len;
    const int q1 = a.T > 0 ? max(0, n1 - a.T) : n1;
    if (q1 > q0) quant_blocks = max(quant_blocks, (q1 - (q0 & ~7) + RPB - 1) / RPB);
  }
  bool bulk = false;
  if constexpr (D == 128) bulk = absmax && a.dtype == KVQ_BF16 && a.outl == 0;
  if (quant_blocks > 0 && bulk) {
    launch_bulk(a, B, s);
  } else if (quant_blocks > 0) {
    const dim3 grid(quant_blocks, a.Hkv, 2 * B);
    if (absmax) hipLaunchKernelGGL((append_quant_kernel<D, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((append_quant_kernel<D, false>), grid, dim3(256), 0, s, a);
  }
  const int n_tail = a.T > 0 ? min(a.n_new, a.T) : 0;
  if (n_tail > 0)
    hipLaunchKernelGGL(append_tail_kernel<D>, dim3((n_tail + RPB - 1) / RPB, a.Hkv, 2 * B),
                       dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int D, const AppendArgs& a, int B, hipStream_t s) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  switch (D) {
    case 64: return launch_append_d<64>(a, B, s);
    case 128: return launch_append_d<128>(a, B, s);
    case 192: return launch_append_d<192>(a, B, s);
    case 256: return launch_append_d<256>(a, B, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
