// Internal interface between the host library and the kernel translation
// units: argument blocks passed by value to the kernels, and launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "kvq.h"

namespace kvq {

// ---------------------------------------------------------------- append
struct AppendArgs {
  const void* src[2];        // k_new, v_new: [B][n_new][Hkv][D]
  uint8_t* codes[2];         // tiled code planes
  uint16_t* scales[2];       // [B][Hkv][cap][D/32] fp16 bits ([..][D/32][2] (s, m) with minf)
  uint16_t* tail[2];         // [B][Hkv][T][D] bf16 bits (unused when T == 0)
  int32_t bits[2];
  int32_t minf[2];           // 1: scale-and-min blocks (4/5-bit only)
  int32_t rotate[2];
  int32_t Hkv, n_new, T, cap, dtype;
  TileMap map;               // tile slots of the code and scale planes
  float cd;                  // fp32(1/sqrt(D))
  int32_t has_signs;         // rotate by H diag(s): flip element e's sign by bit e of signs
  uint32_t signs[8];
  // outlier channels: outl (0 or 32) channels per plane and KV head, listed
  // in out_idx [2][Hkv][outl]; their 8-bit codes and fp16 scales
  int32_t outl;
  const int32_t* out_idx;
  uint8_t* out_codes[2];     // K: [tile][64][32] bytes; V: element-major 8-bit tiles
  uint16_t* out_scales[2];   // [tile][64]
  int32_t len[KVQ_MAX_BATCH];  // lengths before the append
};
hipError_t launch_append(int D, const AppendArgs& a, int B, hipStream_t s);

// Channels of an outlier set (one 32-element block).
constexpr int kOutl = 32;
// Entry o of an outlier list; an entry outside [0, D) reads channel 0 in its
// place (results unspecified; every access stays inside the head vector).
__device__ inline int outlier_channel(const int32_t* list, int o, int D) {
  const int ch = list[o];
  return (unsigned)ch < (unsigned)D ? ch : 0;
}

// What the one-token append of a decode step reads (AppendArgs without the
// lengths, which the caller passes): the fused decode step carries it in its
// own arguments.
struct OneArgs {
  const void* src[2];        // k_new, v_new: [B][1][Hkv][D]
  uint8_t* codes[2];
  uint16_t* scales[2];
  uint16_t* tail[2];
  int32_t bits[2];
  int32_t minf[2];
  int32_t rotate[2];
  int32_t Hkv, T, dtype;
  TileMap map;
  float cd;
  int32_t has_signs;
  uint32_t signs[8];
  int32_t outl;
  const int32_t* out_idx;
  uint8_t* out_codes[2];
  uint16_t* out_scales[2];
};
__host__ __device__ inline OneArgs one_args(const AppendArgs& a) {
  OneArgs o;
  for (int p = 0; p < 2; ++p) {
    o.src[p] = a.src[p];
    o.codes[p] = a.codes[p];
    o.scales[p] = a.scales[p];
    o.tail[p] = a.tail[p];
    o.bits[p] = a.bits[p];
    o.minf[p] = a.minf[p];
    o.rotate[p] = a.rotate[p];
  }
  o.Hkv = a.Hkv;
  o.T = a.T;
  o.dtype = a.dtype;
  o.map = a.map;
  o.cd = a.cd;
  o.has_signs = a.has_signs;
  for (int i = 0; i < 8; ++i) o.signs[i] = a.signs[i];
  o.outl = a.outl;
  o.out_idx = a.out_idx;
  for (int p = 0; p < 2; ++p) {
    o.out_codes[p] = a.out_codes[p];
    o.out_scales[p] = a.out_scales[p];
  }
  return o;
}

// ------------------------------------------------------------- dequantize
struct DequantArgs {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* tail;
  float* out;                // [t1-t0][Hkv][D]
  int32_t which;              // 0 = K (row layout), 1 = V (element-major tiles)
  int32_t bits, rotate, space, Hkv, T, cap, b, t0, t1, nq;
  int32_t minf;              // scale-and-min blocks: (s, m) pairs, x = u * s + m
  TileMap map;
  float cd;
  int32_t has_signs;         // space 1 rotates back by diag(s) H
  uint32_t signs[8];
  int32_t outl;              // outlier channels: added back in space 1
  const uint8_t* out_codes;
  const uint16_t* out_scales;
  const int32_t* out_idx;    // this plane's lists [Hkv][outl]
};
hipError_t launch_dequant(int D, const DequantArgs& a, hipStream_t s);

// ---------------------------------------------------------------- decode
// Resident waves per SIMD the split-K kernel is built for, by head_dim.
// A wave holds two 32-token steps of cache bytes and D/16 accumulator tiles
// in registers: at d <= 128 that fits the 256 registers of two waves per
// SIMD; at d = 256 it needs about 300, which one wave per SIMD (512
// registers, half of them AGPRs) allows.
// At d = 192 two waves per SIMD fit the absmax decode variants (about 250
// registers); variants with scale-and-min blocks or prefill rows ("wide")
// need more and run at one wave per SIMD too.
constexpr int split_waves_per_simd(int D, bool wide = false) {
  return D >= 256 || (D == 192 && wide) ? 1 : 2;
}
// Waves per workgroup: one workgroup fills a compute unit's four SIMDs at
// that occupancy.  The waves of a workgroup share one contiguous range of a
// unit's quantized tiles and take them from an LDS counter; the split count
// S is a multiple of this.
constexpr int split_group_waves(int D, bool wide = false) { return 4 * split_waves_per_simd(D, wide); }

struct DecodeArgs {
  const uint8_t* k_codes;
  const uint16_t* k_scales;
  const uint8_t* v_codes;
  const uint16_t* v_scales;
  const uint16_t* k_tail;
  const uint16_t* v_tail;
  const void* q;             // [B][Hq][D] bf16 or float32, original space
  float* part_ml;            // [B][Hq][S][2]  running max (log2 units), sum
  float* part_acc;           // [B][Hq][S][D]  unnormalised output, rotated space
  int32_t Hkv, Hq, G, n_gchunks, T, cap, S;
  TileMap map;               // tile slots of the code and scale planes
  int32_t n_q, n_rb;         // prefill: queries per sequence, 64-row blocks per KV head
  int32_t q_dtype, rotate_k;
  float cd, sm_scale;        // fp32(1/sqrt(D)); softmax scale
  int32_t has_signs;         // q is rotated by H diag(s) (signs as in AppendArgs)
  uint32_t signs[8];
  // fused decode step: the launch also appends one token per sequence (the
  // lengths below then count it); step_on 0: plain decode over the cache
  int32_t step_on;
  OneArgs step;
  // outlier channels (the OUT kernels): codes and scales of K's and V's
  // outlier planes, the lists [2][Hkv][32], partial sums [B][Hq][S][32]
  const uint8_t* out_codes[2];
  const uint16_t* out_scales[2];
  const int32_t* out_idx;
  float* part_out;
  int32_t len[KVQ_MAX_BATCH];
};
// t0, t1: when non-null, events that take the kernel's own start and end
// times (the instrumentation of kvq_profile_decode_events).
using DecodeLauncher = hipError_t (*)(const DecodeArgs&, dim3, hipStream_t, hipEvent_t t0, hipEvent_t t1);
// Page modes of the split kernel: tiles found at run time in contiguous or
// paged planes (kPageAny), or fixed at compile time.  head_dim 256 builds
// kPageFlat and kPagePaged: its two-tile pipeline fills the register file,
// and carrying both layouts spilled a tile address into the loop.
constexpr int kPageAny = 0, kPageFlat = 1, kPagePaged = 2;
constexpr bool split_fixed_layout(int D) { return D == 256; }
// Table lookup for (D, k_bits, v_bits, heads per chunk, K / V scale-and-min
// blocks, paged planes); nullptr if absent.
DecodeLauncher decode_launcher(int D, int kb, int vb, int gc, bool km, bool vm, bool paged,
                               bool outliers = false);
// The prefill variant of the split kernel for (D, k_bits, v_bits, km, vm, paged).
DecodeLauncher prefill_launcher(int D, int kb, int vb, bool km, bool vm, bool paged);

// ------------------------------------------------------- prefill (matrix)
// Chunked prefill on the matrix cores at head_dim 128 with absmax blocks:
// query rows prepared once (rotated, scaled to log2 units, split into fp16
// hi + lo parts), then per workgroup of kPrefillRows rows of one KV head
// (eight waves) the cache tiles are dequantized once into double-buffered
// LDS and both products run as 32x32x16 f16 matrix-core steps.  Partials as
// the split kernel's.
constexpr int kPrefillRows = 256;
struct PrefillArgs {
  const uint8_t* k_codes;
  const uint16_t* k_scales;
  const uint8_t* v_codes;
  const uint16_t* v_scales;
  const uint16_t* k_tail;
  const uint16_t* v_tail;
  const void* q;             // [B][n_q][Hq][D] bf16 or float32, original space
  uint16_t* q_hi;            // prepared rows [B][Hkv][rows_pad][D], fp16 bits
  uint16_t* q_lo;
  float* q_w;                // [B][Hkv][rows_pad]: 2^-f of each prepared row
  float* part_ml;            // [B][n_q][Hq][S][2]
  float* part_acc;           // [B][n_q][Hq][S][D], rotated space
  int32_t Hkv, Hq, G, T, S, n_q, n_rb, rows_pad;
  TileMap map;
  int32_t q_dtype, rotate_k;
  float cd, sm_scale;
  int32_t has_signs;
  uint32_t signs[8];
  int32_t len[KVQ_MAX_BATCH];
};
// Whether the matrix-core prefill covers a configuration.
constexpr bool prefill_mfma_supported(int D, int kb, int vb, bool km, bool vm) {
  return D == 128 && !km && !vm && (kb == 4 || kb == 5 || kb == 6 || kb == 8) &&
         (vb == 4 || vb == 5 || vb == 6 || vb == 8);
}
// Query preparation (grid: rows_pad / 64, Hkv, B), then the attention
// kernel (grid: S, n_rb * Hkv, B).
hipError_t launch_prefill_q(const PrefillArgs& a, int kb, int B, hipStream_t s);
hipError_t launch_prefill_mfma(const PrefillArgs& a, int kb, int vb, int B, hipStream_t s,
                               hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

// Largest split count the host schedules (bounds the combine kernel's LDS).
constexpr int kMaxSplitsDevice = 1024;

struct CombineArgs {
  const float* part_ml;
  const float* part_acc;
  float* out;                // [B][Hq][D]
  int32_t Hq, S, rotate;
  float cd;
  int32_t has_signs;         // rotate back by diag(s) H
  uint32_t signs[8];
  const float* part_out;     // outlier channels' partials [B][Hq][S][32], or null
  const int32_t* v_out_idx;  // V's outlier lists [Hkv][32]
  int32_t G;                 // query heads per KV head
};
hipError_t launch_combine(int D, const CombineArgs& a, int B, hipStream_t s);

}  // namespace kvq
