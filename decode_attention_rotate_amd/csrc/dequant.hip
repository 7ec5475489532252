// Dequantize (read-back) kernel: code * fp16 scale for quantized positions
// (level * scale + minimum for scale-and-min blocks), the stored bf16 value for tail positions, optionally rotated back to the
// original space with the same float32 transform as the append (the
// normalized Sylvester matrix is its own inverse; velog.io post "fix KV cache
// quantization outliers", section "Hadamard rotation").
//
// K codes are read from their row layout, V codes from the element-major
// tiles.  Thread mapping as in the append: one lane per 32-element block.
#include "common.hpp"
#include "kernels.hpp"

namespace kvq {
namespace {

// V codes of elements 32j..32j+31 of token p from the element-major tiles.
template <int D, int BITS>
__device__ inline void load_v_codes(const uint8_t* plane, int p, int j, int (&c)[32]) {
  constexpr int OFF = 1 << (BITS - 1);
  const uint8_t* tile = plane + (size_t)(p / kTile) * v_tile_bytes(D, BITS);
  const int t = p % kTile, k = t % 8;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int item = v_item(D, t, kBlock * j + i);
    int u;
    if constexpr (BITS == 8) {
      u = tile[item * 8 + k];
    } else {
      const uint32_t w = reinterpret_cast<const uint32_t*>(tile)[item];
      u = (int)((w >> (4 * v_nibble(k))) & 15u);
      if constexpr (BITS == 5) u |= (int)((tile[32 * D + item] >> v_nibble(k)) & 1u) << 4;
      if constexpr (BITS == 6)
        u |= (int)((reinterpret_cast<const uint16_t*>(tile + 32 * D)[item] >> (2 * v_nibble(k))) & 3u) << 4;
    }
    c[i] = u - OFF;
  }
}

template <int D>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  constexpr int LPR = D / kBlock;
  constexpr int RPB = rows_per_block(D);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = tid % LPR;
  const int g = blockIdx.y;
  const int p = a.t0 + blockIdx.x * RPB + tid / LPR;
  const bool active = tid / LPR < RPB && p < a.t1;
  const size_t unit = (size_t)a.b * a.Hkv + g;
  // outlier channels (space 1): the block's outlier values, and the list
  // slot of each channel (-1: not an outlier), in LDS
  __shared__ float oval[RPB][kOutl];
  __shared__ int inv[D];
  const bool outl = a.outl && a.space == 1;   // uniform
  if (outl) {
    for (int i = tid; i < D; i += 256) inv[i] = -1;
    __syncthreads();
    if (tid < kOutl) inv[outlier_channel(a.out_idx + (size_t)g * kOutl, tid, D)] = tid;
    for (int it = tid; it < RPB * kOutl; it += 256) {
      const int r = it / kOutl, o = it % kOutl;
      const int pp = a.t0 + blockIdx.x * RPB + r;
      float v = 0.f;
      if (pp < a.t1 && pp < a.nq) {
        const size_t slot = tile_slot_read(a.map, a.b, g, pp / kTile);
        const int l = pp % kTile;
        const float s = (float)__builtin_bit_cast(_Float16, a.out_scales[slot * kTile + l]);
        const uint8_t* tile = a.out_codes + slot * kTile * kOutl;
        const int c = a.which == 0 ? (int)(int8_t)tile[l * kOutl + o]
                                   : (int)tile[8 * v_item(kOutl, l, o) + l % 8] - 128;
        v = (float)c * s;
      }
      oval[r][o] = v;
    }
    __syncthreads();
  }
  float x[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) x[e] = 0.f;
  if (active) {
    if (p < a.nq) {
      // p's tile in the contiguous or paged planes; l is p's place in it
      const size_t slot = tile_slot_read(a.map, a.b, g, p / kTile);
      const int l = p % kTile;
      const size_t srow = slot * kTile + l;
      float s, mn = 0.f;
      if (a.minf) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(a.scales)[srow * (D / kBlock) + j];
        s = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
        mn = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
      } else {
        s = (float)__builtin_bit_cast(_Float16, a.scales[srow * (D / kBlock) + j]);
      }
      int c[32];
      if (a.which == 0) {
        const uint8_t* tile = a.codes + slot * kTile * padded_row_bytes(D, a.bits);
        if (a.bits == 4) load_codes<D, 4>(tile, l, j, c);
        else if (a.bits == 5) load_codes<D, 5>(tile, l, j, c);
        else if (a.bits == 6) load_codes<D, 6>(tile, l, j, c);
        else load_codes<D, 8>(tile, l, j, c);
      } else {
        const uint8_t* tile = a.codes + slot * v_tile_bytes(D, a.bits);
        if (a.bits == 4) load_v_codes<D, 4>(tile, l, j, c);
        else if (a.bits == 5) load_v_codes<D, 5>(tile, l, j, c);
        else if (a.bits == 6) load_v_codes<D, 6>(tile, l, j, c);
        else load_v_codes<D, 8>(tile, l, j, c);
      }
      if (a.minf) {
        // level u = c + 2^(bits-1); u * s is exact, one rounding in the add
        const int off = 1 << (a.bits - 1);
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = (float)(c[e] + off) * s + mn;
      } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = (float)c[e] * s;
      }
    } else {
      const uint16_t* row = a.tail + (unit * a.T + p % a.T) * D + kBlock * j;
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] = bf16_to_f32(row[e]);
    }
  }
  if (a.space == 1 && a.rotate) {
    rotate_row<D>(x, lane, a.cd);
    if (a.has_signs) apply_signs(x, a.signs[j]);   // back by diag(s) H
  }
  if (!active) return;
  if (outl) {
    const int r = tid / LPR;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int k = inv[kBlock * j + e];
      if (k >= 0) x[e] = x[e] + oval[r][k];
    }
  }
  float4* dst = reinterpret_cast<float4*>(a.out + ((size_t)(p - a.t0) * a.Hkv + g) * D + kBlock * j);
#pragma unroll
  for (int q = 0; q < 8; ++q) dst[q] = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
}

}  // namespace

hipError_t launch_dequant(int D, const DequantArgs& a, hipStream_t s) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  const int rpb = rows_per_block(D);
  const int n = a.t1 - a.t0;
  if (n <= 0) return hipSuccess;
  const dim3 grid((n + rpb - 1) / rpb, a.Hkv, 1);
  switch (D) {
    case 64: hipLaunchKernelGGL(dequant_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(dequant_kernel<128>, grid, dim3(256), 0, s, a); break;
    case 192: hipLaunchKernelGGL(dequant_kernel<192>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(dequant_kernel<256>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
