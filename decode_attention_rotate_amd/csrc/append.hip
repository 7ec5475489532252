// Rotate-quantize-append kernel.
//
// Each new K/V head vector is rotated by the normalized Hadamard matrix
// (velog.io post "fix KV cache quantization outliers", section "Hadamard
// rotation") and either quantized into 32-element blocks with one fp16 absmax
// scale (byte cost per the aiwitness.kr table "Qwen 3.6 27B Q5_K_S + 64k
// context KLD results") or, for the newest tail_len positions, stored in the
// bf16 precision tail (aitrends.kr article 92204, glossary "Precision Tail").
//
// Thread mapping: one lane per 32-element block, D/32 consecutive lanes per
// head vector, so a 256-thread block covers 256*32/D consecutive tokens of one
// (sequence, KV head, plane).  The in-lane butterfly stages h = 1..16 run in
// registers, the remaining stages cross lanes with DPP / ds_swizzle, and the
// block absmax and the codes never leave the lane.
//
// Tail ring: a new tail token at position p goes to slot p % T; the token it
// displaces (if it is leaving the tail in this call) is read and quantized by
// the same thread first, so no slot is read after it is overwritten.
#include "common.hpp"
#include "kernels.hpp"

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

// Quantize block j of the row of position p and store codes and scale.
template <int D, int BITS>
__device__ inline void quantize_store(const float (&x)[32], uint8_t* plane, uint16_t* scale_row,
                                      int p, int j) {
  constexpr int RP = padded_row_bytes(D, BITS);
  int c[32];
  scale_row[j] = (uint16_t)quantize_block<BITS>(x, c);
  if constexpr (BITS == 8) {
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = (uint32_t)(c[4 * k] & 0xFF) | ((uint32_t)(c[4 * k + 1] & 0xFF) << 8) |
             ((uint32_t)(c[4 * k + 2] & 0xFF) << 16) | ((uint32_t)(c[4 * k + 3] & 0xFF) << 24);
    *reinterpret_cast<uint4*>(plane + chunk_offset(p, 2 * j, RP)) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(plane + chunk_offset(p, 2 * j + 1, RP)) = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    constexpr int OFF = 1 << (BITS - 1);
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t v = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) v |= (uint32_t)((c[8 * k + e] + OFF) & 15) << (4 * e);
      w[k] = v;
    }
    *reinterpret_cast<uint4*>(plane + chunk_offset(p, j, RP)) = make_uint4(w[0], w[1], w[2], w[3]);
    if constexpr (BITS == 5) {
      uint32_t hw = 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) hw |= (uint32_t)(((c[e] + OFF) >> 4) & 1) << hibit_pos(e);
      const int byte = D / 2 + 4 * j;
      *reinterpret_cast<uint32_t*>(plane + chunk_offset(p, byte / kChunk, RP) + byte % kChunk) = hw;
    }
  }
}

template <int D>
__device__ inline void quantize_store_bits(int bits, const float (&x)[32], uint8_t* plane,
                                           uint16_t* scale_row, int p, int j) {
  if (bits == 4) quantize_store<D, 4>(x, plane, scale_row, p, j);
  else if (bits == 5) quantize_store<D, 5>(x, plane, scale_row, p, j);
  else quantize_store<D, 8>(x, plane, scale_row, p, j);
}

template <int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int LPR = D / kBlock;
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = tid % LPR;
  const int g = blockIdx.y;
  const int b = blockIdx.z >> 1;
  const int pl = blockIdx.z & 1;
  const int i = blockIdx.x * RPB + tid / LPR;
  const bool active = i < a.n_new;
  const int len = a.len[b];
  const int T = a.T;
  const int n1 = len + a.n_new;
  const int q_end = T > 0 ? n1 - T : n1;
  const int Hkv = a.Hkv;

  float x[32];
  if (active) {
    const size_t off = ((size_t)(b * (size_t)a.n_new + i) * Hkv + g) * D + (size_t)kBlock * j;
    load_row_block(a.src[pl], a.dtype, off, x);
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = 0.f;
  }
  // every lane takes part in the cross-lane stages
  if (a.rotate[pl]) rotate_row<D>(x, lane, a.cd);
  if (T > 0) {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = bf16_round(x[e]);
  }
  if (!active) return;

  const size_t unit = (size_t)b * Hkv + g;
  const int bits = a.bits[pl];
  uint8_t* plane = a.codes[pl] + unit * (size_t)a.cap * padded_row_bytes(D, bits);
  uint16_t* scales = a.scales[pl] + unit * (size_t)a.cap * (D / kBlock);
  const int p = len + i;
  if (p < q_end) {
    quantize_store_bits<D>(bits, x, plane, scales + (size_t)p * (D / kBlock), p, j);
    return;
  }
  const int slot = p % T;
  uint16_t* tail_row = a.tail[pl] + (unit * T + slot) * D + kBlock * j;
  const int o0 = len > T ? len - T : 0;
  const int pg = o0 + (slot - o0 % T + T) % T;   // old occupant of the slot
  if (pg < len && pg < q_end) {
    float y[32];
    const uint4* src = reinterpret_cast<const uint4*>(tail_row);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = src[q];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[q * 8 + 2 * k] = __uint_as_float(w[k] << 16);
        y[q * 8 + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
    quantize_store_bits<D>(bits, y, plane, scales + (size_t)pg * (D / kBlock), pg, j);
  }
  uint4* dst = reinterpret_cast<uint4*>(tail_row);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = f32_to_bf16_bits(x[q * 8 + 2 * k]) | (f32_to_bf16_bits(x[q * 8 + 2 * k + 1]) << 16);
    dst[q] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_append(int D, const AppendArgs& a, int B, hipStream_t s) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  const int rpb = 256 / (D / kBlock);
  const dim3 grid((a.n_new + rpb - 1) / rpb, a.Hkv, 2 * B);
  switch (D) {
    case 64: hipLaunchKernelGGL(append_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(append_kernel<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(append_kernel<256>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
