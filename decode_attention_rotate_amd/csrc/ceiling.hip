// Read-bandwidth ceilings of the part, for judging the split-K decode
// kernel's HBM rate against what plain reads reach (measurement only; the
// attention path never calls these).
//
//  * stream: a linear read of a buffer with 16-byte loads, UNROLL loads per
//    lane in flight before the first is consumed, grid-stride over the
//    buffer, optionally with non-temporal loads.
//  * tiles: the split kernel's access pattern without its arithmetic: per
//    (sequence, KV head) unit, S waves in workgroups of 8 take contiguous
//    ranges of 64-token tiles (or chunks of 8 tiles dealt round-robin) and
//    pull tiles from an LDS counter; each tile is its K codes, V codes, K
//    scales and V scales (four separate planes), read with 16-byte loads
//    (optionally non-temporal), AHEAD tiles loaded before the first is used.
// Both fold what they read into an XOR per lane, written to `sink`, so no
// load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4* __restrict__ p, size_t n16,
                                                     uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

struct TileLoads {
  static constexpr int kMax = 16;   // 16-byte loads per lane per tile, at most
};

template <int AHEAD, bool NT, bool CHUNKED>
__global__ __launch_bounds__(512) void tiles_kernel(kvq_ceiling_tiles_args a, uint32_t* __restrict__ sink) {
  __shared__ uint32_t ctr;
  if (threadIdx.x == 0) ctr = 0u;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const size_t unit = blockIdx.y;
  const int NG = (int)gridDim.x;
  const int t0 = (int)((int64_t)a.tiles * blockIdx.x / NG), t1 = (int)((int64_t)a.tiles * (blockIdx.x + 1) / NG);
  const int kl = a.k_tile_bytes / 1024, vl = a.v_tile_bytes / 1024;   // loads per lane
  const char* kp = static_cast<const char*>(a.k_codes) + unit * (size_t)a.tiles * a.k_tile_bytes;
  const char* vp = static_cast<const char*>(a.v_codes) + unit * (size_t)a.tiles * a.v_tile_bytes;
  const char* ksp = static_cast<const char*>(a.k_scales) + unit * (size_t)a.tiles * a.s_tile_bytes;
  const char* vsp = static_cast<const char*>(a.v_scales) + unit * (size_t)a.tiles * a.s_tile_bytes;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 buf[AHEAD][TileLoads::kMax + 1];
  // CHUNKED: the unit's tiles go in chunks of 8 dealt round-robin to its NG
  // workgroups (chunk c to workgroup c % NG), so at any time the workgroups
  // of a unit read neighbouring chunks; otherwise each workgroup owns the
  // contiguous range [t0, t1).
  const int tend = CHUNKED ? a.tiles : t1;
  auto grab = [&]() {
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(&ctr, 1u);
    const int c = (int)__builtin_amdgcn_readfirstlane(v);
    return CHUNKED ? ((c >> 3) * NG + (int)blockIdx.x) * 8 + (c & 7) : t0 + c;
  };
  auto ld = [&](const u32x4* p) { return NT ? __builtin_nontemporal_load(p) : *p; };
  auto load = [&](u32x4 (&r)[TileLoads::kMax + 1], int t) {
    const u32x4* k = reinterpret_cast<const u32x4*>(kp + (size_t)t * a.k_tile_bytes) + lane;
    const u32x4* v = reinterpret_cast<const u32x4*>(vp + (size_t)t * a.v_tile_bytes) + lane;
#pragma unroll
    for (int i = 0; i < TileLoads::kMax; ++i) {
      if (i < kl) r[i] = ld(k + 64 * i);
      else if (i - kl < vl) r[i] = ld(v + 64 * (i - kl));
    }
    // scale rows: lanes 0..31 read K's, 32..63 V's (s_tile_bytes <= 512)
    const char* s = lane < 32 ? ksp : vsp;
    const int sl = lane & 31;
    r[TileLoads::kMax] = 16 * sl < a.s_tile_bytes
                             ? ld(reinterpret_cast<const u32x4*>(s + (size_t)t * a.s_tile_bytes + 16 * sl))
                             : u32x4{0u, 0u, 0u, 0u};
  };
  auto fold = [&](const u32x4 (&r)[TileLoads::kMax + 1]) {
#pragma unroll
    for (int i = 0; i < TileLoads::kMax; ++i)
      if (i < kl + vl) acc ^= r[i];
    acc ^= r[TileLoads::kMax];
  };
  int tn[AHEAD];
#pragma unroll
  for (int k = 0; k < AHEAD; ++k) {
    tn[k] = grab();
    if (tn[k] < tend) load(buf[k], tn[k]);
  }
  while (true) {
    bool any = false;
#pragma unroll
    for (int k = 0; k < AHEAD; ++k) {
      if (tn[k] < tend) {
        any = true;
        fold(buf[k]);
        tn[k] = grab();
        if (tn[k] < tend) load(buf[k], tn[k]);
      }
    }
    if (!any) break;
  }
  sink[((size_t)blockIdx.y * gridDim.x + blockIdx.x) * 512 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

int kvq_ceiling_stream(const void* buf, size_t bytes, int32_t blocks, int32_t unroll, int32_t nontemporal,
                       uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || blocks < 1 || (reinterpret_cast<uintptr_t>(buf) & 15u)) return -1;
  const u32x4* p = static_cast<const u32x4*>(buf);
  const size_t n16 = bytes / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
#define KVQ_STREAM(U)                                                                         \
  if (unroll == U) {                                                                          \
    if (nontemporal) hipLaunchKernelGGL((stream_kernel<U, true>), dim3(blocks), dim3(256), 0, s, p, n16, sink); \
    else hipLaunchKernelGGL((stream_kernel<U, false>), dim3(blocks), dim3(256), 0, s, p, n16, sink);            \
    return hipGetLastError() == hipSuccess ? 0 : -5;                                          \
  }
  KVQ_STREAM(1)
  KVQ_STREAM(4)
  KVQ_STREAM(8)
  KVQ_STREAM(16)
#undef KVQ_STREAM
  return -1;
}

int kvq_ceiling_tiles(const kvq_ceiling_tiles_args* args, int32_t splits, int32_t ahead, int32_t mode,
                      uint32_t* sink, void* stream) {
  if (!args || !sink || splits < 1 || args->units < 1 || args->units > 65535 || args->tiles < 1) return -1;
  const kvq_ceiling_tiles_args& a = *args;
  if (a.k_tile_bytes % 1024 || a.v_tile_bytes % 1024 || a.k_tile_bytes / 1024 + a.v_tile_bytes / 1024 > 16 ||
      a.s_tile_bytes < 16 || a.s_tile_bytes > 512 || a.s_tile_bytes % 16)
    return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(splits, a.units);
  if (mode < 0 || mode > 3 || (ahead != 1 && ahead != 2)) return -1;
  (void)hipGetLastError();
#define KVQ_TILES(A, M)                                                                              \
  if (ahead == A && mode == M) hipLaunchKernelGGL((tiles_kernel<A, (M & 1) != 0, (M & 2) != 0>), grid, \
                                                  dim3(512), 0, s, a, sink);
  KVQ_TILES(1, 0) KVQ_TILES(1, 1) KVQ_TILES(1, 2) KVQ_TILES(1, 3)
  KVQ_TILES(2, 0) KVQ_TILES(2, 1) KVQ_TILES(2, 2) KVQ_TILES(2, 3)
#undef KVQ_TILES
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

size_t kvq_ceiling_sink_words(int32_t blocks_or_splits, int32_t units) {
  return (size_t)blocks_or_splits * (units > 0 ? units : 1) * 512;
}

}  // extern "C"
