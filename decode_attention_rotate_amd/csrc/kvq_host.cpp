// Host side of the kvq C ABI: argument validation, sizing of cache planes and
// of the decode workspace, split-K scheduling and kernel launches.
//
// Configuration rules: K and V widths are independent (velog.io post "fix KV
// cache quantization outliers", section "the essence of the problem", the
// --cache-type-k / --cache-type-v options); rotation defaults to on for
// head_dim >= 64 and a multiple of 64 and is switchable per plane (same post,
// section "application and background"); the bf16 tail length is a setting
// (aitrends.kr article 92204, glossary "Precision Tail").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "kvq.h"

// Workspace of kvq_decode_attention_static: one copy of this array on each
// GPU the library runs on, held until the process ends.  In host code its
// name only stands in for the symbol; the device address comes from
// hipGetSymbolAddress, once per device (static_workspace below).
static __device__ __align__(256) uint8_t scratch[KVQ_STATIC_WORKSPACE_BYTES];

namespace {

using namespace kvq;

// Split-K waves per decode launch: one resident round on 256 compute units
// of 4 SIMDs at the kernel's occupancy.
int target_waves(int D, bool wide) { return 256 * 4 * split_waves_per_simd(D, wide); }
constexpr int kMaxSplits = kMaxSplitsDevice;
constexpr int32_t kMaxCtx = 2147483647 - 2 * kTile;
constexpr int32_t kOutlierChannels = 32;

thread_local hipEvent_t g_ev_before = nullptr;
thread_local hipEvent_t g_ev_after = nullptr;

bool bits_ok(int b) { return b == 4 || b == 5 || b == 6 || b == 8; }
bool dim_ok(int d) { return d == 64 || d == 128 || d == 192 || d == 256; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t cap_tokens(const kvq_config& c) { return ((int64_t)c.max_ctx + kTile - 1) / kTile * kTile; }

kvq_status check_cfg(const kvq_config* c) {
  if (!c) return KVQ_ERR_INVALID;
  if (c->batch < 1 || c->batch > KVQ_MAX_BATCH || c->n_kv_heads < 1 || c->max_ctx < 1 ||
      c->tail_len < 0 || (c->rotate_k != 0 && c->rotate_k != 1) ||
      (c->rotate_v != 0 && c->rotate_v != 1) || (c->k_min != 0 && c->k_min != 1) ||
      (c->v_min != 0 && c->v_min != 1) || c->page_pool < 0)
    return KVQ_ERR_INVALID;
  if (!dim_ok(c->head_dim) || !bits_ok(c->k_bits) || !bits_ok(c->v_bits)) return KVQ_ERR_UNSUPPORTED;
  // scale-and-min blocks come in the 4- and 5-bit widths (q4_1, q5_1)
  if ((c->k_min && c->k_bits > 5) || (c->v_min && c->v_bits > 5)) return KVQ_ERR_UNSUPPORTED;
  if (c->n_kv_heads > 65535 / 2) return KVQ_ERR_INVALID;
  // lengths, capacities and plane offsets are int32 in the kernels: the
  // capacity rounded up to a whole tile, plus a tile of slack, must fit
  if (c->max_ctx > kMaxCtx) return KVQ_ERR_INVALID;
  if (c->outliers != 0 && c->outliers != kOutlierChannels) return KVQ_ERR_INVALID;
  // outlier channels are built without a tail, at head_dim 128, with absmax
  // blocks for the rest
  if (c->outliers && (c->tail_len != 0 || c->head_dim != 128 || c->k_min || c->v_min))
    return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

kvq_status check_cache(const kvq_config& c, const kvq_cache* k) {
  if (!k) return KVQ_ERR_INVALID;
  const void* need[4] = {k->k_codes, k->k_scales, k->v_codes, k->v_scales};
  for (const void* p : need) {
    if (!p) return KVQ_ERR_INVALID;
    if (!aligned16(p)) return KVQ_ERR_ALIGN;
  }
  if (c.tail_len > 0) {
    if (!k->k_tail || !k->v_tail) return KVQ_ERR_INVALID;
    if (!aligned16(k->k_tail) || !aligned16(k->v_tail)) return KVQ_ERR_ALIGN;
  }
  if (c.page_pool > 0) {
    if (!k->page_table) return KVQ_ERR_INVALID;
    if ((reinterpret_cast<uintptr_t>(k->page_table) & 3u) != 0) return KVQ_ERR_ALIGN;
  }
  if (c.outliers) {
    const void* out[4] = {k->k_out_codes, k->k_out_scales, k->v_out_codes, k->v_out_scales};
    for (const void* p : out) {
      if (!p) return KVQ_ERR_INVALID;
      if (!aligned16(p)) return KVQ_ERR_ALIGN;
    }
    if (!k->outlier_idx) return KVQ_ERR_INVALID;
    if ((reinterpret_cast<uintptr_t>(k->outlier_idx) & 3u) != 0) return KVQ_ERR_ALIGN;
  }
  return KVQ_OK;
}

// Where the kernels find the 64-token tiles of the code and scale planes.
TileMap tile_map(const kvq_config& c, const kvq_cache* k) {
  TileMap m;
  m.ptab = c.page_pool > 0 ? k->page_table : nullptr;
  m.n_pages = c.page_pool;
  m.tiles = (int32_t)(cap_tokens(c) / kTile);
  m.Hkv = c.n_kv_heads;
  return m;
}

// Largest divisor of G that is at most 8 (query heads per kernel instance).
int head_chunk(int G) {
  for (int c = std::min(G, 8); c >= 1; --c)
    if (G % c == 0) return c;
  return 1;
}

// Splits per unit: enough waves for one resident round, at most one per
// 64-token tile of the longest sequence, a multiple of the workgroup size and
// at most kMaxSplits.  Non-decreasing in max_len.
int split_count(int D, bool wide, int64_t units, int max_len) {
  const int64_t tiles = std::max(1, (max_len + kTile - 1) / kTile);
  const int64_t gw = split_group_waves(D, wide);
  const int64_t want = std::max<int64_t>(1, (target_waves(D, wide) + units - 1) / units);
  int64_t S = (std::min(want, tiles) + gw - 1) / gw * gw;
  if (S > kMaxSplits) S = kMaxSplits / gw * gw;
  return (int)S;
}

struct Schedule {
  int gc, nchunk, S;
};

// Splits per (sequence, KV head, head chunk): enough waves to fill the chip,
// at most one split per 64-token tile of the longest sequence.  The kernel
// divides each sequence's work among the S splits by cost.
Schedule schedule(const kvq_config& c, int n_q_heads, int max_len) {
  Schedule s;
  const int G = n_q_heads / c.n_kv_heads;
  s.gc = head_chunk(G);
  s.nchunk = G / s.gc;
  const int64_t units = (int64_t)c.batch * c.n_kv_heads * s.nchunk;
  s.S = split_count(c.head_dim, c.k_min || c.v_min, units, max_len);
  return s;
}

// Upper bound of Schedule::S over every length up to max_ctx (S never exceeds
// the wanted split count, which never exceeds the tile count).
int max_splits(const kvq_config& c, int n_q_heads) {
  const int G = n_q_heads / c.n_kv_heads;
  const int nchunk = G / head_chunk(G);
  const int64_t units = (int64_t)c.batch * c.n_kv_heads * nchunk;
  return split_count(c.head_dim, c.k_min || c.v_min, units, c.max_ctx);
}

// Chunked prefill: the n_q * G rows of a KV head go in blocks of 8 rows per
// wave of a workgroup; each row block is split along the cache into S
// ranges.  One workgroup fills a compute unit, so a launch of W workgroups
// runs ceil(W / 256) rounds of 1/S of the work each: S minimises
// ceil(blocks * S / 256) / S (the first S within 2% of the best) up to
// max(16, twice what fills the chip), at most one split per 64-token tile of
// the longest sequence.  Non-decreasing in max_len.
struct PrefillSchedule {
  int n_rb, S;
};
// The matrix-core prefill covers head_dim 128 with absmax blocks.
bool prefill_on_mfma(const kvq_config& c) {
  return prefill_mfma_supported(c.head_dim, c.k_bits, c.v_bits, c.k_min != 0, c.v_min != 0);
}
PrefillSchedule prefill_schedule(const kvq_config& c, int n_q_heads, int n_q, int max_len) {
  PrefillSchedule p;
  const int64_t G = n_q_heads / c.n_kv_heads;
  const int64_t rows_per_block = prefill_on_mfma(c) ? kPrefillRows : 8 * split_group_waves(c.head_dim, true);
  p.n_rb = (int)(((int64_t)n_q * G + rows_per_block - 1) / rows_per_block);
  const int64_t blocks = (int64_t)c.batch * c.n_kv_heads * p.n_rb;
  const int64_t tiles = std::max(1, (max_len + kTile - 1) / kTile);
  const int64_t smax = std::min<int64_t>(std::min<int64_t>(kMaxSplits, tiles),
                                         std::max<int64_t>(16, 2 * ((256 + blocks - 1) / blocks)));
  auto cost = [&](int64_t S) { return (double)((blocks * S + 255) / 256) / (double)S; };
  double best = cost(1);
  for (int64_t S = 2; S <= smax; ++S) best = std::min(best, cost(S));
  p.S = 1;
  while (p.S < smax && cost(p.S) > best * 1.02) ++p.S;
  return p;
}

// Workspace: (max, sum) pairs, then partial vectors, per split; with outlier
// channels, then the partial sums of the 32 outlier channels of V.
struct WsLayout {
  size_t ml, acc, out, total;
};
WsLayout ws_layout(const kvq_config& c, int n_q_heads, int S) {
  WsLayout w;
  const size_t heads = (size_t)c.batch * n_q_heads;
  w.ml = 0;
  const size_t ml_bytes = heads * (size_t)S * 2 * sizeof(float);
  w.acc = w.ml + (ml_bytes + 255) / 256 * 256;
  const size_t acc_bytes = heads * (size_t)S * c.head_dim * sizeof(float);
  w.out = w.acc + (acc_bytes + 255) / 256 * 256;
  w.total = w.out + heads * (size_t)S * c.outliers * sizeof(float);
  return w;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): the golden-gamma
// increment, two xor-shift-multiply rounds and a final xor-shift.
uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Sign mask of the random-sign rotation H diag(s): bit e (word e / 32) is set
// where s_e = -1, i.e. where the top bit of SplitMix64(seed * 2^32 + e) is.
// Returns 0 (no signs) for seed 0.
int sign_mask(const kvq_config& c, uint32_t (&w)[8]) {
  for (int i = 0; i < 8; ++i) w[i] = 0;
  if (c.sign_seed == 0) return 0;
  for (int e = 0; e < c.head_dim; ++e)
    if (splitmix64(((uint64_t)c.sign_seed << 32) | (uint64_t)e) >> 63) w[e / 32] |= 1u << (e % 32);
  return 1;
}

// Append arguments of a checked call (lengths left to the caller).
AppendArgs append_args(const kvq_config& c, const kvq_cache* cache, const void* k_new, const void* v_new,
                       kvq_dtype dtype, int32_t n_new) {
  AppendArgs a;
  std::memset(&a, 0, sizeof(a));
  a.src[0] = k_new;
  a.src[1] = v_new;
  a.codes[0] = static_cast<uint8_t*>(cache->k_codes);
  a.codes[1] = static_cast<uint8_t*>(cache->v_codes);
  a.scales[0] = static_cast<uint16_t*>(cache->k_scales);
  a.scales[1] = static_cast<uint16_t*>(cache->v_scales);
  a.tail[0] = static_cast<uint16_t*>(cache->k_tail);
  a.tail[1] = static_cast<uint16_t*>(cache->v_tail);
  a.bits[0] = c.k_bits;
  a.bits[1] = c.v_bits;
  a.minf[0] = c.k_min;
  a.minf[1] = c.v_min;
  a.rotate[0] = c.rotate_k;
  a.rotate[1] = c.rotate_v;
  a.Hkv = c.n_kv_heads;
  a.n_new = n_new;
  a.T = c.tail_len;
  a.cap = (int32_t)cap_tokens(c);
  a.map = tile_map(c, cache);
  a.dtype = dtype;
  a.cd = (float)(1.0 / std::sqrt((double)rot_block(c.head_dim)));
  a.has_signs = sign_mask(c, a.signs);
  a.outl = c.outliers;
  if (c.outliers) {
    a.out_idx = cache->outlier_idx;
    a.out_codes[0] = static_cast<uint8_t*>(cache->k_out_codes);
    a.out_codes[1] = static_cast<uint8_t*>(cache->v_out_codes);
    a.out_scales[0] = static_cast<uint16_t*>(cache->k_out_scales);
    a.out_scales[1] = static_cast<uint16_t*>(cache->v_out_scales);
  }
  return a;
}

}  // namespace

extern "C" {

kvq_config kvq_config_default(int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t max_ctx) {
  kvq_config c{};
  c.batch = batch;
  c.n_kv_heads = n_kv_heads;
  c.head_dim = head_dim;
  c.k_bits = 4;
  c.v_bits = 4;
  c.tail_len = 0;
  c.max_ctx = max_ctx;
  const int on = (head_dim >= 64 && head_dim % 64 == 0) ? 1 : 0;
  c.rotate_k = on;
  c.rotate_v = on;
  c.sign_seed = 0;
  c.k_min = 0;
  c.v_min = 0;
  c.page_pool = 0;
  c.outliers = 0;
  return c;
}

kvq_status kvq_config_check(const kvq_config* cfg) { return check_cfg(cfg); }

size_t kvq_plane_bytes(const kvq_config* cfg, kvq_plane plane) {
  if (check_cfg(cfg) != KVQ_OK) return 0;
  const kvq_config& c = *cfg;
  const size_t units = (size_t)c.batch * c.n_kv_heads;
  // 64-token tiles of the code and scale planes: cap/64 per (b, g), or
  // page_pool per KV head for a paged cache
  const size_t tiles = c.page_pool > 0 ? (size_t)c.page_pool * c.n_kv_heads
                                       : units * (size_t)(cap_tokens(c) / kTile);
  const size_t nb = (size_t)(c.head_dim / kBlock);
  switch (plane) {
    case KVQ_K_CODES: return tiles * kTile * padded_row_bytes(c.head_dim, c.k_bits);
    case KVQ_V_CODES: return tiles * v_tile_bytes(c.head_dim, c.v_bits);
    case KVQ_K_SCALES: return tiles * kTile * nb * sizeof(uint16_t) * (c.k_min ? 2 : 1);
    case KVQ_V_SCALES: return tiles * kTile * nb * sizeof(uint16_t) * (c.v_min ? 2 : 1);
    case KVQ_K_TAIL:
    case KVQ_V_TAIL: return units * (size_t)c.tail_len * c.head_dim * sizeof(uint16_t);
    case KVQ_K_OUT_CODES:
    case KVQ_V_OUT_CODES: return tiles * kTile * (size_t)c.outliers;
    case KVQ_K_OUT_SCALES:
    case KVQ_V_OUT_SCALES: return c.outliers ? tiles * kTile * sizeof(uint16_t) : 0;
    default: break;
  }
  return 0;
}

size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t n_q_heads) {
  if (check_cfg(cfg) != KVQ_OK) return 0;
  if (n_q_heads < cfg->n_kv_heads || n_q_heads % cfg->n_kv_heads != 0) return 0;
  return ws_layout(*cfg, n_q_heads, max_splits(*cfg, n_q_heads)).total;
}

kvq_status kvq_rotate_quantize_append(const kvq_config* cfg, const kvq_cache* cache,
                                      const void* k_new, const void* v_new, kvq_dtype dtype,
                                      int32_t n_new, const int32_t* seq_len, void* stream) {
  kvq_status st = check_cfg(cfg);
  if (st != KVQ_OK) return st;
  const kvq_config& c = *cfg;
  if ((st = check_cache(c, cache)) != KVQ_OK) return st;
  if (dtype != KVQ_BF16 && dtype != KVQ_F32) return KVQ_ERR_INVALID;
  if (n_new < 0 || !seq_len) return KVQ_ERR_INVALID;
  for (int b = 0; b < c.batch; ++b) {
    if (seq_len[b] < 0) return KVQ_ERR_INVALID;
    if ((int64_t)seq_len[b] + n_new > c.max_ctx) return KVQ_ERR_CAPACITY;
  }
  if (n_new == 0) return KVQ_OK;
  if (!k_new || !v_new) return KVQ_ERR_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_ALIGN;

  AppendArgs a = append_args(c, cache, k_new, v_new, dtype, n_new);
  for (int b = 0; b < c.batch; ++b) a.len[b] = seq_len[b];
  return hip_status(launch_append(c.head_dim, a, c.batch, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Host checks of a decode call (everything but the workspace); on success
// the schedule, the workspace it needs and the kernel to launch.
struct DecodePlan {
  Schedule sc;
  WsLayout wl;
  DecodeLauncher fn;
};
kvq_status plan_decode(const kvq_config* cfg, const kvq_cache* cache, const void* q, kvq_dtype dtype,
                       int32_t n_q_heads, float sm_scale, const int32_t* seq_len, const float* out,
                       DecodePlan* plan) {
  kvq_status st = check_cfg(cfg);
  if (st != KVQ_OK) return st;
  const kvq_config& c = *cfg;
  if ((st = check_cache(c, cache)) != KVQ_OK) return st;
  if (dtype != KVQ_BF16 && dtype != KVQ_F32) return KVQ_ERR_INVALID;
  if (!q || !out || !seq_len) return KVQ_ERR_INVALID;
  if (!aligned16(q) || !aligned16(out)) return KVQ_ERR_ALIGN;
  if (n_q_heads < c.n_kv_heads || n_q_heads % c.n_kv_heads != 0) return KVQ_ERR_INVALID;
  if ((int64_t)c.batch * n_q_heads > 2147483647 / 8) return KVQ_ERR_INVALID;
  if (!std::isfinite(sm_scale)) return KVQ_ERR_INVALID;
  int max_len = 0;
  for (int b = 0; b < c.batch; ++b) {
    if (seq_len[b] < 1) return KVQ_ERR_INVALID;
    if (seq_len[b] > c.max_ctx) return KVQ_ERR_CAPACITY;
    max_len = std::max(max_len, (int)seq_len[b]);
  }
  plan->sc = schedule(c, n_q_heads, max_len);
  // grid y is (KV head, head chunk); the hardware limit of a grid dimension
  if ((int64_t)c.n_kv_heads * plan->sc.nchunk > 65535) return KVQ_ERR_INVALID;
  plan->wl = ws_layout(c, n_q_heads, plan->sc.S);
  plan->fn = decode_launcher(c.head_dim, c.k_bits, c.v_bits, plan->sc.gc, c.k_min != 0, c.v_min != 0,
                             c.page_pool > 0, c.outliers != 0);
  if (!plan->fn) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

// Queue the split kernel and the combine of a checked decode call.
// step: the fused decode step's one-token append (seq_len then counts the
// token), or null.
kvq_status run_decode(const kvq_config& c, const kvq_cache* cache, const void* q, kvq_dtype dtype,
                      int32_t n_q_heads, float sm_scale, const int32_t* seq_len, float* out,
                      void* workspace, const DecodePlan& plan, void* stream, const OneArgs* step = nullptr) {
  kvq_status st;
  const Schedule& sc = plan.sc;
  const WsLayout& wl = plan.wl;
  const DecodeLauncher fn = plan.fn;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const float cd = (float)(1.0 / std::sqrt((double)rot_block(c.head_dim)));

  DecodeArgs da;
  std::memset(&da, 0, sizeof(da));
  da.k_codes = static_cast<const uint8_t*>(cache->k_codes);
  da.k_scales = static_cast<const uint16_t*>(cache->k_scales);
  da.v_codes = static_cast<const uint8_t*>(cache->v_codes);
  da.v_scales = static_cast<const uint16_t*>(cache->v_scales);
  da.k_tail = static_cast<const uint16_t*>(cache->k_tail);
  da.v_tail = static_cast<const uint16_t*>(cache->v_tail);
  da.q = q;
  da.q_dtype = dtype;
  da.rotate_k = c.rotate_k;
  da.cd = cd;
  da.has_signs = sign_mask(c, da.signs);
  da.sm_scale = sm_scale;
  da.part_ml = reinterpret_cast<float*>(ws + wl.ml);
  da.part_acc = reinterpret_cast<float*>(ws + wl.acc);
  da.Hkv = c.n_kv_heads;
  da.Hq = n_q_heads;
  da.G = n_q_heads / c.n_kv_heads;
  da.n_gchunks = sc.nchunk;
  da.T = c.tail_len;
  da.cap = (int32_t)cap_tokens(c);
  da.map = tile_map(c, cache);
  da.S = sc.S;
  if (c.outliers) {
    da.out_codes[0] = static_cast<const uint8_t*>(cache->k_out_codes);
    da.out_codes[1] = static_cast<const uint8_t*>(cache->v_out_codes);
    da.out_scales[0] = static_cast<const uint16_t*>(cache->k_out_scales);
    da.out_scales[1] = static_cast<const uint16_t*>(cache->v_out_scales);
    da.out_idx = cache->outlier_idx;
    da.part_out = reinterpret_cast<float*>(ws + wl.out);
  }
  if (step) {
    da.step_on = 1;
    da.step = *step;
  }
  for (int b = 0; b < c.batch; ++b) da.len[b] = seq_len[b];
  const dim3 grid(sc.S / split_group_waves(c.head_dim, c.k_min || c.v_min), c.n_kv_heads * sc.nchunk,
                  c.batch);
  if ((st = hip_status(fn(da, grid, s, g_ev_before, g_ev_after))) != KVQ_OK) return st;

  CombineArgs ca;
  ca.part_ml = da.part_ml;
  ca.part_acc = da.part_acc;
  ca.out = out;
  ca.Hq = n_q_heads;
  ca.S = sc.S;
  ca.rotate = c.rotate_v;
  ca.cd = cd;
  ca.has_signs = da.has_signs;
  for (int i = 0; i < 8; ++i) ca.signs[i] = da.signs[i];
  ca.part_out = da.part_out;
  ca.v_out_idx = c.outliers ? cache->outlier_idx + (size_t)c.n_kv_heads * c.outliers : nullptr;
  ca.G = n_q_heads / c.n_kv_heads;
  return hip_status(launch_combine(c.head_dim, ca, c.batch, s));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the
// first call there; nullptr if the runtime reports an error.
void* static_workspace() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attention(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                kvq_dtype dtype, int32_t n_q_heads, float sm_scale,
                                const int32_t* seq_len, float* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  DecodePlan plan;
  kvq_status st = plan_decode(cfg, cache, q, dtype, n_q_heads, sm_scale, seq_len, out, &plan);
  if (st != KVQ_OK) return st;
  if (!workspace) return KVQ_ERR_INVALID;
  if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
  if (workspace_bytes < plan.wl.total) return KVQ_ERR_WORKSPACE;
  return run_decode(*cfg, cache, q, dtype, n_q_heads, sm_scale, seq_len, out, workspace, plan, stream);
}

kvq_status kvq_decode_step(const kvq_config* cfg, const kvq_cache* cache, const void* k_new,
                           const void* v_new, kvq_dtype kv_dtype, const void* q, kvq_dtype q_dtype,
                           int32_t n_q_heads, float sm_scale, const int32_t* seq_len, float* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  kvq_status st = check_cfg(cfg);
  if (st != KVQ_OK) return st;
  const kvq_config& c = *cfg;
  if ((st = check_cache(c, cache)) != KVQ_OK) return st;
  if (kv_dtype != KVQ_BF16 && kv_dtype != KVQ_F32) return KVQ_ERR_INVALID;
  if (!seq_len || !k_new || !v_new) return KVQ_ERR_INVALID;
  if (!aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_ALIGN;
  int32_t lens[KVQ_MAX_BATCH];
  for (int b = 0; b < c.batch; ++b) {
    if (seq_len[b] < 0) return KVQ_ERR_INVALID;
    if ((int64_t)seq_len[b] + 1 > c.max_ctx) return KVQ_ERR_CAPACITY;
    lens[b] = seq_len[b] + 1;
  }
  DecodePlan plan;
  if ((st = plan_decode(cfg, cache, q, q_dtype, n_q_heads, sm_scale, lens, out, &plan)) != KVQ_OK) return st;
  if (!workspace) return KVQ_ERR_INVALID;
  if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
  if (workspace_bytes < plan.wl.total) return KVQ_ERR_WORKSPACE;
  AppendArgs a = append_args(c, cache, k_new, v_new, kv_dtype, 1);
  if (plan.sc.nchunk > 1 || c.outliers) {
    // a KV head's query heads span several chunks, each of which would
    // need the values of the position leaving the tail while another one
    // overwrites it (or the cache has outlier channels, which the fused
    // path does not carry): append first, then attend
    for (int b = 0; b < c.batch; ++b) a.len[b] = seq_len[b];
    if ((st = hip_status(launch_append(c.head_dim, a, c.batch, static_cast<hipStream_t>(stream)))) != KVQ_OK)
      return st;
    return run_decode(c, cache, q, q_dtype, n_q_heads, sm_scale, lens, out, workspace, plan, stream);
  }
  const OneArgs one = one_args(a);
  return run_decode(c, cache, q, q_dtype, n_q_heads, sm_scale, lens, out, workspace, plan, stream, &one);
}

kvq_status kvq_decode_attention_static(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                       kvq_dtype dtype, int32_t n_q_heads, float sm_scale,
                                       const int32_t* seq_len, float* out, void* stream) {
  DecodePlan plan;
  kvq_status st = plan_decode(cfg, cache, q, dtype, n_q_heads, sm_scale, seq_len, out, &plan);
  if (st != KVQ_OK) return st;
  if (plan.wl.total > KVQ_STATIC_WORKSPACE_BYTES) return KVQ_ERR_WORKSPACE;
  void* ws = static_workspace();
  if (!ws) return KVQ_ERR_HIP;
  return run_decode(*cfg, cache, q, dtype, n_q_heads, sm_scale, seq_len, out, ws, plan, stream);
}

// Prefill workspace: the split partials, then (matrix-core path) the
// prepared query rows, fp16 hi and lo parts and one factor per row.
struct PrefillWs {
  WsLayout parts;
  size_t q_hi, q_lo, q_w, total;
  int rows_pad;
};
PrefillWs prefill_ws(const kvq_config& c, int n_q_heads, int n_q, const PrefillSchedule& p) {
  PrefillWs w;
  w.parts = ws_layout(c, n_q * n_q_heads, p.S);
  w.rows_pad = p.n_rb * kPrefillRows;
  w.total = (w.parts.total + 255) / 256 * 256;
  w.q_hi = w.q_lo = w.q_w = 0;
  if (prefill_on_mfma(c)) {
    const size_t rows = (size_t)c.batch * c.n_kv_heads * w.rows_pad;
    const size_t half_bytes = (rows * c.head_dim * 2 + 255) / 256 * 256;
    w.q_hi = w.total;
    w.q_lo = w.q_hi + half_bytes;
    w.q_w = w.q_lo + half_bytes;
    w.total = w.q_w + rows * sizeof(float);
  }
  return w;
}

size_t kvq_prefill_workspace_bytes(const kvq_config* cfg, int32_t n_q_heads, int32_t n_q) {
  if (check_cfg(cfg) != KVQ_OK) return 0;
  if (n_q_heads < cfg->n_kv_heads || n_q_heads % cfg->n_kv_heads != 0 || n_q < 1) return 0;
  if ((int64_t)n_q * n_q_heads > 2147483647 / 8) return 0;
  const PrefillSchedule p = prefill_schedule(*cfg, n_q_heads, n_q, cfg->max_ctx);
  return prefill_ws(*cfg, n_q_heads, n_q, p).total;
}

kvq_status kvq_prefill_attention(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                 kvq_dtype dtype, int32_t n_q_heads, int32_t n_q, float sm_scale,
                                 const int32_t* seq_len, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  kvq_status st = check_cfg(cfg);
  if (st != KVQ_OK) return st;
  const kvq_config& c = *cfg;
  if ((st = check_cache(c, cache)) != KVQ_OK) return st;
  if (dtype != KVQ_BF16 && dtype != KVQ_F32) return KVQ_ERR_INVALID;
  if (!q || !out || !workspace || !seq_len) return KVQ_ERR_INVALID;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return KVQ_ERR_ALIGN;
  if (n_q_heads < c.n_kv_heads || n_q_heads % c.n_kv_heads != 0 || n_q < 1) return KVQ_ERR_INVALID;
  if ((int64_t)c.batch * n_q * n_q_heads > 2147483647 / 8) return KVQ_ERR_INVALID;
  if (!std::isfinite(sm_scale)) return KVQ_ERR_INVALID;
  if (c.outliers) return KVQ_ERR_UNSUPPORTED;   // prefill is built without outlier channels
  int max_len = 0;
  for (int b = 0; b < c.batch; ++b) {
    if (seq_len[b] < n_q) return KVQ_ERR_INVALID;
    if (seq_len[b] > c.max_ctx) return KVQ_ERR_CAPACITY;
    max_len = std::max(max_len, (int)seq_len[b]);
  }
  const PrefillSchedule ps = prefill_schedule(c, n_q_heads, n_q, max_len);
  if ((int64_t)c.n_kv_heads * ps.n_rb > 65535) return KVQ_ERR_INVALID;
  const PrefillWs pw = prefill_ws(c, n_q_heads, n_q, ps);
  const WsLayout& wl = pw.parts;
  if (workspace_bytes < pw.total) return KVQ_ERR_WORKSPACE;
  const bool mfma = prefill_on_mfma(c);
  const DecodeLauncher fn = mfma ? nullptr
                                 : prefill_launcher(c.head_dim, c.k_bits, c.v_bits, c.k_min != 0,
                                                    c.v_min != 0, c.page_pool > 0);
  if (!mfma && !fn) return KVQ_ERR_UNSUPPORTED;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const float cd = (float)(1.0 / std::sqrt((double)rot_block(c.head_dim)));

  if (mfma) {
    PrefillArgs pa;
    std::memset(&pa, 0, sizeof(pa));
    pa.k_codes = static_cast<const uint8_t*>(cache->k_codes);
    pa.k_scales = static_cast<const uint16_t*>(cache->k_scales);
    pa.v_codes = static_cast<const uint8_t*>(cache->v_codes);
    pa.v_scales = static_cast<const uint16_t*>(cache->v_scales);
    pa.k_tail = static_cast<const uint16_t*>(cache->k_tail);
    pa.v_tail = static_cast<const uint16_t*>(cache->v_tail);
    pa.q = q;
    pa.q_dtype = dtype;
    pa.q_hi = reinterpret_cast<uint16_t*>(ws + pw.q_hi);
    pa.q_lo = reinterpret_cast<uint16_t*>(ws + pw.q_lo);
    pa.q_w = reinterpret_cast<float*>(ws + pw.q_w);
    pa.part_ml = reinterpret_cast<float*>(ws + wl.ml);
    pa.part_acc = reinterpret_cast<float*>(ws + wl.acc);
    pa.Hkv = c.n_kv_heads;
    pa.Hq = n_q_heads;
    pa.G = n_q_heads / c.n_kv_heads;
    pa.T = c.tail_len;
    pa.S = ps.S;
    pa.n_q = n_q;
    pa.n_rb = ps.n_rb;
    pa.rows_pad = pw.rows_pad;
    pa.map = tile_map(c, cache);
    pa.rotate_k = c.rotate_k;
    pa.cd = cd;
    pa.sm_scale = sm_scale;
    pa.has_signs = sign_mask(c, pa.signs);
    for (int b = 0; b < c.batch; ++b) pa.len[b] = seq_len[b];
    if ((st = hip_status(launch_prefill_q(pa, c.k_bits, c.batch, s))) != KVQ_OK) return st;
    if ((st = hip_status(launch_prefill_mfma(pa, c.k_bits, c.v_bits, c.batch, s, g_ev_before, g_ev_after))) !=
        KVQ_OK)
      return st;
    CombineArgs ca;
    ca.part_ml = pa.part_ml;
    ca.part_acc = pa.part_acc;
    ca.out = out;
    ca.Hq = n_q * n_q_heads;   // rows [B][n_q][Hq] are combined like heads
    ca.part_out = nullptr;
    ca.v_out_idx = nullptr;
    ca.G = 1;
    ca.S = ps.S;
    ca.rotate = c.rotate_v;
    ca.cd = cd;
    ca.has_signs = pa.has_signs;
    for (int i = 0; i < 8; ++i) ca.signs[i] = pa.signs[i];
    return hip_status(launch_combine(c.head_dim, ca, c.batch, s));
  }

  DecodeArgs da;
  std::memset(&da, 0, sizeof(da));
  da.k_codes = static_cast<const uint8_t*>(cache->k_codes);
  da.k_scales = static_cast<const uint16_t*>(cache->k_scales);
  da.v_codes = static_cast<const uint8_t*>(cache->v_codes);
  da.v_scales = static_cast<const uint16_t*>(cache->v_scales);
  da.k_tail = static_cast<const uint16_t*>(cache->k_tail);
  da.v_tail = static_cast<const uint16_t*>(cache->v_tail);
  da.q = q;
  da.q_dtype = dtype;
  da.rotate_k = c.rotate_k;
  da.cd = cd;
  da.has_signs = sign_mask(c, da.signs);
  da.sm_scale = sm_scale;
  da.part_ml = reinterpret_cast<float*>(ws + wl.ml);
  da.part_acc = reinterpret_cast<float*>(ws + wl.acc);
  da.Hkv = c.n_kv_heads;
  da.Hq = n_q_heads;
  da.G = n_q_heads / c.n_kv_heads;
  da.n_gchunks = 1;
  da.T = c.tail_len;
  da.cap = (int32_t)cap_tokens(c);
  da.map = tile_map(c, cache);
  da.S = ps.S;
  da.n_q = n_q;
  da.n_rb = ps.n_rb;
  for (int b = 0; b < c.batch; ++b) da.len[b] = seq_len[b];
  const dim3 grid(ps.S, c.n_kv_heads * ps.n_rb, c.batch);
  if ((st = hip_status(fn(da, grid, s, g_ev_before, g_ev_after))) != KVQ_OK) return st;

  CombineArgs ca;
  ca.part_ml = da.part_ml;
  ca.part_acc = da.part_acc;
  ca.out = out;
  ca.Hq = n_q * n_q_heads;   // rows [B][n_q][Hq] are combined like heads
  ca.part_out = nullptr;
  ca.v_out_idx = nullptr;
  ca.G = 1;
  ca.S = ps.S;
  ca.rotate = c.rotate_v;
  ca.cd = cd;
  ca.has_signs = da.has_signs;
  for (int i = 0; i < 8; ++i) ca.signs[i] = da.signs[i];
  return hip_status(launch_combine(c.head_dim, ca, c.batch, s));
}

kvq_status kvq_dequantize(const kvq_config* cfg, const kvq_cache* cache, int32_t which, int32_t b,
                          int32_t t0, int32_t t1, const int32_t* seq_len, int32_t space,
                          float* out, void* stream) {
  kvq_status st = check_cfg(cfg);
  if (st != KVQ_OK) return st;
  const kvq_config& c = *cfg;
  if ((st = check_cache(c, cache)) != KVQ_OK) return st;
  if ((which != 0 && which != 1) || (space != 0 && space != 1) || !seq_len)
    return KVQ_ERR_INVALID;
  if (b < 0 || b >= c.batch) return KVQ_ERR_INVALID;
  const int n = seq_len[b];
  if (n < 0) return KVQ_ERR_INVALID;
  if (n > c.max_ctx) return KVQ_ERR_CAPACITY;
  if (t0 < 0 || t0 > t1 || t1 > n) return KVQ_ERR_INVALID;
  if (t0 == t1) return KVQ_OK;
  if (!out) return KVQ_ERR_INVALID;
  if (!aligned16(out)) return KVQ_ERR_ALIGN;
  DequantArgs a;
  a.codes = static_cast<const uint8_t*>(which == 0 ? cache->k_codes : cache->v_codes);
  a.scales = static_cast<const uint16_t*>(which == 0 ? cache->k_scales : cache->v_scales);
  a.tail = static_cast<const uint16_t*>(which == 0 ? cache->k_tail : cache->v_tail);
  a.out = out;
  a.which = which;
  a.bits = which == 0 ? c.k_bits : c.v_bits;
  a.minf = which == 0 ? c.k_min : c.v_min;
  a.rotate = which == 0 ? c.rotate_k : c.rotate_v;
  a.space = space;
  a.Hkv = c.n_kv_heads;
  a.T = c.tail_len;
  a.cap = (int32_t)cap_tokens(c);
  a.map = tile_map(c, cache);
  a.b = b;
  a.t0 = t0;
  a.t1 = t1;
  a.nq = n - (c.tail_len > 0 ? std::min(n, (int)c.tail_len) : 0);
  a.cd = (float)(1.0 / std::sqrt((double)rot_block(c.head_dim)));
  a.has_signs = sign_mask(c, a.signs);
  a.outl = c.outliers;
  a.out_codes = static_cast<const uint8_t*>(which == 0 ? cache->k_out_codes : cache->v_out_codes);
  a.out_scales = static_cast<const uint16_t*>(which == 0 ? cache->k_out_scales : cache->v_out_scales);
  a.out_idx = c.outliers ? cache->outlier_idx + (size_t)which * c.n_kv_heads * c.outliers : nullptr;
  return hip_status(launch_dequant(c.head_dim, a, static_cast<hipStream_t>(stream)));
}

const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported head_dim or bit width";
    case KVQ_ERR_CAPACITY: return "sequence length exceeds max_ctx";
    case KVQ_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case KVQ_ERR_HIP: return "HIP runtime error";
    case KVQ_ERR_WORKSPACE: return "decode workspace too small";
    default: break;
  }
  return "unknown status";
}

void kvq_profile_decode_events(void* before, void* after) {
  if (before && after) {
    g_ev_before = static_cast<hipEvent_t>(before);
    g_ev_after = static_cast<hipEvent_t>(after);
  } else {
    g_ev_before = nullptr;
    g_ev_after = nullptr;
  }
}

}  // extern "C"
