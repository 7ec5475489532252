// Host-side checks of the kvq C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of the library (the kernels
// are not instrumented and never run here): configuration checks, plane and
// workspace sizes over many configurations, and every argument error of the
// entry points, each of which must return its status before any device
// work.  Prints "ok" and exits 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kvq.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::printf("FAILED line %d: %s\n", __LINE__, #cond);           \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static void* fake(uintptr_t a = 0x10000) { return reinterpret_cast<void*>(a); }

static kvq_cache cache_of(uintptr_t codes = 0x10000, uintptr_t tail = 0x10000) {
  kvq_cache c{};
  c.k_codes = fake(codes);
  c.k_scales = fake();
  c.v_codes = fake();
  c.v_scales = fake();
  c.k_tail = fake(tail);
  c.v_tail = fake(tail);
  c.page_table = reinterpret_cast<const int32_t*>(0x10000);
  return c;
}

int main() {
  // sizes over a grid of configurations (pure host arithmetic)
  const int dims[] = {64, 128, 192, 256, 96, 320};
  const int bits[] = {4, 5, 6, 8, 3};
  for (int d : dims)
    for (int kb : bits)
      for (int vb : bits)
        for (int T : {0, 1, 1024})
          for (int pool : {0, 7}) {
            kvq_config c = kvq_config_default(3, 5, d, 70001);
            c.k_bits = kb;
            c.v_bits = vb;
            c.tail_len = T;
            c.page_pool = pool;
            c.sign_seed = (uint32_t)(d * 7 + kb);
            const kvq_status st = kvq_config_check(&c);
            size_t total = 0;
            for (int p = 0; p < 6; ++p) total += kvq_plane_bytes(&c, (kvq_plane)p);
            if (st == KVQ_OK) {
              CHECK(total > 0);
              CHECK(kvq_decode_workspace_bytes(&c, 10) > 0);
              CHECK(kvq_prefill_workspace_bytes(&c, 10, 33) > 0);
            } else {
              CHECK(total == 0);
              CHECK(kvq_decode_workspace_bytes(&c, 10) == 0);
            }
          }
  // limits
  kvq_config big = kvq_config_default(KVQ_MAX_BATCH, 8, 256, 2147483647);
  CHECK(kvq_config_check(&big) == KVQ_ERR_INVALID);
  big.max_ctx = 2147483647 - 128;
  CHECK(kvq_config_check(&big) == KVQ_OK);
  CHECK(kvq_decode_workspace_bytes(&big, 64) > 0);
  kvq_config many = kvq_config_default(1, 10000, 128, 100);
  std::vector<int32_t> lens(KVQ_MAX_BATCH, 50);
  kvq_cache ch = cache_of();
  CHECK(kvq_decode_attention(&many, &ch, fake(), KVQ_BF16, 110000, 0.1f, lens.data(), (float*)fake(),
                             fake(), (size_t)1 << 40, nullptr) == KVQ_ERR_INVALID);

  // argument errors of every entry point
  kvq_config c = kvq_config_default(2, 4, 128, 100);
  c.k_bits = 8;
  c.tail_len = 16;
  int32_t l_ok[2] = {5, 5}, l_neg[2] = {-1, 5}, l_big[2] = {100, 5}, l_over[2] = {101, 5}, l_zero[2] = {0, 5};
  float* out = (float*)fake();
  CHECK(kvq_rotate_quantize_append(&c, &ch, fake(), fake(), KVQ_BF16, 96, l_ok, nullptr) == KVQ_ERR_CAPACITY);
  CHECK(kvq_rotate_quantize_append(&c, &ch, fake(), fake(), KVQ_BF16, 1, l_neg, nullptr) == KVQ_ERR_INVALID);
  CHECK(kvq_rotate_quantize_append(&c, &ch, nullptr, fake(), KVQ_BF16, 1, l_ok, nullptr) == KVQ_ERR_INVALID);
  CHECK(kvq_rotate_quantize_append(&c, &ch, fake(0x10008), fake(), KVQ_BF16, 1, l_ok, nullptr) == KVQ_ERR_ALIGN);
  CHECK(kvq_rotate_quantize_append(&c, &ch, fake(), fake(), (kvq_dtype)7, 1, l_ok, nullptr) == KVQ_ERR_INVALID);
  CHECK(kvq_rotate_quantize_append(&c, &ch, fake(), fake(), KVQ_BF16, 0, l_ok, nullptr) == KVQ_OK);
  kvq_cache notail = cache_of(0x10000, 0);
  CHECK(kvq_rotate_quantize_append(&c, &notail, fake(), fake(), KVQ_BF16, 1, l_ok, nullptr) == KVQ_ERR_INVALID);
  kvq_cache misal = cache_of(0x10008);
  CHECK(kvq_decode_attention(&c, &misal, fake(), KVQ_BF16, 8, 0.1f, l_ok, out, fake(), 1 << 30, nullptr) ==
        KVQ_ERR_ALIGN);
  CHECK(kvq_decode_attention(&c, &ch, fake(), KVQ_BF16, 6, 0.1f, l_ok, out, fake(), 1 << 30, nullptr) ==
        KVQ_ERR_INVALID);
  CHECK(kvq_decode_attention(&c, &ch, fake(), KVQ_BF16, 8, 0.1f, l_zero, out, fake(), 1 << 30, nullptr) ==
        KVQ_ERR_INVALID);
  CHECK(kvq_decode_attention(&c, &ch, fake(), KVQ_BF16, 8, 0.1f, l_over, out, fake(), 1 << 30, nullptr) ==
        KVQ_ERR_CAPACITY);
  CHECK(kvq_decode_attention(&c, &ch, fake(), KVQ_BF16, 8, 0.1f, l_ok, out, fake(), 16, nullptr) ==
        KVQ_ERR_WORKSPACE);
  CHECK(kvq_decode_attention(&c, &ch, fake(), KVQ_BF16, 8, 1.0f / 0.0f, l_ok, out, fake(), 1 << 30, nullptr) ==
        KVQ_ERR_INVALID);
  CHECK(kvq_decode_attention_static(&c, &ch, fake(), KVQ_BF16, 6, 0.1f, l_ok, out, nullptr) == KVQ_ERR_INVALID);
  kvq_config huge = kvq_config_default(KVQ_MAX_BATCH, 8, 256, 70000);
  huge.k_bits = huge.v_bits = 8;
  std::vector<int32_t> l_full(KVQ_MAX_BATCH, 65536);
  CHECK(kvq_decode_attention_static(&huge, &ch, fake(), KVQ_BF16, 64, 0.1f, l_full.data(), out, nullptr) ==
        KVQ_ERR_WORKSPACE);
  CHECK(kvq_decode_step(&c, &ch, fake(), fake(), KVQ_BF16, fake(), KVQ_BF16, 8, 0.1f, l_big, out, fake(),
                        1 << 30, nullptr) == KVQ_ERR_CAPACITY);
  CHECK(kvq_decode_step(&c, &ch, fake(), nullptr, KVQ_BF16, fake(), KVQ_BF16, 8, 0.1f, l_ok, out, fake(),
                        1 << 30, nullptr) == KVQ_ERR_INVALID);
  CHECK(kvq_decode_step(&c, &ch, fake(), fake(), KVQ_BF16, fake(), KVQ_BF16, 8, 0.1f, l_ok, out, fake(), 16,
                        nullptr) == KVQ_ERR_WORKSPACE);
  CHECK(kvq_prefill_attention(&c, &ch, fake(), KVQ_BF16, 8, 6, 0.1f, l_ok, out, fake(), 1 << 30, nullptr) ==
        KVQ_ERR_INVALID);
  CHECK(kvq_prefill_attention(&c, &ch, fake(), KVQ_BF16, 8, 0, 0.1f, l_ok, out, fake(), 1 << 30, nullptr) ==
        KVQ_ERR_INVALID);
  CHECK(kvq_dequantize(&c, &ch, 2, 0, 0, 1, l_ok, 0, out, nullptr) == KVQ_ERR_INVALID);
  CHECK(kvq_dequantize(&c, &ch, 0, 2, 0, 1, l_ok, 0, out, nullptr) == KVQ_ERR_INVALID);
  CHECK(kvq_dequantize(&c, &ch, 0, 0, 3, 2, l_ok, 0, out, nullptr) == KVQ_ERR_INVALID);
  CHECK(kvq_dequantize(&c, &ch, 0, 0, 0, 6, l_ok, 0, out, nullptr) == KVQ_ERR_INVALID);
  CHECK(kvq_dequantize(&c, &ch, 0, 0, 2, 2, l_ok, 0, nullptr, nullptr) == KVQ_OK);
  kvq_config paged = c;
  paged.page_pool = 10;
  kvq_cache nopt = cache_of();
  nopt.page_table = nullptr;
  CHECK(kvq_decode_attention(&paged, &nopt, fake(), KVQ_BF16, 8, 0.1f, l_ok, out, fake(), 1 << 30, nullptr) ==
        KVQ_ERR_INVALID);
  // outlier channels: 32 per plane and KV head, no tail, head_dim 128,
  // absmax blocks; the lists and the four planes must be given
  kvq_config oc = kvq_config_default(2, 4, 128, 1000);
  oc.outliers = 32;
  CHECK(kvq_config_check(&oc) == KVQ_OK);
  CHECK(kvq_plane_bytes(&oc, KVQ_K_OUT_CODES) == (size_t)2 * 4 * 1024 * 32);
  CHECK(kvq_plane_bytes(&oc, KVQ_V_OUT_SCALES) == (size_t)2 * 4 * 1024 * 2);
  kvq_config oc_bad = oc;
  oc_bad.outliers = 16;
  CHECK(kvq_config_check(&oc_bad) == KVQ_ERR_INVALID);
  oc_bad = oc;
  oc_bad.tail_len = 8;
  CHECK(kvq_config_check(&oc_bad) == KVQ_ERR_UNSUPPORTED);
  kvq_cache och = cache_of(0x10000, 0);
  CHECK(kvq_decode_attention(&oc, &och, fake(), KVQ_BF16, 8, 0.1f, l_ok, out, fake(), 1 << 30, nullptr) ==
        KVQ_ERR_INVALID);   // no outlier planes
  och.k_out_codes = fake();
  och.k_out_scales = fake();
  och.v_out_codes = fake();
  och.v_out_scales = fake();
  och.outlier_idx = reinterpret_cast<const int32_t*>(0x10002);
  CHECK(kvq_decode_attention(&oc, &och, fake(), KVQ_BF16, 8, 0.1f, l_ok, out, fake(), 1 << 30, nullptr) ==
        KVQ_ERR_ALIGN);
  och.outlier_idx = reinterpret_cast<const int32_t*>(0x10000);
  CHECK(kvq_prefill_attention(&oc, &och, fake(), KVQ_BF16, 8, 1, 0.1f, l_ok, out, fake(), 1 << 30, nullptr) ==
        KVQ_ERR_UNSUPPORTED);
  for (int s = -6; s <= 0; ++s) CHECK(kvq_status_str((kvq_status)s) != nullptr);
  CHECK(kvq_status_str((kvq_status)-99) != nullptr);
  kvq_profile_decode_events(nullptr, nullptr);

  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
