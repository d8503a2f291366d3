// abi_sanitize_main.cpp -- the C ABI's host-side validation under
// AddressSanitizer and UndefinedBehaviorSanitizer: every entry point of
// include/kvq.h called with valid arguments (exactly one launch of the right
// kind must be requested) and with each kind of invalid argument (the status
// the header documents, and no launch).  Built for the host alone against
// abi_sanitize_stubs.cpp by tests/test_abi_sanitized.py; device pointers
// are stand-in addresses that are never dereferenced.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "kvq.h"

extern int g_launch_count;
extern int g_last_launch;
extern uint32_t g_debug_bits;
extern int g_debug_checks;

static int failures = 0;

static void expect(const char* what, int got, int want, int kind) {
  const int before = g_launch_count;
  (void)before;
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    failures++;
  }
  (void)kind;
}

// Runs `call` and checks its status and the launch it requested (kind 0: none).
#define CHECK(what, call, want, kind)                                                            \
  do {                                                                                           \
    const int n0 = g_launch_count;                                                               \
    const int st = (int)(call);                                                                  \
    expect(what, st, want, kind);                                                                \
    const int launched = g_launch_count - n0;                                                    \
    if ((kind) == 0 && launched != 0) {                                                          \
      fprintf(stderr, "FAIL %s: a rejected call requested %d launches\n", what, launched);       \
      failures++;                                                                                \
    }                                                                                            \
    if ((kind) != 0 && (launched < 1 || g_last_launch != (kind))) {                              \
      fprintf(stderr, "FAIL %s: expected a launch of kind %d, got %d launches (last %d)\n", what, \
              (int)(kind), launched, g_last_launch);                                             \
      failures++;                                                                                \
    }                                                                                            \
  } while (0)

static void* const F = (void*)(uintptr_t)0x10000;  // 16-byte aligned stand-in address
static void* off(void* p, int b) { return (void*)((uintptr_t)p + b); }

static kvq_cache cache(int fmt = KVQ_FMT_NVFP4, int pages = 64, int P = 16, int H = 4, int D = 256, void* pool = F,
                       const void* gs = F, int flags = 0) {
  kvq_cache c;
  c.fmt = fmt;
  c.num_pages = pages;
  c.page_size = P;
  c.num_kv_heads = H;
  c.head_dim = D;
  c.pool = pool;
  c.global_scale = (const float*)gs;
  c.flags = flags;
  return c;
}

int main() {
  // ---- quantize-store
  kvq_cache c = cache();
  CHECK("store ok", kvq_quantize_store(&c, F, F, KVQ_DT_BF16, 1024, (const int32_t*)F, 4, nullptr), KVQ_OK, 1);
  CHECK("store fp32 ok", kvq_quantize_store(&c, F, F, KVQ_DT_F32, 1024, (const int32_t*)F, 4, nullptr), KVQ_OK, 1);
  CHECK("store null cache", kvq_quantize_store(nullptr, F, F, 1, 1024, (const int32_t*)F, 4, nullptr), KVQ_ERR_NULL,
        0);
  kvq_cache bad = cache(KVQ_FMT_NVFP4, 64, 16, 4, 256, nullptr);
  CHECK("store null pool", kvq_quantize_store(&bad, F, F, 1, 1024, (const int32_t*)F, 4, nullptr), KVQ_ERR_NULL, 0);
  bad = cache(KVQ_FMT_NVFP4, 64, 16, 4, 256, F, nullptr);
  CHECK("store null gs", kvq_quantize_store(&bad, F, F, 1, 1024, (const int32_t*)F, 4, nullptr), KVQ_ERR_NULL, 0);
  bad = cache(7);
  CHECK("store fmt", kvq_quantize_store(&bad, F, F, 1, 1024, (const int32_t*)F, 4, nullptr), KVQ_ERR_UNSUPPORTED, 0);
  bad = cache(KVQ_FMT_NVFP4, 64, 16, 4, 64);
  CHECK("store D 64", kvq_quantize_store(&bad, F, F, 1, 256, (const int32_t*)F, 4, nullptr), KVQ_ERR_UNSUPPORTED, 0);
  bad = cache(KVQ_FMT_NVFP4, 64, 24);
  CHECK("store P 24", kvq_quantize_store(&bad, F, F, 1, 1024, (const int32_t*)F, 4, nullptr), KVQ_ERR_UNSUPPORTED, 0);
  bad = cache(KVQ_FMT_NVFP4, 0);
  CHECK("store pages 0", kvq_quantize_store(&bad, F, F, 1, 1024, (const int32_t*)F, 4, nullptr), KVQ_ERR_SHAPE, 0);
  bad = cache(KVQ_FMT_NVFP4, 64, 16, 4, 256, off(F, 8));
  CHECK("store pool align", kvq_quantize_store(&bad, F, F, 1, 1024, (const int32_t*)F, 4, nullptr), KVQ_ERR_ALIGN, 0);
  bad = cache(KVQ_FMT_NVFP4, 64, 16, 4, 256, F, F, 2);
  CHECK("store flags", kvq_quantize_store(&bad, F, F, 1, 1024, (const int32_t*)F, 4, nullptr), KVQ_ERR_UNSUPPORTED,
        0);
  CHECK("store dtype", kvq_quantize_store(&c, F, F, 7, 1024, (const int32_t*)F, 4, nullptr), KVQ_ERR_UNSUPPORTED, 0);
  CHECK("store n -1", kvq_quantize_store(&c, F, F, 1, 1024, (const int32_t*)F, -1, nullptr), KVQ_ERR_SHAPE, 0);
  CHECK("store n 0", kvq_quantize_store(&c, F, F, 1, 1024, (const int32_t*)F, 0, nullptr), KVQ_OK, 0);
  CHECK("store k null", kvq_quantize_store(&c, nullptr, F, 1, 1024, (const int32_t*)F, 4, nullptr), KVQ_ERR_NULL, 0);
  CHECK("store stride", kvq_quantize_store(&c, F, F, 1, 1000, (const int32_t*)F, 4, nullptr), KVQ_ERR_SHAPE, 0);
  CHECK("store stride align", kvq_quantize_store(&c, F, F, 1, 1028, (const int32_t*)F, 4, nullptr), KVQ_ERR_ALIGN, 0);
  CHECK("store k align", kvq_quantize_store(&c, off(F, 2), F, 1, 1024, (const int32_t*)F, 4, nullptr), KVQ_ERR_ALIGN,
        0);
  kvq_cache i4 = cache(KVQ_FMT_INT4_TOKHEAD, 64, 1600, 4, 256, F, nullptr);
  CHECK("store int4 no gs", kvq_quantize_store(&i4, F, F, 1, 1024, (const int32_t*)F, 4, nullptr), KVQ_OK, 1);

  // ---- decode (workspace and static scratch), split plan and workspace size
  int32_t splits = 0;
  size_t bytes = 0;
  CHECK("num splits", kvq_decode_num_splits(&c, 32, 24, 32768, &splits), KVQ_OK, 0);
  CHECK("num splits null", kvq_decode_num_splits(&c, 32, 24, 32768, nullptr), KVQ_ERR_NULL, 0);
  CHECK("ws size", kvq_decode_workspace_size(&c, 32, 24, 32768, 0, &bytes), KVQ_OK, 0);
  if (bytes != (size_t)32 * 4 * splits * 6 * 258 * 4) {
    fprintf(stderr, "FAIL workspace size %zu for %d splits\n", bytes, splits);
    failures++;
  }
  const int32_t* T = (const int32_t*)F;
  CHECK("decode ok", kvq_decode_attention(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, F, 1, nullptr, F, bytes, nullptr),
        KVQ_OK, 6);
  CHECK("decode lse ok",
        kvq_decode_attention(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, F, 0, (float*)F, F, bytes, nullptr), KVQ_OK, 6);
  CHECK("decode q null",
        kvq_decode_attention(&c, nullptr, 24, T, 2048, T, 32, 32768, 0.f, 0, F, 1, nullptr, F, bytes, nullptr),
        KVQ_ERR_NULL, 0);
  CHECK("decode ws null",
        kvq_decode_attention(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, F, 1, nullptr, nullptr, bytes, nullptr),
        KVQ_ERR_NULL, 0);
  CHECK("decode hq", kvq_decode_attention(&c, F, 26, T, 2048, T, 32, 32768, 0.f, 0, F, 1, nullptr, F, bytes, nullptr),
        KVQ_ERR_SHAPE, 0);
  CHECK("decode group 17",
        kvq_decode_attention(&c, F, 68, T, 2048, T, 32, 32768, 0.f, 0, F, 1, nullptr, F, 1ull << 40, nullptr),
        KVQ_ERR_UNSUPPORTED, 0);
  CHECK("decode table", kvq_decode_attention(&c, F, 24, T, 100, T, 32, 32768, 0.f, 0, F, 1, nullptr, F, bytes, nullptr),
        KVQ_ERR_SHAPE, 0);
  CHECK("decode out dtype",
        kvq_decode_attention(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, F, 5, nullptr, F, bytes, nullptr),
        KVQ_ERR_UNSUPPORTED, 0);
  CHECK("decode out align",
        kvq_decode_attention(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, off(F, 4), 1, nullptr, F, bytes, nullptr),
        KVQ_ERR_ALIGN, 0);
  CHECK("decode lse align",
        kvq_decode_attention(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, F, 1, (float*)off(F, 2), F, bytes, nullptr),
        KVQ_ERR_ALIGN, 0);
  CHECK("decode batch 0", kvq_decode_attention(&c, F, 24, T, 2048, T, 0, 32768, 0.f, 0, F, 1, nullptr, F, bytes, nullptr),
        KVQ_ERR_SHAPE, 0);
  CHECK("decode L -1", kvq_decode_attention(&c, F, 24, T, 2048, T, 32, -1, 0.f, 0, F, 1, nullptr, F, bytes, nullptr),
        KVQ_ERR_SHAPE, 0);
  CHECK("decode ws small", kvq_decode_attention(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, F, 1, nullptr, F, 16, nullptr),
        KVQ_ERR_WORKSPACE, 0);
  CHECK("decode ws align",
        kvq_decode_attention(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, F, 1, nullptr, off(F, 8), bytes, nullptr),
        KVQ_ERR_ALIGN, 0);
  CHECK("decode splits 70000",
        kvq_decode_attention(&c, F, 24, T, 1 << 18, T, 1, 1 << 22, 0.f, 70000, F, 1, nullptr, F, 1ull << 40, nullptr),
        KVQ_ERR_UNSUPPORTED, 0);
  CHECK("noalloc ok", kvq_decode_attention_noalloc(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, F, 1, nullptr, nullptr),
        KVQ_OK, 6);
  CHECK("noalloc scratch",
        kvq_decode_attention_noalloc(&c, F, 24, T, 2048, T, 4096, 32768, 0.f, 1, F, 1, nullptr, nullptr),
        KVQ_ERR_SCRATCH, 0);
  CHECK("noalloc out null",
        kvq_decode_attention_noalloc(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, nullptr, 1, nullptr, nullptr),
        KVQ_ERR_NULL, 0);

  // ---- prefix dequant
  CHECK("dequant ok", kvq_dequant_prefix(&c, T, 16, F, F, 1024, nullptr), KVQ_OK, 2);
  CHECK("dequant 0", kvq_dequant_prefix(&c, T, 0, F, F, 1024, nullptr), KVQ_OK, 0);
  CHECK("dequant -1", kvq_dequant_prefix(&c, T, -1, F, F, 1024, nullptr), KVQ_ERR_SHAPE, 0);
  CHECK("dequant table null", kvq_dequant_prefix(&c, nullptr, 16, F, F, 1024, nullptr), KVQ_ERR_NULL, 0);
  CHECK("dequant stride", kvq_dequant_prefix(&c, T, 16, F, F, 512, nullptr), KVQ_ERR_SHAPE, 0);
  CHECK("dequant stride align", kvq_dequant_prefix(&c, T, 16, F, F, 1028, nullptr), KVQ_ERR_ALIGN, 0);
  kvq_cache f8 = cache(KVQ_FMT_FP8_E4M3);
  CHECK("dequant fp8", kvq_dequant_prefix(&f8, T, 16, F, F, 1024, nullptr), KVQ_ERR_UNSUPPORTED, 0);

  // ---- extend (workspace and paged)
  CHECK("extend ok", kvq_extend_attention(F, 6144, 24, F, F, 1024, 4, 256, 100, 64, 0.f, F, 1, 6144, nullptr, nullptr),
        KVQ_OK, 7);
  CHECK("extend n 0", kvq_extend_attention(F, 6144, 24, F, F, 1024, 4, 256, 100, 0, 0.f, F, 1, 6144, nullptr, nullptr),
        KVQ_OK, 0);
  CHECK("extend D 96", kvq_extend_attention(F, 6144, 24, F, F, 1024, 4, 96, 100, 64, 0.f, F, 1, 6144, nullptr, nullptr),
        KVQ_ERR_UNSUPPORTED, 0);
  CHECK("extend heads", kvq_extend_attention(F, 6144, 25, F, F, 1024, 4, 256, 100, 64, 0.f, F, 1, 6144, nullptr, nullptr),
        KVQ_ERR_SHAPE, 0);
  CHECK("extend q stride",
        kvq_extend_attention(F, 100, 24, F, F, 1024, 4, 256, 100, 64, 0.f, F, 1, 6144, nullptr, nullptr), KVQ_ERR_SHAPE,
        0);
  CHECK("extend q align",
        kvq_extend_attention(off(F, 2), 6144, 24, F, F, 1024, 4, 256, 100, 64, 0.f, F, 1, 6144, nullptr, nullptr),
        KVQ_ERR_ALIGN, 0);
  CHECK("paged ok",
        kvq_extend_attention_paged(&c, T, 100, F, 6144, 24, F, F, 1024, 64, 0.f, F, 1, 6144, nullptr, nullptr), KVQ_OK,
        7);
  CHECK("paged table null",
        kvq_extend_attention_paged(&c, nullptr, 100, F, 6144, 24, F, F, 1024, 64, 0.f, F, 1, 6144, nullptr, nullptr),
        KVQ_ERR_NULL, 0);
  CHECK("paged no prefix",
        kvq_extend_attention_paged(&c, nullptr, 0, F, 6144, 24, F, F, 1024, 64, 0.f, F, 1, 6144, nullptr, nullptr),
        KVQ_OK, 7);
  CHECK("paged fp8", kvq_extend_attention_paged(&f8, T, 100, F, 6144, 24, F, F, 1024, 64, 0.f, F, 1, 6144, nullptr,
                                                nullptr),
        KVQ_ERR_UNSUPPORTED, 0);

  // ---- calibration, rotation, bandwidth aids, strings
  CHECK("amax ok", kvq_calibrate_amax(&c, F, F, 1, 1024, 8, (float*)F, nullptr), KVQ_OK, 3);
  CHECK("amax int4", kvq_calibrate_amax(&i4, F, F, 1, 1024, 8, (float*)F, nullptr), KVQ_ERR_UNSUPPORTED, 0);
  CHECK("amax null", kvq_calibrate_amax(&c, F, F, 1, 1024, 8, nullptr, nullptr), KVQ_ERR_NULL, 0);
  CHECK("gs ok", kvq_calibrate_global_scale(&c, (const float*)F, nullptr), KVQ_OK, 4);
  CHECK("rotate ok", kvq_hadamard_rotate(F, 1, 256, F, 0, 256, 10, 256, nullptr), KVQ_OK, 5);
  CHECK("rotate D", kvq_hadamard_rotate(F, 1, 256, F, 0, 256, 10, 64, nullptr), KVQ_ERR_UNSUPPORTED, 0);
  CHECK("rotate stride", kvq_hadamard_rotate(F, 1, 100, F, 0, 256, 10, 256, nullptr), KVQ_ERR_SHAPE, 0);
  CHECK("read ok", kvq_stream_read(F, 4096, (uint32_t*)F, 0, nullptr), KVQ_OK, 8);
  CHECK("read align", kvq_stream_read(F, 4100, (uint32_t*)F, 0, nullptr), KVQ_ERR_ALIGN, 0);
  CHECK("write ok", kvq_stream_write(F, 4096, 7u, 0, nullptr), KVQ_OK, 9);
  CHECK("write null", kvq_stream_write(nullptr, 4096, 7u, 0, nullptr), KVQ_ERR_NULL, 0);
  CHECK("copy ok", kvq_stream_copy(F, off(F, 4096), 4096, 0, nullptr), KVQ_OK, 10);
  CHECK("copy align", kvq_stream_copy(F, off(F, 8), 4096, 0, nullptr), KVQ_ERR_ALIGN, 0);
  CHECK("mfma ok", kvq_mfma_rate(1, 10, 4, (uint32_t*)F, nullptr), KVQ_OK, 11);
  CHECK("mfma null", kvq_mfma_rate(0, 10, 4, nullptr, nullptr), KVQ_ERR_NULL, 0);
  CHECK("mfma mixed", kvq_mfma_rate(2, 10, 4, (uint32_t*)F, nullptr), KVQ_OK, 11);
  CHECK("mfma mode", kvq_mfma_rate(3, 10, 4, (uint32_t*)F, nullptr), KVQ_ERR_UNSUPPORTED, 0);
  CHECK("mfma shape", kvq_mfma_rate(0, 0, 4, (uint32_t*)F, nullptr), KVQ_ERR_SHAPE, 0);
  // ---- debug mode: each call that reads device index arrays runs its check
  // first; reported faults turn into KVQ_ERR_DEVICE_INPUT with no launch
  {
    const int32_t* T = (const int32_t*)F;
    const int checks0 = g_debug_checks;
    CHECK("no debug: store", kvq_quantize_store(&c, F, F, KVQ_DT_BF16, 1024, T, 4, nullptr), KVQ_OK, 1);
    if (g_debug_checks != checks0) {
      fprintf(stderr, "FAIL a check ran without KVQ_DEBUG\n");
      failures++;
    }
    setenv("KVQ_DEBUG", "1", 1);
    size_t dbytes = 0;
    (void)kvq_decode_workspace_size(&c, 32, 24, 32768, 0, &dbytes);
    for (uint32_t bits : {0u, 1u, 2u, 4u}) {
      g_debug_bits = bits;
      const int want = bits ? KVQ_ERR_DEVICE_INPUT : KVQ_OK;
      CHECK("debug store", kvq_quantize_store(&c, F, F, KVQ_DT_BF16, 1024, T, 4, nullptr), want, bits ? 0 : 1);
      CHECK("debug decode",
            kvq_decode_attention(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, F, 1, nullptr, F, dbytes, nullptr), want,
            bits ? 0 : 6);
      CHECK("debug noalloc",
            kvq_decode_attention_noalloc(&c, F, 24, T, 2048, T, 32, 32768, 0.f, 0, F, 1, nullptr, nullptr), want,
            bits ? 0 : 6);
      CHECK("debug dequant", kvq_dequant_prefix(&c, T, 16, F, F, 1024, nullptr), want, bits ? 0 : 2);
      CHECK("debug extend paged",
            kvq_extend_attention_paged(&c, T, 100, F, 24 * 256, 24, F, F, 4 * 256, 8, 0.f, F, 1, 24 * 256, nullptr,
                                       nullptr),
            want, bits ? 0 : 7);
    }
    const int checks1 = g_debug_checks;
    g_debug_bits = 1u;
    CHECK("debug: invalid arguments fail before the check",
          kvq_quantize_store(&c, F, F, 7, 1024, T, 4, nullptr), KVQ_ERR_UNSUPPORTED, 0);
    CHECK("debug: no prefix, no check", kvq_dequant_prefix(&c, T, 0, F, F, 1024, nullptr), KVQ_OK, 0);
    if (g_debug_checks != checks1) {
      fprintf(stderr, "FAIL a check ran for a call rejected or empty on the host\n");
      failures++;
    }
    setenv("KVQ_DEBUG", "0", 1);
    CHECK("debug 0: store", kvq_quantize_store(&c, F, F, KVQ_DT_BF16, 1024, T, 4, nullptr), KVQ_OK, 1);
    unsetenv("KVQ_DEBUG");
    g_debug_bits = 0u;
  }
  for (int s = -8; s <= 1; s++) {
    const char* str = kvq_status_string(s);
    if (str == nullptr || str[0] == 0) {
      fprintf(stderr, "FAIL status string %d\n", s);
      failures++;
    }
  }
  if (kvq_slab_bytes(KVQ_FMT_INT4_TOKHEAD, 1600, 256) != 422400) {
    fprintf(stderr, "FAIL slab bytes\n");
    failures++;
  }
  printf("%d failures, %d launches requested\n", failures, g_launch_count);
  return failures == 0 ? 0 : 1;
}
