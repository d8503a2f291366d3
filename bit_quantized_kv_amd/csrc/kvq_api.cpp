// kvq_api.cpp -- the extern "C" boundary of libkvq: argument validation, the
// split plan and kernel dispatch.  Every host-checkable condition is tested
// before anything touches the GPU, so a rejected call launches nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>

#include "../../include/kvq.h"
#include "kvq_debug.h"
#include "kvq_device.h"
#include "kvq_launch.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr int kDefaultCUs = 256;   // MI355X
constexpr int kMaxDevices = 64;
constexpr int kMinChunksPerWave = 4;    // 128 tokens per wavefront at least
constexpr int kMaxChunksPerWave = 256;  // 8,192 tokens per wavefront at most
constexpr int kStreamWorkgroups = 2048;  // 8 per CU: the best plain streaming read measured on MI355X

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

kvq_status check_cache(const kvq_cache* c) {
  if (c == nullptr || c->pool == nullptr) return KVQ_ERR_NULL;
  if (c->fmt != KVQ_FMT_NVFP4 && c->fmt != KVQ_FMT_INT4_TOKHEAD && c->fmt != KVQ_FMT_FP8_E4M3 &&
      c->fmt != KVQ_FMT_K8V4)
    return KVQ_ERR_UNSUPPORTED;
  if (c->fmt != KVQ_FMT_INT4_TOKHEAD && c->global_scale == nullptr) return KVQ_ERR_NULL;
  if (c->num_pages <= 0 || c->num_kv_heads <= 0 || c->page_size <= 0) return KVQ_ERR_SHAPE;
  if (c->head_dim != 128 && c->head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  if (c->page_size % 16 != 0) return KVQ_ERR_UNSUPPORTED;
  if (!aligned16(c->pool)) return KVQ_ERR_ALIGN;
  if (c->flags & ~KVQ_FLAG_HADAMARD) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

float rotation_scale(int32_t head_dim) { return (float)(1.0 / __builtin_sqrt((double)head_dim)); }

kvq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KVQ_OK;
  g_last_hip_error = (int32_t)e;
  return KVQ_ERR_HIP;
}

// KVQ_DEBUG=1 (read on every call): check the device index arrays before
// launching; the call then waits for its stream.
bool debug_mode() {
  const char* e = getenv("KVQ_DEBUG");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

kvq_status debug_status(hipError_t e, uint32_t bits) {
  if (e != hipSuccess) return hip_status(e);
  return bits != 0u ? KVQ_ERR_DEVICE_INPUT : KVQ_OK;
}

// the page ids of a single prefix row (dequant, fused extend)
kvq_status debug_prefix_row(const kvq_cache* c, const int32_t* row, int32_t prefix_len, void* stream) {
  if (!debug_mode() || prefix_len <= 0) return KVQ_OK;
  uint32_t bits = 0u;
  const hipError_t e = kvq::debug_check_pages(row, 0, 1, nullptr, prefix_len, prefix_len, c->page_size, c->num_pages,
                                              (hipStream_t)stream, &bits);
  return debug_status(e, bits);
}

// Compute units of the current device (queried once per device; 256, an
// MI355X, when no device is visible, e.g. for a host-only planning call).
int device_cus() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = kDefaultCUs;
  }
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Splits per (sequence, KV head): the grid of batch x num_kv_heads x splits
// four-wavefront workgroups is sized to one workgroup per CU for NVFP4 and
// two for INT4 (whose heavier dequantization gains from a second wavefront
// per SIMD); measured best on MI355X at the 32K, 160K, 1M and INT4 220K
// shapes.  Each wavefront keeps at least kMinChunksPerWave chunks and at
// most kMaxChunksPerWave: its output accumulators are MFMA accumulators,
// whose sums keep only about 3 bits below the accumulator's ulp, so the
// number of chunks summed into one is bounded (8,192 tokens).
int32_t auto_splits(int32_t fmt, int32_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
  const int64_t chunks = ((int64_t)max_seq_len + 31) / 32;
  if (chunks <= 0) return 1;
  const int64_t units = (int64_t)batch * num_kv_heads;
  const int64_t target = (int64_t)device_cus() * (fmt == KVQ_FMT_INT4_TOKHEAD ? 2 : 1);
  int64_t s = (target + units / 2) / units;
  const int64_t longest = (int64_t)kMaxChunksPerWave * kvq::kDecodeWaves;
  const int64_t need = (chunks + longest - 1) / longest;
  if (s < need) s = need;
  const int64_t per_split = (int64_t)kMinChunksPerWave * kvq::kDecodeWaves;
  const int64_t cap = (chunks + per_split - 1) / per_split;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int32_t)s;
}

kvq_status decode_shape(const kvq_cache* c, int32_t batch, int32_t num_q_heads, int32_t max_seq_len) {
  kvq_status st = check_cache(c);
  if (st != KVQ_OK) return st;
  if (batch <= 0 || num_q_heads <= 0 || max_seq_len < 0) return KVQ_ERR_SHAPE;
  if (num_q_heads % c->num_kv_heads != 0) return KVQ_ERR_SHAPE;
  if (num_q_heads / c->num_kv_heads > 16) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

size_t workspace_bytes(const kvq_cache* c, int32_t batch, int32_t num_q_heads, int32_t splits) {
  const size_t G = (size_t)(num_q_heads / c->num_kv_heads);
  const size_t parts = (size_t)batch * c->num_kv_heads * splits;
  return parts * G * ((size_t)c->head_dim + 2) * sizeof(float);
}

// Checks shared by both decode entry points (everything but the workspace).
kvq_status decode_args(const kvq_cache* c, const void* q, int32_t num_q_heads, const int32_t* block_table,
                       int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, void* out,
                       int32_t out_dtype, float* lse_out) {
  kvq_status st = decode_shape(c, batch, num_q_heads, max_seq_len);
  if (st != KVQ_OK) return st;
  if (q == nullptr || block_table == nullptr || seq_lens == nullptr || out == nullptr) return KVQ_ERR_NULL;
  if (out_dtype != KVQ_DT_F32 && out_dtype != KVQ_DT_BF16) return KVQ_ERR_UNSUPPORTED;
  if (max_pages <= 0 || (int64_t)max_pages * c->page_size < max_seq_len) return KVQ_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(out) || (lse_out && ((uintptr_t)lse_out & 3u))) return KVQ_ERR_ALIGN;
  if (batch > 65535) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

// The split decode and its merge over `splits` parts, partials in `workspace`.
kvq_status decode_launch(const kvq_cache* cache, const void* q, int32_t num_q_heads, const int32_t* block_table,
                         int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                         float sm_scale, int32_t splits, void* out, int32_t out_dtype, float* lse_out,
                         void* workspace, void* stream) {
  if (debug_mode()) {
    uint32_t bits = 0u;
    const kvq_status st = debug_status(
        kvq::debug_check_pages(block_table, max_pages, batch, seq_lens, 0, max_seq_len, cache->page_size,
                               cache->num_pages, (hipStream_t)stream, &bits),
        bits);
    if (st != KVQ_OK) return st;
  }
  const kvq::SlabLayout lay = kvq::slab_layout(cache->fmt, cache->page_size, cache->head_dim);
  const int64_t chunks = ((int64_t)max_seq_len + 31) / 32;
  kvq::DecodeParams p;
  p.pool = (const uint8_t*)cache->pool;
  p.gs = cache->global_scale;
  p.q = (const uint16_t*)q;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  const int32_t G = num_q_heads / cache->num_kv_heads;
  const size_t parts = (size_t)batch * cache->num_kv_heads * splits;
  p.part_o = (float*)workspace;
  p.part_ml = (float*)workspace + parts * G * cache->head_dim;
  p.out = out;
  p.lse = lse_out;
  p.slab = lay.slab;
  p.half = lay.half;
  p.scales_off = lay.scales_off;
  p.sm_scale = sm_scale > 0.0f ? sm_scale : 1.0f / __builtin_sqrtf((float)cache->head_dim);
  p.max_pages = max_pages;
  p.batch = batch;
  p.num_kv_heads = cache->num_kv_heads;
  p.num_q_heads = num_q_heads;
  p.group = G;
  p.page_size = cache->page_size;
  p.num_splits = splits;
  p.chunks_per_split = (int32_t)((chunks + splits - 1) / splits);
  if (p.chunks_per_split < 1) p.chunks_per_split = 1;
  p.out_bf16 = out_dtype == KVQ_DT_BF16;
  return hip_status(kvq::launch_decode(p, cache->fmt, cache->head_dim, (hipStream_t)stream));
}

}  // namespace

extern "C" {

size_t kvq_slab_bytes(int32_t fmt, int32_t page_size, int32_t head_dim) {
  if ((fmt != KVQ_FMT_NVFP4 && fmt != KVQ_FMT_INT4_TOKHEAD && fmt != KVQ_FMT_FP8_E4M3 && fmt != KVQ_FMT_K8V4) ||
      page_size <= 0 ||
      head_dim <= 0 || head_dim % 16)
    return 0;
  return (size_t)kvq::slab_layout(fmt, page_size, head_dim).slab;
}

kvq_status kvq_quantize_store(const kvq_cache* cache, const void* k, const void* v, int32_t in_dtype,
                              int64_t in_token_stride, const int32_t* slot_mapping, int32_t num_tokens,
                              void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (num_tokens < 0) return KVQ_ERR_SHAPE;
  if (in_dtype != KVQ_DT_F32 && in_dtype != KVQ_DT_BF16) return KVQ_ERR_UNSUPPORTED;
  if (num_tokens == 0) return KVQ_OK;
  if (k == nullptr || v == nullptr || slot_mapping == nullptr) return KVQ_ERR_NULL;
  if (in_token_stride < (int64_t)cache->num_kv_heads * cache->head_dim) return KVQ_ERR_SHAPE;
  const int64_t esize = in_dtype == KVQ_DT_F32 ? 4 : 2;
  if (!aligned16(k) || !aligned16(v) || (in_token_stride * esize) % 16 != 0) return KVQ_ERR_ALIGN;
  if (debug_mode()) {
    uint32_t bits = 0u;
    const kvq_status dst = debug_status(
        kvq::debug_check_slots(slot_mapping, num_tokens, (int64_t)cache->num_pages * cache->page_size,
                               (hipStream_t)stream, &bits),
        bits);
    if (dst != KVQ_OK) return dst;
  }
  const kvq::SlabLayout lay = kvq::slab_layout(cache->fmt, cache->page_size, cache->head_dim);
  kvq::StoreParams p;
  p.pool = (uint8_t*)cache->pool;
  p.gs = cache->global_scale;
  p.k = k;
  p.v = v;
  p.slots = slot_mapping;
  p.in_stride = in_token_stride;
  p.slab = lay.slab;
  p.half = lay.half;
  p.scales_off = lay.scales_off;
  p.num_tokens = num_tokens;
  p.page_size = cache->page_size;
  p.num_kv_heads = cache->num_kv_heads;
  p.rotate = (cache->flags & KVQ_FLAG_HADAMARD) != 0;
  p.rot_scale = rotation_scale(cache->head_dim);
  return hip_status(kvq::launch_quantize_store(p, cache->fmt, cache->head_dim, in_dtype == KVQ_DT_BF16,
                                               (hipStream_t)stream));
}

kvq_status kvq_decode_num_splits(const kvq_cache* cache, int32_t batch, int32_t num_q_heads, int32_t max_seq_len,
                                 int32_t* num_splits) {
  if (num_splits == nullptr) return KVQ_ERR_NULL;
  kvq_status st = decode_shape(cache, batch, num_q_heads, max_seq_len);
  if (st != KVQ_OK) return st;
  *num_splits = auto_splits(cache->fmt, batch, cache->num_kv_heads, max_seq_len);
  return KVQ_OK;
}

kvq_status kvq_decode_workspace_size(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                                     int32_t max_seq_len, int32_t num_splits, size_t* bytes) {
  if (bytes == nullptr) return KVQ_ERR_NULL;
  kvq_status st = decode_shape(cache, batch, num_q_heads, max_seq_len);
  if (st != KVQ_OK) return st;
  const int32_t s = num_splits > 0 ? num_splits : auto_splits(cache->fmt, batch, cache->num_kv_heads, max_seq_len);
  *bytes = workspace_bytes(cache, batch, num_q_heads, s);
  return KVQ_OK;
}

kvq_status kvq_decode_attention(const kvq_cache* cache, const void* q, int32_t num_q_heads,
                                const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                                int32_t batch, int32_t max_seq_len, float sm_scale, int32_t num_splits, void* out,
                                int32_t out_dtype, float* lse_out, void* workspace, size_t workspace_bytes_,
                                void* stream) {
  kvq_status st = decode_args(cache, q, num_q_heads, block_table, max_pages, seq_lens, batch, max_seq_len, out,
                              out_dtype, lse_out);
  if (st != KVQ_OK) return st;
  if (workspace == nullptr) return KVQ_ERR_NULL;
  if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
  const int32_t splits = num_splits > 0 ? num_splits : auto_splits(cache->fmt, batch, cache->num_kv_heads, max_seq_len);
  if (splits > 65535) return KVQ_ERR_UNSUPPORTED;
  if (workspace_bytes_ < workspace_bytes(cache, batch, num_q_heads, splits)) return KVQ_ERR_WORKSPACE;
  return decode_launch(cache, q, num_q_heads, block_table, max_pages, seq_lens, batch, max_seq_len, sm_scale, splits,
                       out, out_dtype, lse_out, workspace, stream);
}

kvq_status kvq_decode_attention_noalloc(const kvq_cache* cache, const void* q, int32_t num_q_heads,
                                        const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                                        int32_t batch, int32_t max_seq_len, float sm_scale, int32_t num_splits,
                                        void* out, int32_t out_dtype, float* lse_out, void* stream) {
  kvq_status st = decode_args(cache, q, num_q_heads, block_table, max_pages, seq_lens, batch, max_seq_len, out,
                              out_dtype, lse_out);
  if (st != KVQ_OK) return st;
  const int32_t splits = num_splits > 0 ? num_splits : auto_splits(cache->fmt, batch, cache->num_kv_heads, max_seq_len);
  if (splits > 65535) return KVQ_ERR_UNSUPPORTED;
  if (workspace_bytes(cache, batch, num_q_heads, splits) > kvq::kDecodeScratchBytes) return KVQ_ERR_SCRATCH;
  void* scratch = nullptr;
  const kvq_status sst = hip_status(kvq::decode_scratch(&scratch));
  if (sst != KVQ_OK) return sst;
  return decode_launch(cache, q, num_q_heads, block_table, max_pages, seq_lens, batch, max_seq_len, sm_scale, splits,
                       out, out_dtype, lse_out, scratch, stream);
}

kvq_status kvq_dequant_prefix(const kvq_cache* cache, const int32_t* block_table_row, int32_t prefix_len,
                              void* k_out, void* v_out, int64_t out_token_stride, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (cache->fmt == KVQ_FMT_FP8_E4M3 || cache->fmt == KVQ_FMT_K8V4) return KVQ_ERR_UNSUPPORTED;
  if (prefix_len < 0) return KVQ_ERR_SHAPE;
  if (prefix_len == 0) return KVQ_OK;
  if (block_table_row == nullptr || k_out == nullptr || v_out == nullptr) return KVQ_ERR_NULL;
  if (out_token_stride < (int64_t)cache->num_kv_heads * cache->head_dim) return KVQ_ERR_SHAPE;
  if (!aligned16(k_out) || !aligned16(v_out) || (out_token_stride * 2) % 16 != 0) return KVQ_ERR_ALIGN;
  st = debug_prefix_row(cache, block_table_row, prefix_len, stream);
  if (st != KVQ_OK) return st;
  const kvq::SlabLayout lay = kvq::slab_layout(cache->fmt, cache->page_size, cache->head_dim);
  kvq::DequantParams p;
  p.pool = (const uint8_t*)cache->pool;
  p.gs = cache->global_scale;
  p.pages = block_table_row;
  p.k_out = (uint16_t*)k_out;
  p.v_out = (uint16_t*)v_out;
  p.out_stride = out_token_stride;
  p.slab = lay.slab;
  p.half = lay.half;
  p.scales_off = lay.scales_off;
  p.prefix_len = prefix_len;
  p.page_size = cache->page_size;
  p.num_kv_heads = cache->num_kv_heads;
  return hip_status(kvq::launch_dequant_prefix(p, cache->fmt, cache->head_dim, (hipStream_t)stream));
}

kvq_status kvq_calibrate_amax(const kvq_cache* cache, const void* k, const void* v, int32_t in_dtype,
                              int64_t in_token_stride, int32_t num_tokens, float* running_amax, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (cache->fmt != KVQ_FMT_NVFP4) return KVQ_ERR_UNSUPPORTED;
  if (num_tokens < 0) return KVQ_ERR_SHAPE;
  if (in_dtype != KVQ_DT_F32 && in_dtype != KVQ_DT_BF16) return KVQ_ERR_UNSUPPORTED;
  if (running_amax == nullptr) return KVQ_ERR_NULL;
  if (num_tokens == 0) return KVQ_OK;
  if (k == nullptr || v == nullptr) return KVQ_ERR_NULL;
  if (in_token_stride < (int64_t)cache->num_kv_heads * cache->head_dim) return KVQ_ERR_SHAPE;
  const int64_t esize = in_dtype == KVQ_DT_F32 ? 4 : 2;
  if (!aligned16(k) || !aligned16(v) || (in_token_stride * esize) % 16 != 0 || ((uintptr_t)running_amax & 3u))
    return KVQ_ERR_ALIGN;
  kvq::StoreParams p{};
  p.k = k;
  p.v = v;
  p.in_stride = in_token_stride;
  p.num_tokens = num_tokens;
  p.num_kv_heads = cache->num_kv_heads;
  p.rotate = (cache->flags & KVQ_FLAG_HADAMARD) != 0;
  p.rot_scale = rotation_scale(cache->head_dim);
  return hip_status(kvq::launch_calibrate_amax(p, cache->head_dim, in_dtype == KVQ_DT_BF16, running_amax,
                                               (hipStream_t)stream));
}

kvq_status kvq_calibrate_global_scale(const kvq_cache* cache, const float* running_amax, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (cache->fmt != KVQ_FMT_NVFP4) return KVQ_ERR_UNSUPPORTED;
  if (running_amax == nullptr) return KVQ_ERR_NULL;
  if (((uintptr_t)running_amax & 3u) || ((uintptr_t)cache->global_scale & 3u)) return KVQ_ERR_ALIGN;
  return hip_status(kvq::launch_global_scale(running_amax, (float*)cache->global_scale, (hipStream_t)stream));
}

kvq_status kvq_extend_attention(const void* q, int64_t q_token_stride, int32_t num_q_heads, const void* k_ws,
                                const void* v_ws, int64_t kv_token_stride, int32_t num_kv_heads, int32_t head_dim,
                                int32_t prefix_len, int32_t chunk_len, float sm_scale, void* out, int32_t out_dtype,
                                int64_t out_token_stride, float* lse_out, void* stream) {
  if (prefix_len < 0 || chunk_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0) return KVQ_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return KVQ_ERR_SHAPE;
  if (head_dim != 128 && head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  if (out_dtype != KVQ_DT_F32 && out_dtype != KVQ_DT_BF16) return KVQ_ERR_UNSUPPORTED;
  if (num_kv_heads > 65535) return KVQ_ERR_UNSUPPORTED;
  if (chunk_len == 0) return KVQ_OK;
  if (q == nullptr || k_ws == nullptr || v_ws == nullptr || out == nullptr) return KVQ_ERR_NULL;
  if (q_token_stride < (int64_t)num_q_heads * head_dim || kv_token_stride < (int64_t)num_kv_heads * head_dim ||
      out_token_stride < (int64_t)num_q_heads * head_dim)
    return KVQ_ERR_SHAPE;
  const int64_t oes = out_dtype == KVQ_DT_F32 ? 4 : 2;
  if (!aligned16(q) || !aligned16(k_ws) || !aligned16(v_ws) || !aligned16(out) || (q_token_stride * 2) % 16 ||
      (kv_token_stride * 2) % 16 || (out_token_stride * oes) % 16 || (lse_out && ((uintptr_t)lse_out & 3u)))
    return KVQ_ERR_ALIGN;
  const int64_t rows = (int64_t)chunk_len * (num_q_heads / num_kv_heads);
  if ((rows + 63) / 64 > 0x7FFFFFFF) return KVQ_ERR_UNSUPPORTED;
  kvq::ExtendParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k_ws;
  p.v = (const uint16_t*)v_ws;
  p.out = out;
  p.lse = lse_out;
  p.q_stride = q_token_stride;
  p.kv_stride = kv_token_stride;
  p.out_stride = out_token_stride;
  p.lse_stride = num_q_heads;
  p.sm_scale = sm_scale > 0.0f ? sm_scale : 1.0f / __builtin_sqrtf((float)head_dim);
  p.prefix_len = prefix_len;
  p.chunk_len = chunk_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.out_bf16 = out_dtype == KVQ_DT_BF16;
  return hip_status(kvq::launch_extend(p, head_dim, 0, (hipStream_t)stream));
}

kvq_status kvq_extend_attention_paged(const kvq_cache* cache, const int32_t* block_table_row, int32_t prefix_len,
                                      const void* q, int64_t q_token_stride, int32_t num_q_heads, const void* k_chunk,
                                      const void* v_chunk, int64_t chunk_token_stride, int32_t chunk_len,
                                      float sm_scale, void* out, int32_t out_dtype, int64_t out_token_stride,
                                      float* lse_out, void* stream) {
  kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (cache->fmt == KVQ_FMT_FP8_E4M3 || cache->fmt == KVQ_FMT_K8V4) return KVQ_ERR_UNSUPPORTED;
  const int32_t Hkv = cache->num_kv_heads, D = cache->head_dim;
  if (prefix_len < 0 || chunk_len < 0 || num_q_heads <= 0 || num_q_heads % Hkv != 0) return KVQ_ERR_SHAPE;
  if (out_dtype != KVQ_DT_F32 && out_dtype != KVQ_DT_BF16) return KVQ_ERR_UNSUPPORTED;
  if (Hkv > 65535) return KVQ_ERR_UNSUPPORTED;
  if (chunk_len == 0) return KVQ_OK;
  if (q == nullptr || k_chunk == nullptr || v_chunk == nullptr || out == nullptr) return KVQ_ERR_NULL;
  if (prefix_len > 0 && block_table_row == nullptr) return KVQ_ERR_NULL;
  if (q_token_stride < (int64_t)num_q_heads * D || chunk_token_stride < (int64_t)Hkv * D ||
      out_token_stride < (int64_t)num_q_heads * D)
    return KVQ_ERR_SHAPE;
  const int64_t oes = out_dtype == KVQ_DT_F32 ? 4 : 2;
  if (!aligned16(q) || !aligned16(k_chunk) || !aligned16(v_chunk) || !aligned16(out) || (q_token_stride * 2) % 16 ||
      (chunk_token_stride * 2) % 16 || (out_token_stride * oes) % 16 || (lse_out && ((uintptr_t)lse_out & 3u)))
    return KVQ_ERR_ALIGN;
  const int64_t rows = (int64_t)chunk_len * (num_q_heads / Hkv);
  if ((rows + 63) / 64 > 0x7FFFFFFF) return KVQ_ERR_UNSUPPORTED;
  const kvq::SlabLayout lay = kvq::slab_layout(cache->fmt, cache->page_size, D);
  if (lay.slab > 0x7FFFFFFF) return KVQ_ERR_UNSUPPORTED;  // a page's slab is addressed with 32-bit offsets
  st = debug_prefix_row(cache, block_table_row, prefix_len, stream);
  if (st != KVQ_OK) return st;
  kvq::ExtendParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k_chunk;
  p.v = (const uint16_t*)v_chunk;
  p.out = out;
  p.lse = lse_out;
  p.q_stride = q_token_stride;
  p.kv_stride = chunk_token_stride;
  p.out_stride = out_token_stride;
  p.lse_stride = num_q_heads;
  p.sm_scale = sm_scale > 0.0f ? sm_scale : 1.0f / __builtin_sqrtf((float)D);
  p.prefix_len = prefix_len;
  p.chunk_len = chunk_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = Hkv;
  p.group = num_q_heads / Hkv;
  p.out_bf16 = out_dtype == KVQ_DT_BF16;
  p.pool = (const uint8_t*)cache->pool;
  p.gs = cache->global_scale;
  p.pages = block_table_row;
  p.slab = lay.slab;
  p.half = lay.half;
  p.scales_off = lay.scales_off;
  p.page_size = cache->page_size;
  return hip_status(kvq::launch_extend(p, D, cache->fmt, (hipStream_t)stream));
}

kvq_status kvq_hadamard_rotate(const void* in, int32_t in_dtype, int64_t in_row_stride, void* out, int32_t out_dtype,
                               int64_t out_row_stride, int32_t rows, int32_t head_dim, void* stream) {
  if (rows < 0) return KVQ_ERR_SHAPE;
  if (head_dim != 128 && head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  if ((in_dtype != KVQ_DT_F32 && in_dtype != KVQ_DT_BF16) || (out_dtype != KVQ_DT_F32 && out_dtype != KVQ_DT_BF16))
    return KVQ_ERR_UNSUPPORTED;
  if (rows == 0) return KVQ_OK;
  if (in == nullptr || out == nullptr) return KVQ_ERR_NULL;
  if (in_row_stride < head_dim || out_row_stride < head_dim) return KVQ_ERR_SHAPE;
  const int64_t ies = in_dtype == KVQ_DT_F32 ? 4 : 2, oes = out_dtype == KVQ_DT_F32 ? 4 : 2;
  if (!aligned16(in) || !aligned16(out) || (in_row_stride * ies) % 16 || (out_row_stride * oes) % 16)
    return KVQ_ERR_ALIGN;
  kvq::RotateParams p;
  p.in = in;
  p.out = out;
  p.in_stride = in_row_stride;
  p.out_stride = out_row_stride;
  p.rows = rows;
  p.scale = rotation_scale(head_dim);
  return hip_status(kvq::launch_hadamard(p, head_dim, in_dtype == KVQ_DT_BF16, out_dtype == KVQ_DT_BF16,
                                         (hipStream_t)stream));
}

kvq_status kvq_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t num_workgroups, void* stream) {
  if (bytes == 0) return KVQ_OK;
  if (buf == nullptr || sink == nullptr) return KVQ_ERR_NULL;
  if (!aligned16(buf) || bytes % 16 != 0 || ((uintptr_t)sink & 3u)) return KVQ_ERR_ALIGN;
  if (num_workgroups > 65535 * 64) return KVQ_ERR_UNSUPPORTED;
  const int wgs = num_workgroups > 0 ? num_workgroups : kStreamWorkgroups;
  return hip_status(kvq::launch_stream_read(buf, (int64_t)bytes, sink, wgs, (hipStream_t)stream));
}

kvq_status kvq_stream_write(void* buf, size_t bytes, uint32_t value, int32_t num_workgroups, void* stream) {
  if (bytes == 0) return KVQ_OK;
  if (buf == nullptr) return KVQ_ERR_NULL;
  if (!aligned16(buf) || bytes % 16 != 0) return KVQ_ERR_ALIGN;
  if (num_workgroups > 65535 * 64) return KVQ_ERR_UNSUPPORTED;
  const int wgs = num_workgroups > 0 ? num_workgroups : kStreamWorkgroups;
  return hip_status(kvq::launch_stream_write(buf, (int64_t)bytes, value, wgs, (hipStream_t)stream));
}

kvq_status kvq_stream_copy(const void* src, void* dst, size_t bytes, int32_t num_workgroups, void* stream) {
  if (bytes == 0) return KVQ_OK;
  if (src == nullptr || dst == nullptr) return KVQ_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst) || bytes % 16 != 0) return KVQ_ERR_ALIGN;
  if (num_workgroups > 65535 * 64) return KVQ_ERR_UNSUPPORTED;
  const int wgs = num_workgroups > 0 ? num_workgroups : kStreamWorkgroups;
  return hip_status(kvq::launch_stream_copy(src, dst, (int64_t)bytes, wgs, (hipStream_t)stream));
}

kvq_status kvq_mfma_rate(int32_t lds_operands, int32_t iterations, int32_t num_workgroups, uint32_t* sink,
                         void* stream) {
  if (sink == nullptr) return KVQ_ERR_NULL;
  if (lds_operands < 0 || lds_operands > 2) return KVQ_ERR_UNSUPPORTED;
  if (iterations <= 0 || num_workgroups <= 0) return KVQ_ERR_SHAPE;
  return hip_status(kvq::launch_mfma_rate(lds_operands, iterations, num_workgroups, sink, (hipStream_t)stream));
}

const char* kvq_status_string(int32_t status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "a required pointer is NULL";
    case KVQ_ERR_SHAPE: return "inconsistent sizes or strides";
    case KVQ_ERR_UNSUPPORTED: return "format or shape outside the supported limits";
    case KVQ_ERR_ALIGN: return "a pointer or stride is not 16-byte aligned";
    case KVQ_ERR_WORKSPACE: return "workspace smaller than kvq_decode_workspace_size";
    case KVQ_ERR_HIP: return "HIP launch failed (see kvq_last_hip_error)";
    case KVQ_ERR_SCRATCH: return "decode partials exceed the static scratch of kvq_decode_attention_noalloc";
    case KVQ_ERR_DEVICE_INPUT: return "a slot, page id or sequence length in a device array is out of range (KVQ_DEBUG)";
    default: return "unknown status";
  }
}

int32_t kvq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
