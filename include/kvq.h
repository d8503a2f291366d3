/*
 * kvq.h -- C ABI of libkvq, a 4-bit paged KV cache for MI355X (gfx950).
 *
 * Three operations make up the hot path, as the pages describe it:
 *   kvq_quantize_store    quantize new K/V rows into cache pages on write
 *   kvq_decode_attention  decode attention that reads the 4-bit pages
 *                         directly and dequantizes inside the kernel
 *   kvq_dequant_prefix    expand a cached prefix into a bf16 workspace
 * ("SGLang's 4-bit KV cache: the 56% is exact, the 1.78x is untested",
 * Figure 2 caption: one shared pool, prefill quantizes and stores into it,
 * decode reads NVFP4 directly, chunked prefill/extend dequantizes the cached
 * prefix into a reused workspace.)
 *
 * Formats
 *   KVQ_FMT_NVFP4: E2M1 elements packed two per byte, one E4M3 (OCP, max 448)
 *     scale per 16 consecutive head-dim elements of a token row, and one FP32
 *     global scale per layer for K and one for V -- 9 bytes per 16 values,
 *     0.5625 of FP8 (same page, section "The 56% survives its own scale, and
 *     names the block size").
 *   KVQ_FMT_INT4_TOKHEAD: symmetric int4 (range -7..7, two's-complement
 *     nibbles) with one FP32 scale per token and KV head, for K and for V --
 *     264 bytes per head and token at head dim 256 ("KV cache in 4 bits: 8.8
 *     instead of 4.7 full sessions on the same four RTX 5090s", section "What
 *     we changed").
 *   KVQ_FMT_FP8_E4M3 (the comparator): one E4M3 byte per value with one FP32
 *     scale per tensor (K and V of a layer) -- the per-tensor-scaled FP8 cache
 *     the 0.5625 ratio is measured against ("SGLang's 4-bit KV cache ...",
 *     section "The 56% survives its own scale, and names the block size").
 *     code = E4M3(fp32(x / s)) with the sign kept, saturating at 448.  Store
 *     and decode only (kvq_dequant_prefix and calibration: UNSUPPORTED).
 *   KVQ_FMT_K8V4: FP8 keys with NVFP4 values -- the split-precision 4-bit
 *     cache ("SGLang's 4-bit KV cache ...", section "Against what this site
 *     already established": another engine keeps keys in FP8 and values in 4
 *     bits, twice the bits on keys; its 4-bit value format is not stated and
 *     NVFP4 is taken).  Keys as KVQ_FMT_FP8_E4M3's (by token, per-tensor
 *     scale global_scale[0]); values as KVQ_FMT_NVFP4's (global scale
 *     global_scale[1]); 400 bytes per token and head at head dim 256.  Store
 *     and decode only.  With KVQ_FLAG_HADAMARD it is that engine's rotated
 *     design.
 *   Quantization rules (4-bit formats): block/row amax; NVFP4 scale
 *   E4M3(fp32(amax / fp32(6 * gs))), elements rounded to nearest-even under the
 *   stored scale fp32(E4M3 * gs), |x| >= 6 saturating; INT4 scale
 *   fp32(amax / 7), q = clamp(rint(fp32(x / s)), -7, 7).  Even element in the
 *   low nibble.  All decisions in IEEE fp32, so packed bytes are bit-exact.
 *
 * Pool layout (one layer): uint8 [num_pages][num_kv_heads][slab], where a
 * slab is one page of one KV head:
 *   [K codes: page_size rows of head_dim/2 bytes][K scales]
 *   [V codes: page_size rows of head_dim/2 bytes][V scales]
 * Scales are page_size rows of head_dim/16 E4M3 bytes (NVFP4) or page_size
 * fp32 values (INT4).  FP8 slabs are [K: page_size rows of head_dim bytes]
 * [V: head_dim rows (channels) of page_size bytes], values stored by channel
 * as in paged-attention value caches.  K8V4 slabs are [K: page_size rows of
 * head_dim bytes][V codes: page_size rows of head_dim/2 bytes][V scales:
 * page_size rows of head_dim/16 bytes].  Cache token t of a sequence lives in page
 * block_table[t / page_size] at row t % page_size; a write slot is
 * page * page_size + row.
 *
 * Conventions
 *   - The caller owns all memory.  The library allocates and frees nothing and
 *     keeps no state between calls beyond per-device constants it looks up
 *     once (compute-unit count, kernel attributes), the static decode
 *     scratch of kvq_decode_attention_noalloc (16 MiB per device, a device
 *     array of the library itself) and debug mode's 4-byte result word.
 *   - All work is enqueued on the caller's HIP stream (`stream`, a
 *     hipStream_t; NULL = the default stream) and is asynchronous.  The calls
 *     record nothing but kernel launches (no allocation, copy or memset), so
 *     they can be captured into a HIP graph and replayed (debug mode below
 *     excepted).
 *   - Every host-checkable condition is validated before any launch; a
 *     failing call returns a negative kvq_status and launches nothing.  A
 *     failed launch returns KVQ_ERR_HIP; kvq_last_hip_error() then gives the
 *     hipError_t of the calling thread.  Nothing throws and nothing prints.
 *   - Contents of device arrays (slots, page ids, sequence lengths) are not
 *     validated: out-of-range values are undefined behaviour, as an
 *     out-of-bounds index would be.  Two tokens written to one slot in one call
 *     leave an unspecified winner.
 *   - Debug mode: with the environment variable KVQ_DEBUG set to 1 (read on
 *     every call), the calls that read device index arrays check them on the
 *     device first -- kvq_quantize_store: every slot below num_pages *
 *     page_size; the decode calls: every seq_lens[b] in [0, max_seq_len] and
 *     the page ids those lengths use in [0, num_pages); kvq_dequant_prefix
 *     and kvq_extend_attention_paged: the prefix's page ids in [0, num_pages)
 *     -- then wait for the stream and return KVQ_ERR_DEVICE_INPUT, launching
 *     nothing else, if any entry is out of range.  The check's result word is
 *     a device word of the library (one per device, looked up once with
 *     hipGetSymbolAddress); the call records a copy and a stream
 *     synchronisation, so debug mode is for eager use, not graph capture.
 *   - Limits: head_dim in {128, 256}; page_size a positive multiple of 16;
 *     num_q_heads a multiple of num_kv_heads with group size <= 16; device
 *     pointers 16-byte aligned; token strides keep rows 16-byte aligned.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = -1,        /* a required pointer is NULL */
  KVQ_ERR_SHAPE = -2,       /* inconsistent sizes or strides */
  KVQ_ERR_UNSUPPORTED = -3, /* outside the supported formats / limits */
  KVQ_ERR_ALIGN = -4,       /* a pointer or stride breaks 16-byte alignment */
  KVQ_ERR_WORKSPACE = -5,   /* workspace smaller than kvq_decode_workspace_size */
  KVQ_ERR_HIP = -6,         /* a HIP launch failed; see kvq_last_hip_error() */
  KVQ_ERR_SCRATCH = -7,     /* kvq_decode_attention_noalloc: the shape needs more
                               than its static scratch (16 MiB) */
  KVQ_ERR_DEVICE_INPUT = -8 /* KVQ_DEBUG=1 only: a slot, page id or sequence
                               length in a device array is out of range */
} kvq_status;

typedef enum { KVQ_FMT_NVFP4 = 1, KVQ_FMT_INT4_TOKHEAD = 2, KVQ_FMT_FP8_E4M3 = 3, KVQ_FMT_K8V4 = 4 } kvq_format;

typedef enum { KVQ_DT_F32 = 0, KVQ_DT_BF16 = 1 } kvq_dtype;

/* One layer's cache.  A host struct, read only during a call. */
typedef struct {
  int32_t fmt;                /* kvq_format */
  int32_t num_pages;          /* pages in the pool */
  int32_t page_size;          /* tokens per page (multiple of 16) */
  int32_t num_kv_heads;
  int32_t head_dim;           /* 128 or 256 */
  void* pool;                 /* device, uint8 [num_pages][num_kv_heads][slab] */
  const float* global_scale;  /* device float[2] = {gs_K, gs_V}, positive and
                                 finite; NVFP4 global scales, FP8 per-tensor
                                 scales, K8V4 {FP8 key scale, NVFP4 value
                                 global scale} (ignored for INT4) */
  int32_t flags;              /* 0, or KVQ_FLAG_HADAMARD */
} kvq_cache;

/* Rotated cache ("SGLang's 4-bit KV cache ...", section "Against what this
 * site already established": rotate every vector by an orthogonal matrix
 * before quantizing it, as TurboQuant argues; another engine's 4-bit cache
 * applies a fixed FP32 D256 Hadamard rotation to both operands).  With this
 * flag every K and V row is multiplied by R = H_D / sqrt(D) (Sylvester
 * Hadamard matrix; the fast transform's stages in order in fp32, the scale
 * last) before it is quantized; calibration sees the rotated rows and prefix
 * dequantization returns them.  Decode is unchanged: since R is orthogonal
 * and its own inverse, attention over the rotated cache with the rotated
 * query R q yields R o, so callers pass R q (kvq_hadamard_rotate) and rotate
 * the output back the same way. */
#define KVQ_FLAG_HADAMARD 1

/* Bytes of one slab (one page of one KV head, K and V with their scales);
 * 0 for an unknown format or a head_dim not divisible by 16.
 * NVFP4: 2 * page_size * (head_dim/2 + head_dim/16); INT4: 2 * page_size *
 * (head_dim/2 + 4), i.e. 422,400 bytes for a 1,600-token page at head dim
 * 256, the page size "KV cache in 4 bits ..." ("What we changed") prints;
 * FP8: 2 * page_size * head_dim; K8V4: page_size * (head_dim + head_dim/2 +
 * head_dim/16). */
size_t kvq_slab_bytes(int32_t fmt, int32_t page_size, int32_t head_dim);

/* Quantize-on-write ("SGLang's 4-bit KV cache ...", Figure 2 caption: prefill
 * quantizes and stores into the cache; decode writes the new token's K/V).
 *   k, v            device, [num_tokens][token stride] rows; head g of token i
 *                   starts at element i * in_token_stride + g * head_dim
 *   in_dtype        KVQ_DT_F32 or KVQ_DT_BF16 (bf16 is widened exactly)
 *   in_token_stride elements between tokens, >= num_kv_heads * head_dim
 *   slot_mapping    device int32 [num_tokens]; slot < 0 skips the token
 * Writes each (token, head) K row and V row -- codes and scales -- into its
 * slot.  NVFP4, FP8 and K8V4 read cache->global_scale.  num_tokens == 0 is a
 * no-op. */
kvq_status kvq_quantize_store(const kvq_cache* cache, const void* k, const void* v, int32_t in_dtype,
                              int64_t in_token_stride, const int32_t* slot_mapping, int32_t num_tokens,
                              void* stream);

/* The split count kvq_decode_attention uses when num_splits <= 0: each
 * (sequence, KV head) is cut into that many token ranges of whole 32-token
 * chunks, sized from (format, batch, num_kv_heads, max_seq_len) and the
 * current device's compute-unit count (256 when no device is visible) so the
 * grid holds about one workgroup per CU (NVFP4, FP8, K8V4) or two (INT4). */
kvq_status kvq_decode_num_splits(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                                 int32_t max_seq_len, int32_t* num_splits);

/* Workspace bytes kvq_decode_attention needs for this shape and split count
 * (num_splits <= 0: the automatic count).  Per (sequence, KV head, split) it
 * holds the unnormalised partial output and (max, sum) of each query head. */
kvq_status kvq_decode_workspace_size(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                                     int32_t max_seq_len, int32_t num_splits, size_t* bytes);

/* Paged decode attention over the 4-bit cache ("SGLang's 4-bit KV cache ...",
 * Figure 2 caption: decode reads NVFP4 directly and dequantizes inside the
 * kernel).  For each sequence b and query head h (KV head h / G, G =
 * num_q_heads / num_kv_heads):
 *     o = softmax(sm_scale * q K^T) V,   lse = log sum exp(sm_scale * q K^T)
 * over the seq_lens[b] cached tokens, all read back from the 4-bit pages (no
 * causal mask: one decode query sees every cached token).  The token range is
 * split into num_splits parts (<= 0: automatic); each part yields a partial
 * (o, max, sum) and a second kernel merges them by the log-sum-exp rule in a
 * fixed order, so results are bitwise reproducible for a fixed split count.
 *   q            device bf16 [batch][num_q_heads][head_dim]
 *   block_table  device int32 [batch][max_pages]; only the first
 *                ceil(seq_lens[b] / page_size) entries of a row are read (the
 *                reads are bounded by max_pages: an index past the row, from a
 *                seq_lens value above max_pages * page_size, reads page 0)
 *   seq_lens     device int32 [batch], each in [0, max_seq_len]; 0 gives o = 0
 *                and lse = -inf
 *   max_seq_len  host upper bound of seq_lens, fixes the split plan
 *   sm_scale     softmax scale; <= 0 means 1/sqrt(head_dim)
 *   out          device [batch][num_q_heads][head_dim], bf16 (round to nearest
 *                even) or fp32 per out_dtype
 *   lse_out      device fp32 [batch][num_q_heads] (natural log), or NULL
 *   workspace    device scratch of at least kvq_decode_workspace_size bytes,
 *                16-byte aligned; its contents need no initialisation */
kvq_status kvq_decode_attention(const kvq_cache* cache, const void* q, int32_t num_q_heads,
                                const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                                int32_t batch, int32_t max_seq_len, float sm_scale, int32_t num_splits, void* out,
                                int32_t out_dtype, float* lse_out, void* workspace, size_t workspace_bytes,
                                void* stream);

/* kvq_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels and split plan,
 * so the results equal kvq_decode_attention's for the same num_splits
 * bit for bit; the split partials go to a static scratch array of the library
 * instead: 16 MiB per device, held from the first call on a device until the
 * process ends (kvq_decode_workspace_size gives a shape's need; a larger need
 * returns KVQ_ERR_SCRATCH and launches nothing).  The first call on a device
 * looks the array's device address up once (hipGetSymbolAddress); no call
 * allocates or frees.  Every call on a device shares that device's array, so
 * calls that overlap on one device (different streams or threads, without
 * ordering between them) race and give undefined results; calls ordered on
 * one stream are safe.  The array needs no clearing: every call writes all of
 * the partials it reads. */
kvq_status kvq_decode_attention_noalloc(const kvq_cache* cache, const void* q, int32_t num_q_heads,
                                        const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                                        int32_t batch, int32_t max_seq_len, float sm_scale, int32_t num_splits,
                                        void* out, int32_t out_dtype, float* lse_out, void* stream);

/* Prefix dequantization for chunked prefill / extend ("SGLang's 4-bit KV cache
 * ...", Figure 2 caption: the cached prefix is dequantized into a reused
 * workspace -- bf16 here).  Cache tokens [0, prefix_len) of the sequence whose
 * page list is block_table_row become rows of k_out and v_out:
 *     NVFP4: bf16_rne(fp32(fp32(e2m1 * e4m3) * gs))   (exact when gs == 1)
 *     INT4:  bf16_rne(fp32(q * s))
 *   block_table_row  device int32 [ceil(prefix_len / page_size)]
 *   k_out, v_out     device bf16; head g of token t at element
 *                    t * out_token_stride + g * head_dim
 *   out_token_stride elements, >= num_kv_heads * head_dim
 * prefix_len == 0 is a no-op.  NVFP4 and INT4 caches (FP8, K8V4:
 * KVQ_ERR_UNSUPPORTED). */
kvq_status kvq_dequant_prefix(const kvq_cache* cache, const int32_t* block_table_row, int32_t prefix_len,
                              void* k_out, void* v_out, int64_t out_token_stride, void* stream);

/* Extend attention over the bf16 workspace ("SGLang's 4-bit KV cache ...",
 * Figure 2 caption: chunked prefill / extend dequantizes the cached prefix
 * into a reused workspace and attends over prefix plus current chunk).
 *   k_ws, v_ws  device bf16 [prefix_len + chunk_len][kv_token_stride]: rows
 *               [0, prefix_len) hold the prefix (kvq_dequant_prefix), rows
 *               [prefix_len, prefix_len + chunk_len) the chunk's own K / V;
 *               head g of a row at element g * head_dim
 *   q           device bf16 [chunk_len][q_token_stride], head h at h * head_dim
 *   out         device [chunk_len][out_token_stride], bf16 or fp32 per out_dtype
 *   lse_out     device fp32 [chunk_len][num_q_heads] (natural log), or NULL
 * Chunk query i (sequence position prefix_len + i) of head h attends to the
 * keys 0 .. prefix_len + i of KV head h / (num_q_heads / num_kv_heads) with
 * softmax(sm_scale q k); sm_scale <= 0 means 1/sqrt(head_dim).  head_dim 128
 * or 256; chunk_len == 0 is a no-op.  The path is the workspace variant of the
 * pages' extend step (bf16 here instead of FP8, lossless at gs = 1). */
kvq_status kvq_extend_attention(const void* q, int64_t q_token_stride, int32_t num_q_heads, const void* k_ws,
                                const void* v_ws, int64_t kv_token_stride, int32_t num_kv_heads, int32_t head_dim,
                                int32_t prefix_len, int32_t chunk_len, float sm_scale, void* out, int32_t out_dtype,
                                int64_t out_token_stride, float* lse_out, void* stream);

/* Fused extend attention: as kvq_extend_attention, but the prefix is read
 * straight from the 4-bit pages (cache tokens 0 .. prefix_len - 1 of the
 * sequence whose page list is block_table_row) and decoded while staged, so
 * no bf16 workspace is needed -- the 1M-token case of the extend path would
 * otherwise hold a 4.3 GB workspace ("SGLang's 4-bit KV cache ...", section
 * "The 1.78x is arithmetic ...": the 1M run handed 15 % of the GPU back for
 * prefill workspace).  The chunk's own K/V come as bf16 rows k_chunk, v_chunk
 * [chunk_len][chunk_token_stride] (head g at g * head_dim).  NVFP4 and INT4
 * caches (FP8, K8V4: KVQ_ERR_UNSUPPORTED); for a rotated cache the caller passes
 * rotated q and chunk rows and rotates the output back.  Arithmetic: prefix keys
 * and values enter at their exact dequantized value; 32-key steps wholly inside
 * the prefix multiply in fp16 with each probability rounded to fp16 (relative
 * error at most 2^-12), later steps in bf16 with each probability split into
 * two bf16 terms; products are exact and accumulate in fp32.  A page's slab
 * (kvq_slab_bytes) must fit in 2^31 - 1 bytes, page sizes up to about seven
 * million tokens (else KVQ_ERR_UNSUPPORTED). */
kvq_status kvq_extend_attention_paged(const kvq_cache* cache, const int32_t* block_table_row, int32_t prefix_len,
                                      const void* q, int64_t q_token_stride, int32_t num_q_heads, const void* k_chunk,
                                      const void* v_chunk, int64_t chunk_token_stride, int32_t chunk_len,
                                      float sm_scale, void* out, int32_t out_dtype, int64_t out_token_stride,
                                      float* lse_out, void* stream);

/* Global-scale calibration for NVFP4 ("SGLang's 4-bit KV cache ...",
 * section '"Near-lossless" is narrower than it sounds': the measured NVFP4
 * drops its per-tensor FP32 scale, which leaves the E4M3 block scale to carry
 * the whole dynamic range; calibration is listed as ongoing work).
 *
 * kvq_calibrate_amax raises running_amax (device float[2] = {K, V}, zeroed by
 * the caller before the first call) to the largest |value| of this call's K
 * and V rows (same row arguments as kvq_quantize_store, no slots).  Run it
 * over the prefill chunks of a layer, then kvq_calibrate_global_scale writes
 * cache->global_scale[i] = fp32(running_amax[i] / (6 * 448)) (1 for an
 * all-zero tensor), which puts the largest calibrated block scale on E4M3's
 * 448.  Call it before the layer's first kvq_quantize_store: blocks already
 * stored keep the scale they were written with.  NVFP4 caches only
 * (KVQ_ERR_UNSUPPORTED otherwise). */
kvq_status kvq_calibrate_amax(const kvq_cache* cache, const void* k, const void* v, int32_t in_dtype,
                              int64_t in_token_stride, int32_t num_tokens, float* running_amax, void* stream);
kvq_status kvq_calibrate_global_scale(const kvq_cache* cache, const float* running_amax, void* stream);

/* out_row = R in_row (R = H_D / sqrt(D), as KVQ_FLAG_HADAMARD) for `rows`
 * rows of head_dim elements: queries before decode over a rotated cache, and
 * the decode output back (R is its own inverse).  in_dtype / out_dtype
 * KVQ_DT_F32 or KVQ_DT_BF16 (bf16 output rounded to nearest even); strides in
 * elements, rows 16-byte aligned; head_dim 128 or 256.  in and out may be the
 * same buffer when the dtypes and strides match. */
kvq_status kvq_hadamard_rotate(const void* in, int32_t in_dtype, int64_t in_row_stride, void* out, int32_t out_dtype,
                               int64_t out_row_stride, int32_t rows, int32_t head_dim, void* stream);

/* Measurement aid, not part of the cache path: a plain streaming read of
 * `bytes` bytes of device memory (the practical HBM read ceiling against which
 * the decode kernel's bandwidth is judged).  Nothing is computed from the data
 * beyond an XOR that decides whether sink[0] is written (it practically never
 * is).  buf 16-byte aligned, bytes a multiple of 16; num_workgroups <= 0 picks
 * 2048 (8 per CU).  Asynchronous on `stream`. */
kvq_status kvq_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t num_workgroups, void* stream);

/* Measurement aids, likewise: a plain streaming write of `bytes` bytes (every
 * 32-bit word set to `value`) and a plain streaming copy of `bytes` bytes from
 * src to dst (non-overlapping) -- the write and read + write ceilings against
 * which the bulk store and the prefix dequantization are judged.  Pointers
 * 16-byte aligned, bytes a multiple of 16; num_workgroups <= 0 picks 2048.
 * Asynchronous on `stream`. */
kvq_status kvq_stream_write(void* buf, size_t bytes, uint32_t value, int32_t num_workgroups, void* stream);
kvq_status kvq_stream_copy(const void* src, void* dst, size_t bytes, int32_t num_workgroups, void* stream);

/* Measurement aid, likewise: the matrix-core ceilings against which the
 * extend kernels' products are judged.  Runs num_workgroups workgroups of 768
 * threads (three wavefronts per SIMD, one workgroup per compute unit, as the
 * fused extend runs), each wavefront issuing 16 v_mfma_f32_16x16x32_f16 per
 * iteration: 16 x 16 x 32 x 2 = 16,384 flops each, so one call is
 * 16,384 x 16 x 12 x iterations x num_workgroups flops.  lds_operands = 0:
 * operands in registers; 1: each product's first operand read from LDS as
 * the extend kernels read their key rows for QK (one 16-byte read per lane);
 * 2: the extend kernels' own mix, products alternating between that read and
 * the PV operand form (two transposing 8-byte reads per lane of the value
 * rows).  Modes 1 and 2 issue their reads eight operands ahead.
 * sink: device word, written only in the practically impossible case that the
 * sum is 1e-30.  KVQ_ERR_NULL, KVQ_ERR_UNSUPPORTED (lds_operands not 0, 1 or 2),
 * KVQ_ERR_SHAPE (iterations or num_workgroups <= 0).  Asynchronous on
 * `stream`. */
kvq_status kvq_mfma_rate(int32_t lds_operands, int32_t iterations, int32_t num_workgroups, uint32_t* sink,
                         void* stream);

/* Static description of a status code. */
const char* kvq_status_string(int32_t status);

/* hipError_t of the last failed launch on the calling thread (0 if none). */
int32_t kvq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
