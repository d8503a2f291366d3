/*
 * kvq_oracle.c -- slow, plain CPU oracle for the 4-bit paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library: every codec below is written from the format definitions.
 *
 * What it follows (pages as printed, cited by title and section):
 *  - "SGLang's 4-bit KV cache: the 56% is exact, the 1.78x is untested",
 *    Figure 2 caption (one shared pool of packed E2M1 K and V, one E4M3 block
 *    scale per 16 elements, per-layer FP32 global scales; decode reads the
 *    4-bit pool directly; extend dequantizes the cached prefix into a
 *    workspace) and section "The 56% survives its own scale, and names the
 *    block size" (E2M1 element, E4M3 block scale, FP32 tensor scale; the
 *    (4 + 8/B)/8 equation).
 *  - "KV cache in 4 bits: 8.8 instead of 4.7 full sessions on the same four
 *    RTX 5090s", section "What we changed" (int4_per_token_head: 4-bit values
 *    with scales per token and head, 264 bytes per head and token at head
 *    dim 256; pages of 1600 tokens = 422,400 bytes).
 * Everything the pages leave open is taken in its plainest reading; each such
 * reading is named where it is used (block axis, scale formula, rounding,
 * nibble order, INT4 range).
 *
 * Precision: quantization decisions (scale and element codes) are made in
 * IEEE fp32, exactly as written (no fused multiply-add, no fast-math); the
 * attention is computed in fp64 over exactly dequantized values.
 *
 * Parity pins: every function here is checked by the CPU tests against
 * something other than itself (torch's float8_e4m3fn and bfloat16 casts,
 * torch's fp64 attention, closed forms and the page-printed byte counts).
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#define KVQO_NVFP4 1
#define KVQO_INT4 2
#define KVQO_FP8 3
#define KVQO_K8V4 4

/* ---------------------------------------------------------------------- */
/* Element and scale formats                                               */
/* ---------------------------------------------------------------------- */

/* E2M1 (4-bit float: 1 sign, 2 exponent, 1 mantissa bit, bias 1, no inf/NaN).
 * Exponent field 0 is subnormal: magnitude = mantissa * 0.5.
 * Otherwise magnitude = 2^(e-1) * (1 + m/2). */
double kvqo_e2m1_value(int code) {
  int sign = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -mag : mag;
}

/* E4M3 in the OCP "FN" flavour (1 sign, 4 exponent, 3 mantissa bits, bias 7,
 * no infinities, S.1111.111 is NaN, largest finite 448).  Exponent field 0 is
 * subnormal: magnitude = m/8 * 2^-6. */
double kvqo_e4m3_value(int code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? (m / 8.0) * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return sign ? -mag : mag;
}

/* Encode an fp32 value as E2M1: the nearest representable value, with a tie
 * going to the code whose mantissa bit is 0 (round-half-to-even); anything
 * at or beyond 6 in magnitude becomes +-6 (saturation, the format has no
 * infinity).  The sign of the input is kept, so -0 encodes as 0x8. */
int kvqo_e2m1_encode(float r) {
  int sign = signbit(r) ? 1 : 0;
  double a = fabs((double)r);
  if (a >= 6.0) return (sign << 3) | 7;
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c < 8; c++) {
    double d = fabs(a - kvqo_e2m1_value(c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return (sign << 3) | best;
}

/* Encode a non-negative fp32 value as E4M3 (OCP FN): the nearest finite
 * value, ties to the even code; values at or above 448 (the largest finite)
 * saturate to 448 (code 0x7E), so the encoder never produces NaN. */
int kvqo_e4m3_encode(float s) {
  if (isnan(s)) return 0x7F;
  if (s >= 448.0f) return 0x7E;
  double a = (double)s;
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c <= 0x7E; c++) {
    double d = fabs(a - kvqo_e4m3_value(c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

/* Round an fp32 value to the nearest bfloat16 (ties to even), returning the
 * 16-bit pattern.  bfloat16 keeps the top 16 bits of the fp32 pattern; the
 * two candidates are the truncation and the next value away from zero. */
uint16_t kvqo_bf16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lo = u & 0xFFFF0000u;
  uint32_t hi = lo + 0x10000u;
  float flo, fhi;
  memcpy(&flo, &lo, 4);
  memcpy(&fhi, &hi, 4);
  double dlo = fabs((double)x - (double)flo);
  double dhi = isinf(fhi) ? INFINITY : fabs((double)fhi - (double)x);
  if (isinf(fhi) && !isinf(x)) {
    /* the value above the largest finite bf16 rounds to infinity only past
       the midpoint 2^128 * (1 - 2^-9) */
    double mid = ldexp(1.0, 128) * (1.0 - ldexp(1.0, -9));
    if (fabs((double)x) >= mid) return (uint16_t)(hi >> 16);
    return (uint16_t)(lo >> 16);
  }
  if (dlo < dhi) return (uint16_t)(lo >> 16);
  if (dhi < dlo) return (uint16_t)(hi >> 16);
  return (uint16_t)((((lo >> 16) & 1) == 0 ? lo : hi) >> 16);
}

/* ---------------------------------------------------------------------- */
/* One row (one token, one KV head, K or V) of D values                    */
/* ---------------------------------------------------------------------- */

/* NVFP4 row quantization.  Reading of the pages: the 16-element block runs
 * along the head dimension of one token row (decode writes one token at a
 * time, so a block cannot span tokens); the block scale maps the block's
 * largest magnitude onto E2M1's largest value 6 relative to the per-layer
 * FP32 global scale gs; elements are rounded under the *stored* (decoded)
 * scale so that decoding gives the nearest grid point.
 *
 *   amax  = max |x_i| over the 16 elements (exact)
 *   den   = fp32(6 * gs)
 *   s_raw = fp32(amax / den)
 *   cs    = E4M3(s_raw)                      (stored scale code)
 *   S     = fp32(value(cs) * gs)
 *   code_i = 0x0 if S == 0, else E2M1(fp32(x_i / S))
 * Codes are packed two per byte, even element in the low nibble. */
void kvqo_nvfp4_quantize_row(const float* x, int D, float gs, uint8_t* codes, uint8_t* scales) {
  for (int b = 0; b < D / 16; b++) {
    const float* xb = x + 16 * b;
    float amax = 0.0f;
    for (int i = 0; i < 16; i++) {
      float a = fabsf(xb[i]);
      if (a > amax) amax = a;
    }
    float den = 6.0f * gs;
    float s_raw = amax / den;
    int cs = kvqo_e4m3_encode(s_raw);
    float S = (float)kvqo_e4m3_value(cs) * gs;
    scales[b] = (uint8_t)cs;
    int c[16];
    for (int i = 0; i < 16; i++) c[i] = (S == 0.0f) ? 0 : kvqo_e2m1_encode(xb[i] / S);
    for (int j = 0; j < 8; j++) codes[8 * b + j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
  }
}

/* INT4 per-token-head row quantization (symmetric): one fp32 scale for the
 * whole row, s = fp32(amax / 7); q_i = clamp(round-half-even(fp32(x_i / s)),
 * -7, 7) stored as a two's-complement nibble (the code -8 is never made);
 * an all-zero row gets s = 0 and all codes 0.  Packing as for NVFP4. */
void kvqo_int4_quantize_row(const float* x, int D, uint8_t* codes, float* scale) {
  float amax = 0.0f;
  for (int i = 0; i < D; i++) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float s = amax / 7.0f;
  *scale = s;
  for (int j = 0; j < D / 2; j++) {
    int q[2];
    for (int h = 0; h < 2; h++) {
      int v = 0;
      if (s != 0.0f) {
        float r = x[2 * j + h] / s;
        float rr = nearbyintf(r); /* default rounding mode: to nearest, ties to even */
        v = (int)rr;
        if (v > 7) v = 7;
        if (v < -7) v = -7;
      }
      q[h] = v & 0xF;
    }
    codes[j] = (uint8_t)(q[0] | (q[1] << 4));
  }
}

/* Exact dequantization of one stored NVFP4 row, in fp64. */
void kvqo_nvfp4_dequant_row(const uint8_t* codes, const uint8_t* scales, int D, float gs, double* out) {
  for (int i = 0; i < D; i++) {
    int byte = codes[i / 2];
    int code = (i & 1) ? (byte >> 4) : (byte & 15);
    out[i] = kvqo_e2m1_value(code) * kvqo_e4m3_value(scales[i / 16]) * (double)gs;
  }
}

/* Exact dequantization of one stored INT4 row, in fp64. */
void kvqo_int4_dequant_row(const uint8_t* codes, float scale, int D, double* out) {
  for (int i = 0; i < D; i++) {
    int byte = codes[i / 2];
    int nib = (i & 1) ? (byte >> 4) : (byte & 15);
    int q = (nib & 8) ? nib - 16 : nib;
    out[i] = (double)q * (double)scale;
  }
}

/* ---------------------------------------------------------------------- */
/* Paged pool                                                              */
/* ---------------------------------------------------------------------- */
/* One page of one KV head is a slab laid out as
 *     [K codes: P rows of D/2 bytes][K scales][V codes: P x D/2][V scales]
 * with K/V scales P x D/16 bytes (NVFP4, E4M3 codes) or P fp32 values
 * (INT4).  The pool is [num_pages][num_kv_heads][slab]. */

static size_t row_code_bytes(int D) { return (size_t)D / 2; }
static size_t row_scale_bytes(int fmt, int D) { return fmt == KVQO_NVFP4 ? (size_t)D / 16 : 4; }

/* FP8 E4M3 with one FP32 scale per tensor (the comparator: "SGLang's 4-bit
 * KV cache ...", section "The 56% survives its own scale, and names the block
 * size", states that the comparison assumes a per-tensor-scaled FP8 cache):
 * one byte per value, no per-token scales.  Slab of one (page, head):
 * [K: P rows x D bytes][V transposed: D rows (channels) x P bytes], so that a
 * channel's values for consecutive tokens are adjacent (the paged-attention
 * value layout). */
/* FP8 keys with NVFP4 values (the split-precision variant: "SGLang's 4-bit KV
 * cache ...", section "Against what this site already established": another
 * engine's 4-bit cache keeps keys in FP8 and values in 4 bits, spending twice
 * the bits on keys; which 4-bit value format it uses is not stated, and the
 * reading here is the pages' own NVFP4).  Keys: E4M3 with the per-tensor
 * scale gs[0], as the FP8 format; values: NVFP4 with global scale gs[1].
 * Slab of one (page, head): [K: P rows x D bytes][V codes: P rows x D/2]
 * [V scales: P rows x D/16]. */
static size_t k8v4_k_bytes(int P, int D) { return (size_t)P * (size_t)D; }

size_t kvqo_slab_bytes(int fmt, int P, int D) {
  if (fmt == KVQO_FP8) return 2 * (size_t)P * (size_t)D;
  if (fmt == KVQO_K8V4) return k8v4_k_bytes(P, D) + (size_t)P * (row_code_bytes(D) + row_scale_bytes(KVQO_NVFP4, D));
  return 2 * (size_t)P * (row_code_bytes(D) + row_scale_bytes(fmt, D));
}

/* Bytes one token costs in one KV head (K and V, codes and scales). */
size_t kvqo_token_head_bytes(int fmt, int D) {
  if (fmt == KVQO_FP8) return 2 * (size_t)D;
  if (fmt == KVQO_K8V4) return (size_t)D + row_code_bytes(D) + row_scale_bytes(KVQO_NVFP4, D);
  return 2 * (row_code_bytes(D) + row_scale_bytes(fmt, D));
}

/* FP8 value code: y = fp32(x / s), then E4M3 of |y| (nearest, ties to the
 * even code, saturating at 448) with the sign of y (so -0 is 0x80). */
int kvqo_fp8_encode(float x, float s) {
  const float y = x / s;
  return kvqo_e4m3_encode(fabsf(y)) | (signbit(y) ? 0x80 : 0);
}

/* Byte offset of value (token offset off, channel c) of K (kv = 0) or V
 * (kv = 1) inside an FP8 slab. */
static size_t fp8_offset(int P, int D, int off, int c, int kv) {
  return kv ? (size_t)P * D + (size_t)c * P + off : (size_t)off * D + c;
}

typedef struct {
  uint8_t* codes;
  uint8_t* scales;
} rowptr;

/* Locate the K (kv = 0) or V (kv = 1) row of token offset `off` in page
 * `page`, head g. */
static rowptr locate(uint8_t* pool, int fmt, int P, int Hkv, int D, int64_t page, int g, int off, int kv) {
  size_t slab = kvqo_slab_bytes(fmt, P, D);
  uint8_t* base = pool + ((size_t)page * Hkv + g) * slab;
  size_t half = (size_t)P * (row_code_bytes(D) + row_scale_bytes(fmt, D));
  uint8_t* sec = base + (kv ? half : 0);
  rowptr r;
  r.codes = sec + (size_t)off * row_code_bytes(D);
  r.scales = sec + (size_t)P * row_code_bytes(D) + (size_t)off * row_scale_bytes(fmt, D);
  return r;
}

/* Orthogonal Walsh-Hadamard rotation of one row, in place, in fp32 ("SGLang's
 * 4-bit KV cache ...", section "Against what this site already established":
 * rotate every vector by an orthogonal matrix before quantizing it, as
 * TurboQuant argues and as another engine's 4-bit cache does with a fixed FP32
 * D256 Hadamard rotation).  Reading: R = H_D / sqrt(D) with H_D the Sylvester
 * Hadamard matrix (H_1 = 1, H_2n = [[H_n, H_n], [H_n, -H_n]]), computed by the
 * standard fast transform -- stages h = 1, 2, 4, ..., D/2, each replacing the
 * pair (x_i, x_{i+h}) (bit h of i clear) by (x_i + x_{i+h}, x_i - x_{i+h}) in
 * fp32 -- and the scale fp32(1 / sqrt(D)) applied last.  R is symmetric and
 * its own inverse. */
void kvqo_hadamard_row(float* x, int D) {
  for (int h = 1; h < D; h <<= 1) {
    for (int i = 0; i < D; i++) {
      if (i & h) continue;
      const float a = x[i], b = x[i + h];
      x[i] = a + b;
      x[i + h] = a - b;
    }
  }
  const float s = (float)(1.0 / sqrt((double)D));
  for (int i = 0; i < D; i++) x[i] = x[i] * s;
}

/* Quantize-on-write: for token i with slot = slot_mapping[i] >= 0, page =
 * slot / P and offset = slot % P; each KV head's K and V row is quantized
 * and stored there.  A negative slot skips the token.  k, v are
 * [n_tok][Hkv][D] fp32 (bf16 inputs widened exactly by the caller);
 * gs = {gs_K, gs_V} (NVFP4: global scales; FP8: the per-tensor scales).
 * rotate != 0: each row is Hadamard-rotated (kvqo_hadamard_row) first. */
void kvqo_quantize_store(int fmt, uint8_t* pool, int P, int Hkv, int D, const float* gs, const float* k,
                         const float* v, int n_tok, const int32_t* slot_mapping, int rotate) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n_tok; i++) {
    int32_t slot = slot_mapping[i];
    if (slot < 0) continue;
    int64_t page = slot / P;
    int off = slot % P;
    for (int g = 0; g < Hkv; g++) {
      for (int kv = 0; kv < 2; kv++) {
        const float* x = (kv ? v : k) + ((size_t)i * Hkv + g) * D;
        float xr[512];
        if (rotate) {
          memcpy(xr, x, sizeof(float) * (size_t)D);
          kvqo_hadamard_row(xr, D);
          x = xr;
        }
        if (fmt == KVQO_FP8) {
          uint8_t* base = pool + ((size_t)page * Hkv + g) * kvqo_slab_bytes(fmt, P, D);
          for (int c = 0; c < D; c++) base[fp8_offset(P, D, off, c, kv)] = (uint8_t)kvqo_fp8_encode(x[c], gs[kv]);
          continue;
        }
        if (fmt == KVQO_K8V4) {
          uint8_t* base = pool + ((size_t)page * Hkv + g) * kvqo_slab_bytes(fmt, P, D);
          if (kv == 0) {
            for (int c = 0; c < D; c++) base[(size_t)off * D + c] = (uint8_t)kvqo_fp8_encode(x[c], gs[0]);
          } else {
            uint8_t* vsec = base + k8v4_k_bytes(P, D);
            kvqo_nvfp4_quantize_row(x, D, gs[1], vsec + (size_t)off * row_code_bytes(D),
                                    vsec + (size_t)P * row_code_bytes(D) + (size_t)off * (D / 16));
          }
          continue;
        }
        rowptr r = locate(pool, fmt, P, Hkv, D, page, g, off, kv);
        if (fmt == KVQO_NVFP4) {
          kvqo_nvfp4_quantize_row(x, D, gs[kv], r.codes, r.scales);
        } else {
          float s;
          kvqo_int4_quantize_row(x, D, r.codes, &s);
          memcpy(r.scales, &s, 4);
        }
      }
    }
  }
}

/* Exact fp64 value of the stored K (kv = 0) or V (kv = 1) row of cache token
 * t of a sequence whose page list is `pages`. */
static void read_token(const uint8_t* pool, int fmt, int P, int Hkv, int D, const float* gs, const int32_t* pages,
                       int64_t t, int g, int kv, double* out) {
  if (fmt == KVQO_FP8) {
    const uint8_t* base = pool + ((size_t)pages[t / P] * Hkv + g) * kvqo_slab_bytes(fmt, P, D);
    for (int c = 0; c < D; c++) out[c] = kvqo_e4m3_value(base[fp8_offset(P, D, (int)(t % P), c, kv)]) * gs[kv];
    return;
  }
  if (fmt == KVQO_K8V4) {
    const uint8_t* base = pool + ((size_t)pages[t / P] * Hkv + g) * kvqo_slab_bytes(fmt, P, D);
    const int off = (int)(t % P);
    if (kv == 0) {
      for (int c = 0; c < D; c++) out[c] = kvqo_e4m3_value(base[(size_t)off * D + c]) * gs[0];
    } else {
      const uint8_t* vsec = base + k8v4_k_bytes(P, D);
      kvqo_nvfp4_dequant_row(vsec + (size_t)off * row_code_bytes(D),
                             vsec + (size_t)P * row_code_bytes(D) + (size_t)off * (D / 16), D, gs[1], out);
    }
    return;
  }
  rowptr r = locate((uint8_t*)pool, fmt, P, Hkv, D, pages[t / P], g, (int)(t % P), kv);
  if (fmt == KVQO_NVFP4) {
    kvqo_nvfp4_dequant_row(r.codes, r.scales, D, gs[kv], out);
  } else {
    float s;
    memcpy(&s, r.scales, 4);
    kvqo_int4_dequant_row(r.codes, s, D, out);
  }
}

/* Scaled dot-product attention of one decode query over cache tokens
 * [t0, t1) of sequence b, query head h, in fp64.  Produces the unnormalised
 * partial state of that token range: m = max score, l = sum exp(s - m),
 * acc = sum exp(s - m) * v.  Query head h reads KV head h / G (contiguous
 * GQA groups).  No mask: the single decode query sees every cached token,
 * all of them read back from the 4-bit cache. */
static void attend_range(const uint8_t* pool, int fmt, int P, int Hkv, int D, const float* gs, const float* qh,
                         const int32_t* pages, int g, int64_t t0, int64_t t1, double sm_scale, double* m_out,
                         double* l_out, double* acc) {
  for (int c = 0; c < D; c++) acc[c] = 0.0;
  if (t1 <= t0) {
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  int64_t n = t1 - t0;
  double* s = (double*)malloc(sizeof(double) * n);
  double* row = (double*)malloc(sizeof(double) * D);
  double m = -INFINITY;
  for (int64_t t = t0; t < t1; t++) {
    read_token(pool, fmt, P, Hkv, D, gs, pages, t, g, 0, row);
    double dot = 0.0;
    for (int c = 0; c < D; c++) dot += (double)qh[c] * row[c];
    s[t - t0] = sm_scale * dot;
    if (s[t - t0] > m) m = s[t - t0];
  }
  double l = 0.0;
  for (int64_t t = t0; t < t1; t++) {
    double p = exp(s[t - t0] - m);
    l += p;
    read_token(pool, fmt, P, Hkv, D, gs, pages, t, g, 1, row);
    for (int c = 0; c < D; c++) acc[c] += p * row[c];
  }
  *m_out = m;
  *l_out = l;
  free(s);
  free(row);
}

/* Decode attention for every (sequence b, query head h):
 *   o = softmax(sm_scale * q K^T) V over the seq_lens[b] cached tokens,
 *   lse = max + log(sum exp(score - max))   (natural log).
 * seq_lens[b] == 0 gives o = 0 and lse = -inf.
 * q: [B][Hq][D] (bf16 values widened to fp32); block_table: [B][max_pages];
 * out: [B][Hq][D] fp64; lse: [B][Hq] fp64.
 * split_tokens > 0 evaluates each sequence as independent token ranges of
 * that length and merges their (o, m, l) states by the log-sum-exp rule; in
 * exact arithmetic the result does not depend on the partition. */
void kvqo_decode_attention(int fmt, const uint8_t* pool, int P, int Hkv, int D, const float* gs, const float* q,
                           int Hq, const int32_t* block_table, int max_pages, const int32_t* seq_lens, int B,
                           double sm_scale, int64_t split_tokens, double* out, double* lse) {
  int G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic) collapse(2)
  for (int b = 0; b < B; b++) {
    for (int h = 0; h < Hq; h++) {
      int g = h / G;
      int64_t L = seq_lens[b];
      const float* qh = q + ((size_t)b * Hq + h) * D;
      const int32_t* pages = block_table + (size_t)b * max_pages;
      double* o = out + ((size_t)b * Hq + h) * D;
      int64_t step = split_tokens > 0 ? split_tokens : (L > 0 ? L : 1);
      int64_t nsplit = L > 0 ? (L + step - 1) / step : 0;
      double M = -INFINITY;
      double* ms = (double*)malloc(sizeof(double) * (nsplit > 0 ? nsplit : 1));
      double* ls = (double*)malloc(sizeof(double) * (nsplit > 0 ? nsplit : 1));
      double* accs = (double*)malloc(sizeof(double) * D * (nsplit > 0 ? nsplit : 1));
      for (int64_t i = 0; i < nsplit; i++) {
        int64_t t0 = i * step, t1 = t0 + step < L ? t0 + step : L;
        attend_range(pool, fmt, P, Hkv, D, gs, qh, pages, g, t0, t1, sm_scale, &ms[i], &ls[i], accs + i * D);
        if (ms[i] > M) M = ms[i];
      }
      double denom = 0.0;
      for (int c = 0; c < D; c++) o[c] = 0.0;
      for (int64_t i = 0; i < nsplit; i++) {
        if (ls[i] == 0.0) continue;
        double w = exp(ms[i] - M);
        denom += w * ls[i];
        for (int c = 0; c < D; c++) o[c] += w * accs[i * D + c];
      }
      if (denom > 0.0) {
        for (int c = 0; c < D; c++) o[c] /= denom;
        lse[(size_t)b * Hq + h] = M + log(denom);
      } else {
        lse[(size_t)b * Hq + h] = -INFINITY;
      }
      free(ms);
      free(ls);
      free(accs);
    }
  }
}

/* Prefix dequantization into a bf16 workspace: cache tokens [0, prefix_len)
 * of one sequence (page list `pages`) become rows of k_out / v_out, laid out
 * [prefix_len][Hkv][D] with a token stride of out_token_stride elements.
 *   NVFP4: bf16_rne(fp32(fp32(e2m1 * e4m3) * gs))  (exact when gs == 1)
 *   INT4:  bf16_rne(fp32(q * s)) */
void kvqo_dequant_prefix(int fmt, const uint8_t* pool, int P, int Hkv, int D, const float* gs,
                         const int32_t* pages, int64_t prefix_len, uint16_t* k_out, uint16_t* v_out,
                         int64_t out_token_stride) {
  if (fmt == KVQO_FP8 || fmt == KVQO_K8V4) return; /* no extend path for the FP8-keyed formats */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < prefix_len; t++) {
    for (int g = 0; g < Hkv; g++) {
      for (int kv = 0; kv < 2; kv++) {
        rowptr r = locate((uint8_t*)pool, fmt, P, Hkv, D, pages[t / P], g, (int)(t % P), kv);
        uint16_t* dst = (kv ? v_out : k_out) + (size_t)t * out_token_stride + (size_t)g * D;
        for (int i = 0; i < D; i++) {
          int byte = r.codes[i / 2];
          int nib = (i & 1) ? (byte >> 4) : (byte & 15);
          float val;
          if (fmt == KVQO_NVFP4) {
            float prod = (float)(kvqo_e2m1_value(nib) * kvqo_e4m3_value(r.scales[i / 16]));
            val = prod * gs[kv];
          } else {
            float s;
            memcpy(&s, r.scales, 4);
            int qv = (nib & 8) ? nib - 16 : nib;
            val = (float)qv * s;
          }
          dst[i] = kvqo_bf16_rne(val);
        }
      }
    }
  }
}

/* Extend attention ("SGLang's 4-bit KV cache ...", Figure 2 caption: the
 * chunked-prefill / extend path dequantizes the cached prefix into a reused
 * workspace and attends over prefix plus current chunk).  Reading: the
 * workspace holds bf16 K and V rows [prefix_len + chunk_len][Hkv][D] (token
 * stride kv_stride elements) -- the dequantized prefix followed by the
 * chunk's own K/V -- and chunk query i (at sequence position prefix_len + i)
 * attends causally to keys 0 .. prefix_len + i: standard scaled dot-product
 * attention, query head h reading KV head h / G, in fp64.  q is
 * [chunk_len][Hq][D] (token stride q_stride); out [chunk_len][Hq][D],
 * lse [chunk_len][Hq] (natural log). */
void kvqo_extend_attention(const float* q, int64_t q_stride, int Hq, const float* k_ws, const float* v_ws,
                           int64_t kv_stride, int Hkv, int D, int64_t prefix_len, int64_t chunk_len,
                           double sm_scale, double* out, double* lse) {
  const int G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic) collapse(2)
  for (int64_t i = 0; i < chunk_len; i++) {
    for (int h = 0; h < Hq; h++) {
      const int g = h / G;
      const float* qh = q + i * q_stride + (int64_t)h * D;
      const int64_t nk = prefix_len + i + 1;
      double* s = (double*)malloc(sizeof(double) * (size_t)nk);
      double m = -INFINITY;
      for (int64_t j = 0; j < nk; j++) {
        const float* kj = k_ws + j * kv_stride + (int64_t)g * D;
        double dot = 0.0;
        for (int c = 0; c < D; c++) dot += (double)qh[c] * (double)kj[c];
        s[j] = dot * sm_scale;
        if (s[j] > m) m = s[j];
      }
      double l = 0.0;
      double* o = out + ((size_t)i * Hq + h) * D;
      for (int c = 0; c < D; c++) o[c] = 0.0;
      for (int64_t j = 0; j < nk; j++) {
        const double p = exp(s[j] - m);
        l += p;
        const float* vj = v_ws + j * kv_stride + (int64_t)g * D;
        for (int c = 0; c < D; c++) o[c] += p * (double)vj[c];
      }
      for (int c = 0; c < D; c++) o[c] /= l;
      lse[(size_t)i * Hq + h] = m + log(l);
      free(s);
    }
  }
}

/* Extend attention over [cached 4-bit prefix | bf16 chunk] without a
 * workspace (the fused form of the same Figure 2 extend step; the pages leave
 * that form open).  Reading: the keys and values are those the workspace
 * would hold, except that the prefix enters at its exact dequantized value
 * (e2m1 * e4m3 * gs, q * s) in fp64 rather than rounded to bf16 -- identical
 * at gs = 1 for NVFP4.  Cache tokens t < prefix_len come from the pool
 * (page list `pages`, read_token), tokens t >= prefix_len from chunk row
 * t - prefix_len of k_chunk / v_chunk ([chunk rows][chunk_stride], head g at
 * g * D, bf16 values widened to fp32).  Query row j of q ([n_q][q_stride],
 * head h at h * D) sits at sequence position q_pos[j] >= prefix_len and
 * attends causally to keys 0 .. q_pos[j], query head h reading KV head h / G.
 * Outputs per (j, h): out [n_q][Hq][D], lse [n_q][Hq] (natural log) and, when
 * out_abs is not NULL, the softmax-weighted mean of |v| per channel,
 * sum_t w_t |v_t,c| (the scale of the error that rounding each weight to a
 * fixed relative precision can cause). */
void kvqo_extend_attention_paged(int fmt, const uint8_t* pool, int P, int Hkv, int D, const float* gs,
                                 const int32_t* pages, int64_t prefix_len, const float* q, int64_t q_stride, int Hq,
                                 const int64_t* q_pos, int64_t n_q, const float* k_chunk, const float* v_chunk,
                                 int64_t chunk_stride, double sm_scale, double* out, double* lse, double* out_abs) {
  const int G = Hq / Hkv;
  /* one (query row, KV head) per iteration: each key and value row is read
   * once and used by the G query heads of the group */
#pragma omp parallel for schedule(dynamic) collapse(2)
  for (int64_t j = 0; j < n_q; j++) {
    for (int g = 0; g < Hkv; g++) {
      const int64_t nk = q_pos[j] + 1;
      double* s = (double*)malloc(sizeof(double) * (size_t)nk * G);  /* [G][nk] */
      double* row = (double*)malloc(sizeof(double) * (size_t)D);
      double* m = (double*)malloc(sizeof(double) * G);
      double* l = (double*)malloc(sizeof(double) * G);
      for (int e = 0; e < G; e++) m[e] = -INFINITY;
      for (int64_t t = 0; t < nk; t++) {
        if (t < prefix_len) {
          read_token(pool, fmt, P, Hkv, D, gs, pages, t, g, 0, row);
        } else {
          const float* kt = k_chunk + (t - prefix_len) * chunk_stride + (int64_t)g * D;
          for (int c = 0; c < D; c++) row[c] = (double)kt[c];
        }
        for (int e = 0; e < G; e++) {
          const float* qh = q + j * q_stride + (int64_t)(g * G + e) * D;
          double dot = 0.0;
          for (int c = 0; c < D; c++) dot += (double)qh[c] * row[c];
          s[(size_t)e * nk + t] = dot * sm_scale;
          if (s[(size_t)e * nk + t] > m[e]) m[e] = s[(size_t)e * nk + t];
        }
      }
      for (int e = 0; e < G; e++) {
        const int h = g * G + e;
        double* o = out + ((size_t)j * Hq + h) * D;
        double* oa = out_abs ? out_abs + ((size_t)j * Hq + h) * D : NULL;
        for (int c = 0; c < D; c++) {
          o[c] = 0.0;
          if (oa) oa[c] = 0.0;
        }
        l[e] = 0.0;
      }
      for (int64_t t = 0; t < nk; t++) {
        if (t < prefix_len) {
          read_token(pool, fmt, P, Hkv, D, gs, pages, t, g, 1, row);
        } else {
          const float* vt = v_chunk + (t - prefix_len) * chunk_stride + (int64_t)g * D;
          for (int c = 0; c < D; c++) row[c] = (double)vt[c];
        }
        for (int e = 0; e < G; e++) {
          const int h = g * G + e;
          const double p = exp(s[(size_t)e * nk + t] - m[e]);
          l[e] += p;
          double* o = out + ((size_t)j * Hq + h) * D;
          for (int c = 0; c < D; c++) o[c] += p * row[c];
          if (out_abs) {
            double* oa = out_abs + ((size_t)j * Hq + h) * D;
            for (int c = 0; c < D; c++) oa[c] += p * fabs(row[c]);
          }
        }
      }
      for (int e = 0; e < G; e++) {
        const int h = g * G + e;
        double* o = out + ((size_t)j * Hq + h) * D;
        for (int c = 0; c < D; c++) o[c] /= l[e];
        if (out_abs) {
          double* oa = out_abs + ((size_t)j * Hq + h) * D;
          for (int c = 0; c < D; c++) oa[c] /= l[e];
        }
        lse[(size_t)j * Hq + h] = m[e] + log(l[e]);
      }
      free(s);
      free(row);
      free(m);
      free(l);
    }
  }
}

/* Global-scale calibration ("SGLang's 4-bit KV cache ...", section
 * '"Near-lossless" is narrower than it sounds': the measured NVFP4 runs
 * without its per-tensor FP32 scale and calibration is listed as ongoing
 * work).  Reading: gs is taken from the running absolute maximum of a
 * layer's K (or V) over the prefill tokens so that the largest block scale
 * lands on E4M3's largest finite value: gs = fp32(amax / (6 * 448)); an
 * all-zero tensor keeps gs = 1. */
float kvqo_amax(const float* x, int64_t n) {
  float m = 0.0f;
  for (int64_t i = 0; i < n; i++) {
    const float a = fabsf(x[i]);
    if (a > m) m = a;
  }
  return m;
}

float kvqo_global_scale(float amax) { return amax > 0.0f ? amax / 2688.0f : 1.0f; }

/* Number of OpenMP threads the oracle's parallel loops use. */
int kvqo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set that number (timing only; results do not depend on it). */
void kvqo_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
