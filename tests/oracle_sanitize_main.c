/* oracle_sanitize_main.c -- drives every entry point of the CPU oracle
 * (oracle/kvq_oracle.c) once per cache format, for a build of the oracle
 * with AddressSanitizer and UndefinedBehaviorSanitizer (test infrastructure:
 * built and run by tests/test_oracle_sanitized.py, which writes the inputs
 * and compares the outputs with the regular build of the same oracle).
 *
 * Fixed shape: head dim 64, 2 KV heads, 6 query heads, 16-token pages,
 * 3 sequences of 45, 20 and 0 tokens in 11 pages, a 9-token extend chunk.
 * Usage: oracle_sanitize_main <dir> -- reads <dir>/{k,v,q,slots,bt,lens,gs,
 * kc,vc,qe}.bin, writes <dir>/out_<name>.bin. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void kvqo_nvfp4_quantize_row(const float* x, int D, float gs, uint8_t* codes, uint8_t* scales);
void kvqo_int4_quantize_row(const float* x, int D, uint8_t* codes, float* scale);
void kvqo_nvfp4_dequant_row(const uint8_t* codes, const uint8_t* scales, int D, float gs, double* out);
void kvqo_int4_dequant_row(const uint8_t* codes, float scale, int D, double* out);
size_t kvqo_slab_bytes(int fmt, int P, int D);
void kvqo_hadamard_row(float* x, int D);
void kvqo_quantize_store(int fmt, uint8_t* pool, int P, int Hkv, int D, const float* gs, const float* k,
                         const float* v, int n_tok, const int32_t* slot_mapping, int rotate);
void kvqo_decode_attention(int fmt, const uint8_t* pool, int P, int Hkv, int D, const float* gs, const float* q,
                           int Hq, const int32_t* block_table, int max_pages, const int32_t* seq_lens, int B,
                           double sm_scale, int64_t split_tokens, double* out, double* lse);
void kvqo_dequant_prefix(int fmt, const uint8_t* pool, int P, int Hkv, int D, const float* gs,
                         const int32_t* pages, int64_t prefix_len, uint16_t* k_out, uint16_t* v_out,
                         int64_t out_token_stride);
void kvqo_extend_attention(const float* q, int64_t q_stride, int Hq, const float* k_ws, const float* v_ws,
                           int64_t kv_stride, int Hkv, int D, int64_t prefix_len, int64_t chunk_len,
                           double sm_scale, double* out, double* lse);
void kvqo_extend_attention_paged(int fmt, const uint8_t* pool, int P, int Hkv, int D, const float* gs,
                                 const int32_t* pages, int64_t prefix_len, const float* q, int64_t q_stride, int Hq,
                                 const int64_t* q_pos, int64_t n_q, const float* k_chunk, const float* v_chunk,
                                 int64_t chunk_stride, double sm_scale, double* out, double* lse, double* out_abs);
float kvqo_amax(const float* x, int64_t n);

enum { D = 64, HKV = 2, HQ = 6, P = 16, NTOK = 65, B = 3, MAXP = 3, NPAGES = 11, NC = 9, LP = 45 };

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[1024];
  snprintf(path, sizeof(path), "%s/%s.bin", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    exit(2);
  }
  void* buf = malloc(bytes);
  if (fread(buf, 1, bytes, f) != bytes) {
    fprintf(stderr, "short read %s\n", path);
    exit(2);
  }
  fclose(f);
  return buf;
}

static void write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[1024];
  snprintf(path, sizeof(path), "%s/out_%s.bin", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(buf, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(2);
  }
  fclose(f);
}

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  const char* dir = argv[1];
  float* k = read_file(dir, "k", sizeof(float) * NTOK * HKV * D);
  float* v = read_file(dir, "v", sizeof(float) * NTOK * HKV * D);
  float* q = read_file(dir, "q", sizeof(float) * B * HQ * D);
  int32_t* slots = read_file(dir, "slots", sizeof(int32_t) * NTOK);
  int32_t* bt = read_file(dir, "bt", sizeof(int32_t) * B * MAXP);
  int32_t* lens = read_file(dir, "lens", sizeof(int32_t) * B);
  float* gs = read_file(dir, "gs", sizeof(float) * 2);
  float* kc = read_file(dir, "kc", sizeof(float) * NC * HKV * D);
  float* vc = read_file(dir, "vc", sizeof(float) * NC * HKV * D);
  float* qe = read_file(dir, "qe", sizeof(float) * NC * HQ * D);
  const double sm = 0.125;
  char name[64];

  for (int fmt = 1; fmt <= 4; fmt++) {
    for (int rot = 0; rot < 2; rot++) {
      const size_t slab = kvqo_slab_bytes(fmt, P, D);
      const size_t pool_bytes = (size_t)NPAGES * HKV * slab;
      uint8_t* pool = malloc(pool_bytes);
      memset(pool, 0x11, pool_bytes);
      kvqo_quantize_store(fmt, pool, P, HKV, D, gs, k, v, NTOK, slots, rot);
      snprintf(name, sizeof(name), "pool_%d_%d", fmt, rot);
      write_file(dir, name, pool, pool_bytes);
      double* o = malloc(sizeof(double) * B * HQ * D);
      double* lse = malloc(sizeof(double) * B * HQ);
      kvqo_decode_attention(fmt, pool, P, HKV, D, gs, q, HQ, bt, MAXP, lens, B, sm, 7, o, lse);
      snprintf(name, sizeof(name), "dec_o_%d_%d", fmt, rot);
      write_file(dir, name, o, sizeof(double) * B * HQ * D);
      snprintf(name, sizeof(name), "dec_lse_%d_%d", fmt, rot);
      write_file(dir, name, lse, sizeof(double) * B * HQ);
      free(o);
      free(lse);
      if (fmt <= 2) {
        uint16_t* ko = malloc(sizeof(uint16_t) * LP * HKV * D);
        uint16_t* vo = malloc(sizeof(uint16_t) * LP * HKV * D);
        kvqo_dequant_prefix(fmt, pool, P, HKV, D, gs, bt, LP, ko, vo, HKV * D);
        snprintf(name, sizeof(name), "dq_k_%d_%d", fmt, rot);
        write_file(dir, name, ko, sizeof(uint16_t) * LP * HKV * D);
        snprintf(name, sizeof(name), "dq_v_%d_%d", fmt, rot);
        write_file(dir, name, vo, sizeof(uint16_t) * LP * HKV * D);
        free(ko);
        free(vo);
        int64_t pos[NC];
        for (int i = 0; i < NC; i++) pos[i] = LP + i;
        double* eo = malloc(sizeof(double) * NC * HQ * D);
        double* el = malloc(sizeof(double) * NC * HQ);
        double* ea = malloc(sizeof(double) * NC * HQ * D);
        kvqo_extend_attention_paged(fmt, pool, P, HKV, D, gs, bt, LP, qe, HQ * D, HQ, pos, NC, kc, vc, HKV * D, sm, eo,
                                    el, ea);
        snprintf(name, sizeof(name), "ext_o_%d_%d", fmt, rot);
        write_file(dir, name, eo, sizeof(double) * NC * HQ * D);
        snprintf(name, sizeof(name), "ext_abs_%d_%d", fmt, rot);
        write_file(dir, name, ea, sizeof(double) * NC * HQ * D);
        free(eo);
        free(el);
        free(ea);
      }
      free(pool);
    }
  }
  /* workspace extend over rows [0, 45 + 9) of k / v */
  double* wo = malloc(sizeof(double) * NC * HQ * D);
  double* wl = malloc(sizeof(double) * NC * HQ);
  kvqo_extend_attention(qe, HQ * D, HQ, k, v, HKV * D, HKV, D, LP, NC, sm, wo, wl);
  write_file(dir, "ws_o", wo, sizeof(double) * NC * HQ * D);
  write_file(dir, "ws_lse", wl, sizeof(double) * NC * HQ);
  free(wo);
  free(wl);
  /* row codecs and helpers */
  uint8_t codes[D / 2], scales[D / 16];
  float s = 0.0f, x[D];
  double row[D];
  kvqo_nvfp4_quantize_row(k, D, gs[0], codes, scales);
  kvqo_nvfp4_dequant_row(codes, scales, D, gs[0], row);
  write_file(dir, "row_nvfp4", row, sizeof(row));
  kvqo_int4_quantize_row(k, D, codes, &s);
  kvqo_int4_dequant_row(codes, s, D, row);
  write_file(dir, "row_int4", row, sizeof(row));
  memcpy(x, k, sizeof(x));
  kvqo_hadamard_row(x, D);
  write_file(dir, "row_hadamard", x, sizeof(x));
  const float amax = kvqo_amax(k, (int64_t)NTOK * HKV * D);
  write_file(dir, "amax", &amax, sizeof(amax));
  free(k);
  free(v);
  free(q);
  free(slots);
  free(bt);
  free(lens);
  free(gs);
  free(kc);
  free(vc);
  free(qe);
  printf("oracle sanitized run ok\n");
  return 0;
}
