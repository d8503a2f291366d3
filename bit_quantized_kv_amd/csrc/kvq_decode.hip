// kvq_decode.hip -- paged split-context decode attention over the 4-bit
// cache, for gfx950 (MI355X).
//
// What it computes ("SGLang's 4-bit KV cache: the 56% is exact, the 1.78x is
// untested", Figure 2 caption: decode reads the NVFP4 pool directly and
// dequantizes inside the kernel; "KV cache in 4 bits: 8.8 instead of 4.7 full
// sessions ...", "What we changed": the INT4 per-token-head read side): for
// each sequence and query head, softmax(sm_scale * q K^T) V over every cached
// token, the K and V rows decoded from their packed nibbles and scales in
// registers, never expanded in memory.
//
// Structure (one 64-lane wavefront per workgroup):
//   grid = (splits, KV heads, batch).  A split is a run of whole 32-token
//   chunks of one (sequence, KV head); its wavefront computes the partial
//   (o, max, sum) of all G <= 16 query heads of the group and a second kernel
//   merges the splits with the log-sum-exp rule in split order.
//   Per 32-token chunk (two 16-token halves, each inside one page):
//     QK  S^T[token][query] = K[token][ch] Q^T[ch][query] with
//         v_mfma_f32_16x16x32_f16 (G padded to 16); lane (j = lane/16,
//         t = lane%16) loads 2 x 16 B of token t's code row, so each load
//         instruction covers 16 rows x 64 contiguous bytes.  The reduction
//         axis is permuted identically for q and K.
//     softmax  online, base 2, lazily rescaled: the running max only moves
//         when a chunk exceeds it by more than 2^8, so the O rescale is rare.
//     PV  O^T[ch][query] += V^T[ch][token] P^T[token][query], 16 channels per
//         MFMA; lane (j, r) loads the 16-channel segment r of tokens
//         4j..4j+3 of each half (again fully coalesced: 4 rows per load);
//         token pairs are interleaved at nibble level so one conversion
//         yields an fp16 pair (token a, token b) of one channel.
//   Dequantization: NVFP4 nibbles -> fp16 with v_cvt_scalef32_pk_f16_fp4
//   (unit scale), times the E4M3 block scale with a packed fp16 multiply --
//   e2m1 * e4m3 has at most 6 significant bits, so K and V are exact in fp16;
//   the per-layer global scales are applied to the fp32 scores / outputs.
//   INT4 nibbles -> fp16 exactly via the 1024-offset trick; the per-token
//   scales are folded into the score (K) and into the probability (V).
//   q is scaled by a power of two so its largest magnitude sits in
//   [2^14, 2^15), keeping fp16 exact for every finite bf16 input range.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;
static constexpr float kRescaleSlack = 8.0f;  // log2 of the largest unnormalised p

template <int D, int FMT>
struct ChunkRegs {
  static constexpr int VEC = D / 128;  // 16-byte K vectors per lane and token
  static constexpr int VW = D / 128;   // V dwords per lane and token (D/32 bytes)
  uint4 kw[2][VEC];
  uint32_t ks[2][VEC];  // NVFP4: two E4M3 block-scale bytes
  float4 ksc[2];        // INT4: K scales of tokens 4j..4j+3
  uint32_t vw[2][4][VW];
  uint32_t vs[2][4];  // NVFP4: V block-scale byte of token 4j+i
  float4 vsc[2];      // INT4: V scales of tokens 4j..4j+3
};

template <int D, int FMT>
struct Decoder {
  static constexpr int VEC = D / 128;
  static constexpr int VW = D / 128;
  static constexpr int KCH = D / 32;  // QK MFMAs per half
  static constexpr int VT = D / 16;   // PV MFMAs (16-channel tiles)
  using Regs = ChunkRegs<D, FMT>;

  const DecodeParams& p;
  const int lane, j, r, b, g, L;
  const uint8_t* head_base;  // pool + g * slab
  const int32_t* pages;      // block_table row of sequence b

  __device__ Decoder(const DecodeParams& p_, int lane_, int b_, int g_, int L_)
      : p(p_), lane(lane_), j(lane_ >> 4), r(lane_ & 15), b(b_), g(g_), L(L_) {
    head_base = p.pool + (int64_t)g * p.slab;
    pages = p.block_table + (int64_t)b * p.max_pages;
  }

  // Slab address of the half-chunk starting at token tok0 (a multiple of 16);
  // a half past the end of the sequence reuses the first half's address.
  __device__ inline const uint8_t* half_base(int tok0, int& off) const {
    const int64_t page = pages[tok0 / p.page_size];
    off = tok0 % p.page_size;
    return head_base + page * p.num_kv_heads * p.slab;
  }

  __device__ inline void load(Regs& R, int c) const {
    const int T = c * 32;
    int off[2];
    const uint8_t* base[2];
    base[0] = half_base(T, off[0]);
    if (T + 16 < L) {
      base[1] = half_base(T + 16, off[1]);
    } else {
      base[1] = base[0];
      off[1] = off[0];
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint8_t* kb = base[h];
      const uint8_t* vb = base[h] + p.half;
      const int krow = off[h] + r;
#pragma unroll
      for (int v = 0; v < VEC; v++) R.kw[h][v] = *(const uint4*)(kb + (int64_t)krow * (D / 2) + 64 * v + 16 * j);
      if (FMT == FMT_NVFP4) {
#pragma unroll
        for (int v = 0; v < VEC; v++)
          R.ks[h][v] = *(const uint16_t*)(kb + p.scales_off + (int64_t)krow * (D / 16) + 8 * v + 2 * j);
      } else {
        R.ksc[h] = *(const float4*)(kb + p.scales_off + (int64_t)(off[h] + 4 * j) * 4);
        R.vsc[h] = *(const float4*)(vb + p.scales_off + (int64_t)(off[h] + 4 * j) * 4);
      }
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int vrow = off[h] + 4 * j + i;
        const uint8_t* vp = vb + (int64_t)vrow * (D / 2) + r * (D / 32);
        if (VW == 2) {
          uint2 w = *(const uint2*)vp;
          R.vw[h][i][0] = w.x;
          R.vw[h][i][VW - 1] = w.y;
        } else {
          R.vw[h][i][0] = *(const uint32_t*)vp;
        }
        if (FMT == FMT_NVFP4) R.vs[h][i] = vb[p.scales_off + (int64_t)vrow * (D / 16) + (r * (D / 16)) / 16];
      }
    }
  }

  // One QK MFMA operand: 8 fp16 K values of chunk (v, w) for this lane's token.
  __device__ inline half8_t k_operand(const Regs& R, int h, int v, int w, half2_t s2) const {
    const uint32_t word = w == 0 ? R.kw[h][v].x : w == 1 ? R.kw[h][v].y : w == 2 ? R.kw[h][v].z : R.kw[h][v].w;
    half2_t a0, a1, a2, a3;
    if (FMT == FMT_NVFP4) {
      a0 = e2m1x2_to_h2<0>(word) * s2;
      a1 = e2m1x2_to_h2<1>(word) * s2;
      a2 = e2m1x2_to_h2<2>(word) * s2;
      a3 = e2m1x2_to_h2<3>(word) * s2;
    } else {
      const uint32_t wb = word ^ 0x88888888u;
      a0 = int4x2_to_h2<0>(wb);
      a1 = int4x2_to_h2<1>(wb);
      a2 = int4x2_to_h2<2>(wb);
      a3 = int4x2_to_h2<3>(wb);
    }
    return (half8_t){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
  }

  // Channel of element e of QK chunk (v, w) for lane group j (must match
  // k_operand's element order).
  __device__ static inline int k_channel(int v, int w, int jj, int e) {
    if (FMT == FMT_NVFP4) return 128 * v + 32 * jj + 8 * w + e;
    return 128 * v + 32 * jj + 8 * w + (e >> 1) + 4 * (e & 1);
  }
};

// DUP (group <= 8): MFMA columns 8..15 repeat queries 0..7 and carry the
// low-order fp16 part of the probabilities, so P = hi + lo costs no extra
// MFMA; otherwise the low part takes a second MFMA per tile.
template <int D, int FMT, bool DUP>
__global__ __launch_bounds__(64) void decode_kernel(const DecodeParams p) {
  using Dec = Decoder<D, FMT>;
  using Regs = typename Dec::Regs;
  constexpr int VEC = Dec::VEC, VW = Dec::VW, KCH = Dec::KCH, VT = Dec::VT;

  const int lane = threadIdx.x;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = p.seq_lens[b];
  const int G = p.group;
  const int j = lane >> 4, n = lane & 15;
  const int64_t part = ((int64_t)b * p.num_kv_heads + g) * p.num_splits + split;
  float* ml = p.part_ml + part * G * 2;
  float* po = p.part_o + part * G * D;

  const int nchunks = (L + 31) / 32;
  const int c0 = split * p.chunks_per_split;
  const int c1 = min(nchunks, c0 + p.chunks_per_split);
  if (c0 >= c1) {
    if (j == 0 && n < G) {
      ml[2 * n] = -__builtin_inff();
      ml[2 * n + 1] = 0.0f;
    }
    return;
  }

  Dec dec(p, lane, b, g, L);

  // ---- q operand (B of the QK MFMA): lane (j, n) holds query n, the 8
  // channels k_channel(v, w, j, 0..7) of chunk (v, w).  Scaled by 2^kq.
  float qf[KCH][8];
  float qmax = 0.0f;
  {
    const int qn = DUP ? (n & 7) : n;
    const uint16_t* qrow = p.q + ((int64_t)b * p.num_q_heads + (int64_t)g * G + (qn < G ? qn : 0)) * D;
#pragma unroll
    for (int v = 0; v < VEC; v++) {
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const uint4 raw = *(const uint4*)(qrow + 128 * v + 32 * j + 8 * w);
        const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
        float nat[8];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          nat[2 * e] = as_f32(rw[e] << 16);
          nat[2 * e + 1] = as_f32(rw[e] & 0xFFFF0000u);
        }
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int ch = Dec::k_channel(v, w, j, e) - (128 * v + 32 * j + 8 * w);
          float x = qn < G ? nat[ch] : 0.0f;
          qf[4 * v + w][e] = x;
          qmax = fmaxf(qmax, __builtin_fabsf(x));
        }
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, m, 64));
  int qexp = 0;
  if (qmax > 0.0f) (void)frexpf(qmax, &qexp);  // qmax < 2^qexp
  const int kq = qmax > 0.0f ? 15 - qexp : 0;
  half8_t qop[KCH];
#pragma unroll
  for (int c = 0; c < KCH; c++) {
#pragma unroll
    for (int e = 0; e < 8; e++) qop[c][e] = (_Float16)ldexpf(qf[c][e], kq);
  }
  const float sm = p.sm_scale * kLog2e * ldexpf(1.0f, -kq) * (FMT == FMT_NVFP4 ? p.gs[0] : 1.0f);

  float4_t oacc[VT];
#pragma unroll
  for (int t = 0; t < VT; t++) oacc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  auto compute = [&](const Regs& R, int c) {
    const int T = c * 32;
    // ---------------- QK
    float4_t sacc[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      sacc[h] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int v = 0; v < VEC; v++) {
        half2_t s_lo = {}, s_hi = {};
        if (FMT == FMT_NVFP4) {
          const float2_t s01 = __builtin_amdgcn_cvt_pk_f32_fp8(R.ks[h][v], false);
          s_lo = (half2_t){(_Float16)s01[0], (_Float16)s01[0]};
          s_hi = (half2_t){(_Float16)s01[1], (_Float16)s01[1]};
        }
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const half8_t a = dec.k_operand(R, h, v, w, w < 2 ? s_lo : s_hi);
          sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qop[4 * v + w], sacc[h], 0, 0, 0);
        }
      }
    }
    // ---------------- scores (log2 units) and chunk max
    float s[2][4], cand[2][4], sv[2][4];
    float cmax = -__builtin_inff();
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const float ksc[4] = {R.ksc[h].x, R.ksc[h].y, R.ksc[h].z, R.ksc[h].w};
      const float vsc[4] = {R.vsc[h].x, R.vsc[h].y, R.vsc[h].z, R.vsc[h].w};
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const bool valid = T + 16 * h + 4 * j + q < L;
        float x = sacc[h][q] * sm;
        if (FMT == FMT_INT4) x *= ksc[q];
        s[h][q] = valid ? x : -__builtin_inff();
        if (FMT == FMT_INT4) {
          sv[h][q] = valid ? vsc[q] : 0.0f;
          const float lv = fmaxf(log2f(sv[h][q]), -64.0f);
          cand[h][q] = valid ? x + lv : -__builtin_inff();
        } else {
          cand[h][q] = s[h][q];
        }
        cmax = fmaxf(cmax, cand[h][q]);
      }
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    if (__builtin_amdgcn_ballot_w64(cmax > m_run + kRescaleSlack) != 0) {
      const float m_new = cmax > m_run + kRescaleSlack ? cmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < VT; t++) oacc[t] *= alpha;
    }
    // ---------------- probabilities -> fp16 B operand of the PV MFMA
    float pr[2][4];
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const float e = __builtin_amdgcn_exp2f(s[h][q] - m_run);
        l_run += e;
        pr[h][q] = FMT == FMT_INT4 ? e * sv[h][q] : e;
      }
    }
    // p = hi + lo, both fp16: the PV product keeps ~22 bits of each p
    half8_t pop_hi, pop_lo;
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const _Float16 hi = (_Float16)pr[h][q];
        const _Float16 lo = (_Float16)(pr[h][q] - (float)hi);
        pop_hi[4 * h + q] = hi;
        pop_lo[4 * h + q] = lo;
      }
    }
    const half8_t pop = DUP ? (n < 8 ? pop_hi : pop_lo) : pop_hi;
    // ---------------- V: nibble-interleave token pairs (2i, 2i+1)
    uint32_t pw[2][2][VW][2];  // [half][pair][dword][lo/hi or W0/W1]
    half2_t vsc2[2][2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
      for (int pp = 0; pp < 2; pp++) {
#pragma unroll
        for (int d = 0; d < VW; d++) {
          const uint32_t a = R.vw[h][2 * pp][d], bb = R.vw[h][2 * pp + 1][d];
          if (FMT == FMT_NVFP4) {
            pw[h][pp][d][0] = bitfield_insert(0x0F0F0F0Fu, a, bb << 4);
            pw[h][pp][d][1] = bitfield_insert(0x0F0F0F0Fu, a >> 4, bb);
          } else {
            pw[h][pp][d][0] = byte_perm(bb, a, 0x05040100u) ^ 0x88888888u;
            pw[h][pp][d][1] = byte_perm(bb, a, 0x07060302u) ^ 0x88888888u;
          }
        }
        if (FMT == FMT_NVFP4) {
          const bool va = T + 16 * h + 4 * j + 2 * pp < L, vb = T + 16 * h + 4 * j + 2 * pp + 1 < L;
          const float2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(R.vs[h][2 * pp] | (R.vs[h][2 * pp + 1] << 8), false);
          vsc2[h][pp] = (half2_t){(_Float16)(va ? f[0] : 0.0f), (_Float16)(vb ? f[1] : 0.0f)};
        }
      }
    }
    // ---------------- PV
#pragma unroll
    for (int t = 0; t < VT; t++) {
      const int d = t / 8, cc = t % 8;
      half2_t parts[4];
#pragma unroll
      for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int pp = 0; pp < 2; pp++) {
          half2_t x;
          if (FMT == FMT_NVFP4) {
            const uint32_t word = pw[h][pp][d][cc & 1];
            switch (cc >> 1) {
              case 0: x = e2m1x2_to_h2<0>(word); break;
              case 1: x = e2m1x2_to_h2<1>(word); break;
              case 2: x = e2m1x2_to_h2<2>(word); break;
              default: x = e2m1x2_to_h2<3>(word); break;
            }
            x = x * vsc2[h][pp];
          } else {
            const uint32_t word = pw[h][pp][d][cc >> 2];
            switch (cc & 3) {
              case 0: x = int4x2_to_h2<0>(word); break;
              case 1: x = int4x2_to_h2<1>(word); break;
              case 2: x = int4x2_to_h2<2>(word); break;
              default: x = int4x2_to_h2<3>(word); break;
            }
          }
          parts[2 * h + pp] = x;
        }
      }
      const half8_t a = {parts[0][0], parts[0][1], parts[1][0], parts[1][1],
                         parts[2][0], parts[2][1], parts[3][0], parts[3][1]};
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pop, oacc[t], 0, 0, 0);
      if (!DUP) oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pop_lo, oacc[t], 0, 0, 0);
    }
  };

  // ---- main loop, software-pipelined by one chunk
  Regs RA, RB;
  dec.load(RA, c0);
  for (int c = c0; c < c1; c += 2) {
    if (c + 1 < c1) dec.load(RB, c + 1);
    compute(RA, c);
    if (c + 1 >= c1) break;
    if (c + 2 < c1) dec.load(RA, c + 2);
    compute(RB, c + 1);
  }

  // ---- partial results
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (DUP) {
    // columns n and n + 8 hold the hi and lo parts of query n
#pragma unroll
    for (int t = 0; t < VT; t++) {
#pragma unroll
      for (int rr = 0; rr < 4; rr++) oacc[t][rr] += __shfl_xor(oacc[t][rr], 8, 64);
    }
  }
  if (n < G) {
    if (j == 0) {
      ml[2 * n] = m_run;
      ml[2 * n + 1] = l_run;
    }
    const float scale_o = FMT == FMT_NVFP4 ? p.gs[1] : 1.0f;
    float* dst = po + (int64_t)n * D;
    // O^T tile t, row 4j + rr <-> channel (4j + rr) * (D/16) + t
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      float* row = dst + (4 * j + rr) * VT;
#pragma unroll
      for (int t = 0; t < VT; t += 4)
        *(float4*)(row + t) = make_float4(oacc[t][rr] * scale_o, oacc[t + 1][rr] * scale_o,
                                          oacc[t + 2][rr] * scale_o, oacc[t + 3][rr] * scale_o);
    }
  }
}

// Merge the splits of one (sequence, query head): M = max m_s,
// o = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s, lse = (M + log2 sum) ln 2.
// Splits are visited in order, so the result is reproducible.
template <int D>
__global__ __launch_bounds__(D) void merge_kernel(const DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int G = p.group, g = h / G, n = h % G, S = p.num_splits;
  const int64_t part0 = ((int64_t)b * p.num_kv_heads + g) * S;
  float M = -__builtin_inff();
  for (int s = 0; s < S; s++) M = fmaxf(M, p.part_ml[((part0 + s) * G + n) * 2]);
  float o = 0.0f, den = 0.0f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < S; s++) {
      const float ms = p.part_ml[((part0 + s) * G + n) * 2];
      if (ms == -__builtin_inff()) continue;
      const float w = exp2f(ms - M);
      den += w * p.part_ml[((part0 + s) * G + n) * 2 + 1];
      o += w * p.part_o[((part0 + s) * G + n) * D + c];
    }
    o = o / den;
  }
  const int64_t oi = ((int64_t)b * p.num_q_heads + h) * D + c;
  if (p.out_bf16)
    ((uint16_t*)p.out)[oi] = f32_to_bf16_rne(o);
  else
    ((float*)p.out)[oi] = o;
  if (p.lse != nullptr && c == 0)
    p.lse[(int64_t)b * p.num_q_heads + h] = den > 0.0f ? (M + log2f(den)) * kLn2 : -__builtin_inff();
}

hipError_t launch_decode(const DecodeParams& p, int fmt, int head_dim, hipStream_t stream) {
  const dim3 grid(p.num_splits, p.num_kv_heads, p.batch), block(64);
  const dim3 mgrid(p.num_q_heads, p.batch);
  const bool dup = p.group <= 8;
#define KVQ_DECODE(D, F)                                                                        \
  do {                                                                                          \
    if (dup) hipLaunchKernelGGL((decode_kernel<D, F, true>), grid, block, 0, stream, p);        \
    else hipLaunchKernelGGL((decode_kernel<D, F, false>), grid, block, 0, stream, p);           \
  } while (0)
  if (head_dim == 256) {
    if (fmt == FMT_NVFP4) KVQ_DECODE(256, FMT_NVFP4);
    else KVQ_DECODE(256, FMT_INT4);
    hipLaunchKernelGGL((merge_kernel<256>), mgrid, dim3(256), 0, stream, p);
  } else {
    if (fmt == FMT_NVFP4) KVQ_DECODE(128, FMT_NVFP4);
    else KVQ_DECODE(128, FMT_INT4);
    hipLaunchKernelGGL((merge_kernel<128>), mgrid, dim3(128), 0, stream, p);
  }
#undef KVQ_DECODE
  return hipGetLastError();
}

}  // namespace kvq
