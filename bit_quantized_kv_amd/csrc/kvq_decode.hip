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
// Structure (kDecodeWaves = 4 wavefronts per workgroup):
//   grid = (splits, KV heads, batch).  A split is a run of whole 32-token
//   chunks of one (sequence, KV head), dealt to the workgroup's wavefronts
//   round-robin; each wavefront keeps a partial (o, max, sum) of all G <= 16
//   query heads of the group, the workgroup combines its wavefronts' partials
//   in LDS, and a second kernel merges the splits with the log-sum-exp rule
//   in split order.  The page walk (chunk cursor, page-table reads, slab
//   descriptors) is wavefront-uniform and runs on the scalar unit; each
//   chunk's loads are issued one chunk ahead of its math.
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
//         yields an fp16 pair (token a, token b) of one channel.  The value
//         scales and the interleave are computed before the softmax, where
//         they fill the wait for the QK products.
//   Dequantization: NVFP4 nibbles -> fp16 times 2^8 with
//   v_cvt_scalef32_pk_f16_fp4 (its scale operand acts as a power of two),
//   times the E4M3 block scale times 2^-8 with a packed fp16 multiply --
//   e2m1 * e4m3 has at most 6 significant bits, so K and V are exact in fp16;
//   the per-layer global scales are applied to the fp32 scores / outputs.
//   INT4 nibbles -> fp16 exactly via the 1024-offset trick; the per-token
//   scales are folded into the score (K) and into the probability (V).
//   q is scaled by a power of two so its largest magnitude sits in
//   [2^14, 2^15): every bf16 element within 2^32 of the largest is then exact
//   in fp16 (smaller ones round, far below the fp32 accumulation's precision).
#include <mutex>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;
static constexpr float kRescaleSlack = 8.0f;  // log2 of the largest unnormalised p
static constexpr int kWaves = kDecodeWaves;   // wavefronts per decode workgroup

// lane l + (l ^ 8): DPP row rotation by 8 within each 16-lane row (VALU only).
__device__ inline float add_xor8(float x) {
  return x + as_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(x), 0x128, 0xF, 0xF, false));
}

// The workgroup's partial result.  Each wave has put its unnormalised o in
// sm_o ([kWaves][G][D], its own slice) and its running (m, l) per query in
// sm_ml ([kWaves][G][2]).  After one barrier every thread takes float4s of
// the [G][D] result: o = sum over waves, in wave order, of o_w * 2^(m_w - M)
// * vscale (an empty wave, m_w = -inf, weighs 0), M the largest m_w; and the
// first G threads write (M, l = sum of 2^(m_w - M) l_w).  Fixed order
// throughout: the partial is reproducible.
template <int D>
__device__ inline void finish_partial(const float* sm_o, const float* sm_ml, int G, float vscale, float* po,
                                      float* ml) {
  __syncthreads();
  const int tid = threadIdx.x;
  for (int i = tid; i < G * (D / 4); i += 64 * kWaves) {
    const int n = i / (D / 4);
    float mw[kWaves], M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
      mw[w] = sm_ml[(w * G + n) * 2];
      M = fmaxf(M, mw[w]);
    }
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
      const float sc = mw[w] == -__builtin_inff() ? 0.0f : exp2f(mw[w] - M) * vscale;
      const float4 x = ((const float4*)(sm_o + (size_t)w * G * D))[i];
      if (w == 0) {
        acc = make_float4(x.x * sc, x.y * sc, x.z * sc, x.w * sc);
      } else {
        acc.x += x.x * sc;
        acc.y += x.y * sc;
        acc.z += x.z * sc;
        acc.w += x.w * sc;
      }
    }
    ((float4*)po)[i] = acc;
  }
  if (tid < G) {
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; w++) M = fmaxf(M, sm_ml[(w * G + tid) * 2]);
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
      const float m = sm_ml[(w * G + tid) * 2];
      if (m != -__builtin_inff()) l += exp2f(m - M) * sm_ml[(w * G + tid) * 2 + 1];
    }
    ml[2 * tid] = M;
    ml[2 * tid + 1] = l;
  }
}

template <int D, int FMT>
struct ChunkRegs {
  static constexpr int VEC = D / 128;  // 16-byte 4-bit K vectors per lane and token
  static constexpr int KVEC = FMT == FMT_K8V4 ? D / 64 : VEC;  // K8V4: FP8 keys, twice the bytes
  static constexpr int VW = D / 128;   // V dwords per lane and token (D/32 bytes)
  u32x4_t kw[2][KVEC];
  uint32_t ks[2][VEC];  // NVFP4: dword holding the lane's two E4M3 block scales
  uint32_t ksc[2];      // INT4: K scale (fp32 bits) of token 4j + r%4 (quad-broadcast later)
  uint32_t vw[2][4][VW];
  uint32_t vs[2];     // NVFP4: one dword of the half's V scales (see load)
  uint32_t vsc[2];    // INT4: V scale (fp32 bits) of token 4j + r%4
};

// Walking one (sequence, KV head)'s pages in 32-token chunks: page-table
// entries, row offsets and the per-slab buffer descriptor.
struct PageWalk {
  const DecodeParams& p;
  const int L;
  const uint8_t* head_base;      // pool + g * slab
  __amdgpu_buffer_rsrc_t pages;  // block_table row of sequence b

  __device__ PageWalk(const DecodeParams& p_, int b, int g, int L_) : p(p_), L(L_) {
    head_base = p.pool + (int64_t)g * p.slab;
    pages = __builtin_amdgcn_make_buffer_rsrc((void*)(p.block_table + (int64_t)b * p.max_pages), (short)0,
                                              p.max_pages * 4, 0x00020000);
  }

  // Position of a chunk in the page table, advanced without division: the
  // chunk's first token T = page_idx * page_size + row.
  struct Cursor {
    int c, page_idx, row;
  };

  __device__ inline Cursor cursor_at(int c) const {
    const int T = __builtin_amdgcn_readfirstlane(c * 32);
    return Cursor{__builtin_amdgcn_readfirstlane(c), T / p.page_size, T % p.page_size};
  }

  // Move the cursor `stride` chunks on (at most up to chunk `clast`), with
  // the precomputed quotient and remainder of 32 * stride by the page size.
  __device__ inline void advance(Cursor& k, int stride, int clast, int dq, int dr) const {
    if (k.c + stride > clast) return;
    k.c += stride;
    k.page_idx += dq;
    k.row += dr;
    if (k.row >= p.page_size) {
      k.row -= p.page_size;
      k.page_idx += 1;
    }
  }

  // Where a chunk's two 16-token halves live: page ids (read with vector
  // loads whose table offsets are scalar, so the walk itself stays on the
  // scalar unit and the wait stays off the scalar counter; issued well before
  // use) and rows.  A half past the end of the sequence repeats the first half.
  struct ChunkRef {
    int2 pg;
    int row0, row1;
  };

  __device__ inline ChunkRef fetch(const Cursor& k) const {
    int i0 = k.page_idx, i1 = k.page_idx, row1 = k.row;
    if (k.c * 32 + 16 < L) {
      row1 = k.row + 16;
      if (row1 >= p.page_size) {
        row1 -= p.page_size;
        i1 += 1;
      }
    }
    return ChunkRef{make_int2(__builtin_amdgcn_raw_buffer_load_b32(pages, 0, 4 * i0, 0),
                              __builtin_amdgcn_raw_buffer_load_b32(pages, 0, 4 * i1, 0)),
                    k.row, row1};
  }

  // Buffer descriptor of one slab: base address in SGPRs, range-checked to
  // the slab, so every load below is one loop-invariant VGPR offset plus
  // uniform (SGPR / immediate) offsets.
  __device__ inline __amdgpu_buffer_rsrc_t slab_rsrc(int page) const {
    const uint8_t* base = head_base + (int64_t)page * p.num_kv_heads * p.slab;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)p.slab, 0x00020000);
  }

};

template <int D, int FMT>
struct Decoder : PageWalk {
  static constexpr int VEC = D / 128;
  static constexpr int VW = D / 128;
  static constexpr int KCH = D / 32;  // QK MFMAs per half
  static constexpr int VT = D / 16;   // PV MFMAs (16-channel tiles)
  static constexpr int KVEC = ChunkRegs<D, FMT>::KVEC;
  static constexpr bool K8 = FMT == FMT_K8V4;   // FP8 keys (by token, per-tensor scale)
  static constexpr bool VNV = FMT != FMT_INT4;  // NVFP4 values
  using Regs = ChunkRegs<D, FMT>;

  const int lane, j, r;
  int vo_k, vo_ks, vo_vs_h, vo_sc, vo_sc_h, vo_v_h;  // per-lane byte offsets inside a slab

  __device__ Decoder(const DecodeParams& p_, int lane_, int b_, int g_, int L_)
      : PageWalk(p_, b_, g_, L_), lane(lane_), j(lane_ >> 4), r(lane_ & 15) {
    // (the _h offsets include the K half, i.e. they address the V half)
    vo_k = r * (K8 ? D : D / 2) + 16 * j;                                   // K code row r
    vo_ks = r * (D / 16) + 4 * (j >> 1);                                    // K scale row r
    vo_vs_h = (int)p.half + (4 * j + (r & 3)) * (D / 16) + 4 * (((r >> 2) * D) / 256);
    vo_sc = (4 * j + (r & 3)) * 4;                                          // INT4 scale of row 4j + r%4
    vo_sc_h = (int)p.half + vo_sc;
    vo_v_h = (int)p.half + 4 * j * (D / 2) + r * (D / 32);                  // V code rows 4j + i
  }

  // Loads of one chunk: the descriptor and the chunk's row offsets are
  // uniform (SGPR descriptor and soffset), the lane's position inside a row is
  // a loop-invariant VGPR offset, and constant parts fold into the
  // instruction's immediate offset, so issuing a load costs no VALU work.
  __device__ inline void load(Regs& R, const ChunkRef& ref) const {
    const int2 pg = ref.pg;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const __amdgpu_buffer_rsrc_t rs = slab_rsrc(__builtin_amdgcn_readfirstlane(h == 0 ? pg.x : pg.y));
      const int off = __builtin_amdgcn_readfirstlane(h == 0 ? ref.row0 : ref.row1);
      const int ko = off * (K8 ? D : D / 2);  // K rows
      const int vko = off * (D / 2);          // V code rows
      const int so = (int)p.scales_off + off * (FMT == FMT_INT4 ? 4 : D / 16);
      // K codes: row off + r, bytes 64v + 16j
#pragma unroll
      for (int v = 0; v < KVEC; v++)
        R.kw[h][v] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo_k + 64 * v, ko, kLoadStream);
      if (FMT == FMT_NVFP4) {
#pragma unroll
        for (int v = 0; v < VEC; v++)
          R.ks[h][v] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo_ks + 8 * v, so, kLoadStream);
      }
      if (VNV) {
        // Lane (j, r) with quad Q = r / 4 loads the dword of V-scale row 4j + r%4
        // that holds block (r * D / 256), the block every lane of quad Q needs;
        // compute() broadcasts row i of the quad with a DPP quad_perm.
        R.vs[h] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo_vs_h, so, kLoadStream);
      } else {
        R.ksc[h] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo_sc, so, kLoadStream);
        R.vsc[h] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo_sc_h, so, kLoadStream);
      }
      // V codes: rows off + 4j + i, the lane's D/32-byte segment r
#pragma unroll
      for (int i = 0; i < 4; i++) {
        if (VW == 2) {
          const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(rs, vo_v_h + i * (D / 2), vko, kLoadStream);
          R.vw[h][i][0] = w.x;
          R.vw[h][i][VW - 1] = w.y;
        } else {
          R.vw[h][i][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo_v_h + i * (D / 2), vko, kLoadStream);
        }
      }
    }
  }

  // One QK MFMA operand: 8 fp16 K values of chunk (v, w) for this lane's token.
  __device__ inline half8_t k_operand(const Regs& R, int h, int v, int w, half2_t s2) const {
    half2_t a0, a1, a2, a3;
    if (K8) {
      // FP8 keys: MFMA m = 4v + w takes 8 bytes (dwords 0-1 or 2-3 of vector
      // m / 2); E4M3 -> fp16 exactly at unit scale
      const int m = 4 * v + w;
      const u32x4_t kv4 = R.kw[h][m / 2];
      const uint32_t d0 = (m % 2) ? kv4.z : kv4.x, d1 = (m % 2) ? kv4.w : kv4.y;
      a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
      a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
      a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
      a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
      return (half8_t){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
    }
    const uint32_t word = w == 0 ? R.kw[h][v].x : w == 1 ? R.kw[h][v].y : w == 2 ? R.kw[h][v].z : R.kw[h][v].w;
    if (FMT == FMT_NVFP4) {
      // (e2m1 * 2^8) * (scale * 2^-8): pairs of channels (2k, 2k + 1)
      a0 = e2m1x2_to_h2_x256<0>(word) * s2;
      a1 = e2m1x2_to_h2_x256<1>(word) * s2;
      a2 = e2m1x2_to_h2_x256<2>(word) * s2;
      a3 = e2m1x2_to_h2_x256<3>(word) * s2;
    } else {
      // pairs 1 and 3 come out times 16; their query channels carry 1/16
      const uint32_t w8 = word >> 8;
      a0 = int4x2_to_h2<0>(word);
      a1 = int4x2_hi_to_h2_x16(word);
      a2 = int4x2_to_h2<0>(w8);
      a3 = int4x2_hi_to_h2_x16(w8);
    }
    return (half8_t){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
  }

  // First channel of the 8 channels of QK chunk (v, w) for lane group jj
  // (k_channel - k_base is in 0..7).
  __device__ static inline int k_base(int v, int w, int jj) {
    if (K8) {
      const int m = 4 * v + w;
      return 64 * (m / 2) + 16 * jj + 8 * (m % 2);
    }
    return 128 * v + 32 * jj + 8 * w;
  }

  // Channel of element e of QK chunk (v, w) for lane group j (must match
  // k_operand's element order).
  __device__ static inline int k_channel(int v, int w, int jj, int e) {
    if (K8) return k_base(v, w, jj) + e;
    if (FMT == FMT_NVFP4) return 128 * v + 32 * jj + 8 * w + e;
    return 128 * v + 32 * jj + 8 * w + (e >> 1) + 4 * (e & 1);
  }
};

// DUP (group <= 8): MFMA columns 8..15 repeat queries 0..7 and carry the
// low-order fp16 part of the probabilities, so P = hi + lo costs no extra
// MFMA; otherwise the low part takes a second MFMA per tile.
template <int D, int FMT, bool DUP>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(
    const DecodeParams p) {
  using Dec = Decoder<D, FMT>;
  using Regs = typename Dec::Regs;
  constexpr int VEC = Dec::VEC, VW = Dec::VW, KCH = Dec::KCH, VT = Dec::VT;
  extern __shared__ float smem[];  // [kWaves][G][D] partial o, then [kWaves][G] (m, l)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: the page walk stays scalar
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = p.seq_lens[b];
  const int G = p.group;
  const int j = lane >> 4, n = lane & 15;
  const int64_t part = ((int64_t)b * p.num_kv_heads + g) * p.num_splits + split;
  float* ml = p.part_ml + part * G * 2;
  float* po = p.part_o + part * G * D;

  // The workgroup's split [c0, c1) of 32-token chunks is dealt to its waves
  // round-robin: wave w takes chunks c0 + w, c0 + w + kWaves, ...
  const int nchunks = (L + 31) / 32;
  const int c0 = split * p.chunks_per_split;
  const int c1 = min(nchunks, c0 + p.chunks_per_split);
  if (c0 >= c1) {
    // empty split: (m, l) = (-inf, 0) and a zero o, so the merge can weight
    // every partial without a branch
    for (int i = threadIdx.x; i < G * D; i += 64 * kWaves) po[i] = 0.0f;
    if (threadIdx.x < G) {
      ml[2 * threadIdx.x] = -__builtin_inff();
      ml[2 * threadIdx.x + 1] = 0.0f;
    }
    return;
  }
  const int cw0 = c0 + wave;  // this wave's first chunk (may be >= c1)

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
        const uint4 raw = *(const uint4*)(qrow + Dec::k_base(v, w, j));
        const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
        float nat[8];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          nat[2 * e] = as_f32(rw[e] << 16);
          nat[2 * e + 1] = as_f32(rw[e] & 0xFFFF0000u);
        }
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int ch = Dec::k_channel(v, w, j, e) - Dec::k_base(v, w, j);
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
    for (int e = 0; e < 8; e++) {
      // INT4: elements 2, 3, 6, 7 meet K pairs decoded times 16 (k_operand)
      const int ke = FMT == FMT_INT4 && (e & 2) ? kq - 4 : kq;
      qop[c][e] = (_Float16)ldexpf(qf[c][e], ke);
    }
  }
  const float sm = p.sm_scale * kLog2e * ldexpf(1.0f, -kq) * (FMT != FMT_INT4 ? p.gs[0] : 1.0f);

  const float lo_sel = n < 8 ? 0.0f : 1.0f;  // DUP: lanes n >= 8 carry the low fp16 part of p
  // byte of block (n * D / 256) within its scale dword, from two dwords -> bytes 0, 2
  const uint32_t vb_byte = ((n * D) / 256) & 3;
  const uint32_t vsel = vb_byte | ((4 + vb_byte) << 16) | 0x0C000C00u;
  // the lane's two K block scales, bytes 2 (j & 1) and 2 (j & 1) + 1 of its
  // scale dword -> bytes 0, 2
  const uint32_t ksel = (2 * (j & 1)) | ((2 * (j & 1) + 1) << 16) | 0x0C000C00u;

  float4_t oacc[VT];
#pragma unroll
  for (int t = 0; t < VT; t++) oacc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  // FULL: all 32 tokens of the chunk are inside the sequence (no masking)
  auto compute = [&](const Regs& R, int c, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
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
          // the lane's two block scales as (scale_0, scale_1) * 2^-8 (the
          // e4m3_to_h_x2m8 move on both halves at once), each broadcast to a pair
          const half2_t s2 = u32_as_h2(e4m3_to_h_x2m8_pair(byte_perm(0u, R.ks[h][v], ksel)));
          s_lo = (half2_t){s2[0], s2[0]};
          s_hi = (half2_t){s2[1], s2[1]};
        }
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const half8_t a = dec.k_operand(R, h, v, w, w < 2 ? s_lo : s_hi);
          sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qop[4 * v + w], sacc[h], 0, 0, 0);
        }
      }
    }
    // (value-side preparation first: it does not depend on the scores and
    // fills the wait for the QK products)
    // ---------------- V scales of the token pairs (2pp, 2pp + 1) of each half
    half2_t vsc2[2][2];
    if (Dec::VNV) {
#pragma unroll
      for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int pp = 0; pp < 2; pp++) {
          // dwords of scale rows 4j + 2pp and 4j + 2pp + 1 (quad lanes 2pp, 2pp+1);
          // (s_a, s_b) * 2^-8 as an fp16 pair.  Past the end of the sequence the
          // bytes are arbitrary but decode finite, and p is exactly 0 there.
          const uint32_t d0 = pp == 0 ? quad_bcast<0>(R.vs[h]) : quad_bcast<2>(R.vs[h]);
          const uint32_t d1 = pp == 0 ? quad_bcast<1>(R.vs[h]) : quad_bcast<3>(R.vs[h]);
          const uint32_t ab = byte_perm(d1, d0, vsel);  // bytes [s_a, 0, s_b, 0]
          vsc2[h][pp] = u32_as_h2(e4m3_to_h_x2m8_pair(ab));
        }
      }
    }
    // token pairs (2i, 2i+1) of the value codes nibble-interleaved so one
    // conversion yields (token a, token b) of a single channel; groups of 4
    // tiles share the interleaved word of each pair (sel 0: even channels, 1: odd)
    uint32_t vpw[VW][2][2][2];
    if (Dec::VNV) {
#pragma unroll
      for (int d = 0; d < VW; d++) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
#pragma unroll
          for (int pp = 0; pp < 2; pp++) {
            const uint32_t a = R.vw[h][2 * pp][d], bb = R.vw[h][2 * pp + 1][d];
            vpw[d][0][h][pp] = bitfield_insert(0x0F0F0F0Fu, a, bb << 4);
            vpw[d][1][h][pp] = bitfield_insert(0x0F0F0F0Fu, a >> 4, bb);
            // computed here, not sunk past the softmax's branches to the PV loop
            asm volatile("" : "+v"(vpw[d][0][h][pp]), "+v"(vpw[d][1][h][pp]));
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 2; h++) asm volatile("" : "+v"(vsc2[h][0]), "+v"(vsc2[h][1]));
    }
    // INT4: nibbles of tokens a, b interleaved 16 bits apart (and the words
    // shifted by 8: nibble positions 2, 3 -> 0, 1), pinned here likewise
    uint32_t vpw8[VW][2][2][2];
    if (!Dec::VNV) {
#pragma unroll
      for (int d = 0; d < VW; d++) {
#pragma unroll
        for (int sel = 0; sel < 2; sel++) {
#pragma unroll
          for (int h = 0; h < 2; h++) {
#pragma unroll
            for (int pp = 0; pp < 2; pp++) {
              const uint32_t a = R.vw[h][2 * pp][d], bb = R.vw[h][2 * pp + 1][d];
              vpw[d][sel][h][pp] = byte_perm(bb, a, sel == 0 ? 0x05040100u : 0x07060302u);
              vpw8[d][sel][h][pp] = vpw[d][sel][h][pp] >> 8;
              asm volatile("" : "+v"(vpw[d][sel][h][pp]), "+v"(vpw8[d][sel][h][pp]));
            }
          }
        }
      }
    }
    // ---------------- scores (log2 units) and chunk max
    float s[2][4], cand[2][4], sv[2][4];
    float cmax = -__builtin_inff();
#pragma unroll
    for (int h = 0; h < 2; h++) {
      float ksc[4] = {}, vsc[4] = {};
      if (FMT == FMT_INT4) {
        // scales of tokens 4j + q, held by lane q of every quad
        ksc[0] = as_f32(quad_bcast<0>(R.ksc[h]));
        ksc[1] = as_f32(quad_bcast<1>(R.ksc[h]));
        ksc[2] = as_f32(quad_bcast<2>(R.ksc[h]));
        ksc[3] = as_f32(quad_bcast<3>(R.ksc[h]));
        vsc[0] = as_f32(quad_bcast<0>(R.vsc[h]));
        vsc[1] = as_f32(quad_bcast<1>(R.vsc[h]));
        vsc[2] = as_f32(quad_bcast<2>(R.vsc[h]));
        vsc[3] = as_f32(quad_bcast<3>(R.vsc[h]));
      }
#pragma unroll
      for (int q = 0; q < 4; q++) {
        float x = sacc[h][q] * sm;
        if (FMT == FMT_INT4) x *= ksc[q];
        s[h][q] = x;
        if (FMT == FMT_INT4) {
          sv[h][q] = vsc[q];
          // the running max also bounds p * (value scale): the scale's binary
          // exponent (frexp: scale < 2^e) is an upper bound of its log2 that
          // keeps p * scale below 2^slack; clamped so tiny scales cannot push
          // exp2(s - max) out of fp32 range
          cand[h][q] = x + (float)max(__builtin_amdgcn_frexp_expf(vsc[q]), -64);
        }
      }
    }
    // only the chunk holding the sequence's end has tokens past it (a
    // workgroup-uniform test, so other chunks skip the masking)
    if (!FULL && T + 32 > L) {
#pragma unroll
      for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          if (T + 16 * h + 4 * j + q >= L) {
            s[h][q] = -__builtin_inff();
            if (FMT == FMT_INT4) {
              sv[h][q] = 0.0f;
              cand[h][q] = -__builtin_inff();
            }
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        if (FMT != FMT_INT4) cand[h][q] = s[h][q];
        cmax = fmaxf(cmax, cand[h][q]);
      }
    }
    // a row's max can only pass m_run + slack where one of its lanes' own
    // maxima does, so the wave-wide test needs no cross-lane reduction; the
    // row max (over the row's 4 lanes) is formed only when some row moves
    if (__builtin_amdgcn_ballot_w64(cmax > m_run + kRescaleSlack) != 0) {
      cmax = max_xor16_xor32(cmax);
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
    // p = hi + lo, both fp16: the PV product keeps ~22 bits of each p.  With
    // DUP, lanes n < 8 feed hi and lanes n >= 8 (the repeated queries) feed lo:
    // each lane converts p - sub with sub = 0 or its own hi.
    half8_t pop, pop_lo;
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const _Float16 hi = (_Float16)pr[h][q];
        if (DUP) {
          pop[4 * h + q] = (_Float16)(pr[h][q] - lo_sel * (float)hi);
        } else {
          pop[4 * h + q] = hi;
          pop_lo[4 * h + q] = (_Float16)(pr[h][q] - (float)hi);
        }
      }
    }
    // ---------------- PV.  The A operand of tile t holds channel t of the
    // lane's 16-channel segment for the 8 tokens 4j..4j+3 of each half, as
    // fp16 pairs (token 2i, token 2i + 1).
    if (Dec::VNV) {
#pragma unroll
      for (int d = 0; d < VW; d++) {
#pragma unroll
        for (int sel = 0; sel < 2; sel++) {
          const uint32_t(&pw)[2][2] = vpw[d][sel];
#pragma unroll
          for (int k = 0; k < 4; k++) {
            const int t = 8 * d + 2 * k + sel;
            half2_t parts[4];
#pragma unroll
            for (int h = 0; h < 2; h++) {
#pragma unroll
              for (int pp = 0; pp < 2; pp++) {
                const uint32_t word = pw[h][pp];
                half2_t x;
                switch (k) {
                  case 0: x = e2m1x2_to_h2_x256<0>(word); break;
                  case 1: x = e2m1x2_to_h2_x256<1>(word); break;
                  case 2: x = e2m1x2_to_h2_x256<2>(word); break;
                  default: x = e2m1x2_to_h2_x256<3>(word); break;
                }
                parts[2 * h + pp] = x * vsc2[h][pp];
              }
            }
            const half8_t a = {parts[0][0], parts[0][1], parts[1][0], parts[1][1],
                               parts[2][0], parts[2][1], parts[3][0], parts[3][1]};
            oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pop, oacc[t], 0, 0, 0);
            if (!DUP) oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pop_lo, oacc[t], 0, 0, 0);
          }
        }
      }
    } else {
      // INT4: nibbles of tokens a, b interleaved 16 bits apart, so the 1024
      // offset trick yields (a, b) of one channel per conversion
#pragma unroll
      for (int d = 0; d < VW; d++) {
#pragma unroll
        for (int sel = 0; sel < 2; sel++) {
          const uint32_t(&pw)[2][2] = vpw[d][sel];
          const uint32_t(&pw8)[2][2] = vpw8[d][sel];
#pragma unroll
          for (int k = 0; k < 4; k++) {
            // odd tiles come out times 16, undone with the output scale
            const int t = 8 * d + 4 * sel + k;
            half2_t parts[4];
#pragma unroll
            for (int h = 0; h < 2; h++) {
#pragma unroll
              for (int pp = 0; pp < 2; pp++) {
                const uint32_t word = k < 2 ? pw[h][pp] : pw8[h][pp];
                parts[2 * h + pp] = (k & 1) ? int4x2_hi_to_h2_x16(word) : int4x2_to_h2<0>(word);
              }
            }
            const half8_t a = {parts[0][0], parts[0][1], parts[1][0], parts[1][1],
                               parts[2][0], parts[2][1], parts[3][0], parts[3][1]};
            oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pop, oacc[t], 0, 0, 0);
            if (!DUP) oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pop_lo, oacc[t], 0, 0, 0);
          }
        }
      }
    }
  };

  // ---- main loop, software-pipelined: chunk data one chunk ahead, page-table
  // entries two chunks ahead.  Loads are unconditional (past the end they
  // repeat the last chunk, an L2 hit) so the wait counts stay exact.
  // Each page-table fetch is issued before the chunk loads that precede its
  // use, so waiting for it never waits for chunk data (the counter is in order).
  constexpr int S1 = kWaves;
  if (cw0 < c1) {
    // last chunk of this wave's sequence c, c + S1, ...
    const int clast = cw0 + (c1 - 1 - cw0) / S1 * S1;
    const int dq = (32 * S1) / p.page_size, dr = (32 * S1) % p.page_size;
    {
      const std::false_type full_tag{};  // masked chunk math (a second, mask-free copy spills registers)
      Regs RA, RB;
      auto fc = dec.cursor_at(cw0);  // page-table fetch position, two chunks ahead
      const auto ref0 = dec.fetch(fc);
      dec.advance(fc, S1, clast, dq, dr);
      auto ref1 = dec.fetch(fc);
      dec.advance(fc, S1, clast, dq, dr);
      dec.load(RA, ref0);
      // scheduling barriers keep each chunk's loads ahead of the previous
      // chunk's math and stop the two computes from interleaving (which would
      // raise register pressure past two wavefronts per SIMD)
      for (int c = cw0; c <= clast; c += 2 * S1) {
        const auto ref2 = dec.fetch(fc);
        dec.advance(fc, S1, clast, dq, dr);
        dec.load(RB, ref1);
        __builtin_amdgcn_sched_barrier(0);
        compute(RA, c, full_tag);
        __builtin_amdgcn_sched_barrier(0);
        if (c + S1 > clast) break;
        ref1 = dec.fetch(fc);
        dec.advance(fc, S1, clast, dq, dr);
        dec.load(RA, ref2);
        __builtin_amdgcn_sched_barrier(0);
        compute(RB, c + S1, full_tag);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- partial results: reduce the lanes, then the waves (in LDS)
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (DUP) {
    // columns n and n + 8 hold the hi and lo parts of query n
#pragma unroll
    for (int t = 0; t < VT; t++) {
#pragma unroll
      for (int rr = 0; rr < 4; rr++) oacc[t][rr] = add_xor8(oacc[t][rr]);
    }
  }
  float* sm_o = smem;                        // [kWaves][G][D]: each wave's o
  float* sm_ml = smem + kWaves * G * D;      // [kWaves][G][2]
  if (n < G) {
    if (j == 0) {
      sm_ml[(wave * G + n) * 2] = m_run;
      sm_ml[(wave * G + n) * 2 + 1] = l_run;
    }
    // O^T tile t, row 4j + rr <-> channel (4j + rr) * (D/16) + t
    float* dst = sm_o + (wave * G + n) * D;
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
      float* row = dst + (4 * j + rr) * VT;
#pragma unroll
      for (int t = 0; t < VT; t += 4) {
        // INT4: odd tiles were accumulated from values times 16
        const float od = FMT == FMT_INT4 ? 0.0625f : 1.0f;
        *(float4*)(row + t) = make_float4(oacc[t][rr], oacc[t + 1][rr] * od, oacc[t + 2][rr], oacc[t + 3][rr] * od);
      }
    }
  }
  finish_partial<D>(sm_o, sm_ml, G, FMT != FMT_INT4 ? p.gs[1] : 1.0f, po, ml);
}

// ---------------------------------------------------------------- FP8 comparator
// Decode over the FP8 E4M3 per-tensor cache (the format the first page's
// 0.5625 ratio is taken against; "SGLang's 4-bit KV cache ...", section "The
// 56% survives its own scale, and names the block size").  Same grid, split
// plan, page walk, online softmax and merge as the 4-bit kernel; the step is
// one 16-token half (a half's K and V are 8 KB at D 256, so one half in
// flight matches the 4-bit kernel's register budget):
//   QK  v_mfma_f32_16x16x32_f16, lane (j, r) loads 16 B of token r's K row at
//       bytes 64w + 16j (w < D/64), i.e. channels 64w + 16j .. +16, which
//       feed MFMAs 2w and 2w + 1; q is permuted the same way.
//   PV  v_mfma_f32_16x16x16_f16 over the half's 16 tokens: the V section is
//       stored by channel, so lane (j, r) reads the 4 bytes of tokens 4j..4j+3
//       of channel 16t + r for tile t with one dword load, and the QK output
//       layout (lane (j, n): tokens 4j..4j+3 of query n) is already the B
//       operand of the PV product.
//   E4M3 -> fp16 with v_cvt_scalef32_pk_f16_fp8 at unit scale (exact); the
//   per-tensor scales go into the score scale (K) and the output (V).
template <int D>
struct Fp8Regs {
  u32x4_t kw[D / 64];
  uint32_t vw[D / 16];
};

template <int D, bool DUP>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2))) void decode_fp8_kernel(
    const DecodeParams p) {
  constexpr int KW = D / 64, KCH = D / 32, VT = D / 16;
  using Regs = Fp8Regs<D>;
  extern __shared__ float smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: the page walk stays scalar
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
    for (int i = threadIdx.x; i < G * D; i += 64 * kWaves) po[i] = 0.0f;
    if (threadIdx.x < G) {
      ml[2 * threadIdx.x] = -__builtin_inff();
      ml[2 * threadIdx.x + 1] = 0.0f;
    }
    return;
  }
  const int cw0 = c0 + wave;
  PageWalk walk(p, b, g, L);
  const int P = p.page_size;
  const int vo_k = n * D + 16 * j;                   // K row n, bytes 16j (+ 64w)
  const int vo_v = (int)p.half + n * P + 4 * j;      // V channel row n (+ 16t), tokens 4j..4j+3

  auto load = [&](Regs& R, int page, int row0) {
    const __amdgpu_buffer_rsrc_t rs = walk.slab_rsrc(__builtin_amdgcn_readfirstlane(page));
    const int off = __builtin_amdgcn_readfirstlane(row0);
#pragma unroll
    for (int w = 0; w < KW; w++)
      R.kw[w] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo_k + 64 * w, off * D, kLoadStream);
#pragma unroll
    for (int t = 0; t < VT; t++)
      R.vw[t] =
          __builtin_amdgcn_raw_buffer_load_b32(rs, vo_v, __builtin_amdgcn_readfirstlane(off + 16 * t * P), kLoadStream);
  };

  // q operand: lane (j, n) holds query n, channels 64(m/2) + 16j + 8(m%2) + e
  // of MFMA m, scaled by 2^kq as in the 4-bit kernel
  float qf[KCH][8];
  float qmax = 0.0f;
  {
    const int qn = DUP ? (n & 7) : n;
    const uint16_t* qrow = p.q + ((int64_t)b * p.num_q_heads + (int64_t)g * G + (qn < G ? qn : 0)) * D;
#pragma unroll
    for (int m = 0; m < KCH; m++) {
      const uint4 raw = *(const uint4*)(qrow + 64 * (m / 2) + 16 * j + 8 * (m % 2));
      const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float lo = qn < G ? as_f32(rw[e] << 16) : 0.0f;
        const float hi = qn < G ? as_f32(rw[e] & 0xFFFF0000u) : 0.0f;
        qf[m][2 * e] = lo;
        qf[m][2 * e + 1] = hi;
        qmax = fmaxf(qmax, fmaxf(__builtin_fabsf(lo), __builtin_fabsf(hi)));
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, m, 64));
  int qexp = 0;
  if (qmax > 0.0f) (void)frexpf(qmax, &qexp);
  const int kq = qmax > 0.0f ? 15 - qexp : 0;
  half8_t qop[KCH];
#pragma unroll
  for (int c = 0; c < KCH; c++) {
#pragma unroll
    for (int e = 0; e < 8; e++) qop[c][e] = (_Float16)ldexpf(qf[c][e], kq);
  }
  const float sm = p.sm_scale * kLog2e * ldexpf(1.0f, -kq) * p.gs[0];
  const float lo_sel = n < 8 ? 0.0f : 1.0f;

  float4_t oacc[VT];
#pragma unroll
  for (int t = 0; t < VT; t++) oacc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  // one 16-token half starting at token T
  auto compute = [&](Regs& R, int T) {
    float4_t sacc = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < KCH; m++) {
      const u32x4_t kw = R.kw[m / 2];
      const uint32_t d0 = (m % 2) ? kw.z : kw.x, d1 = (m % 2) ? kw.w : kw.y;
      const half2_t a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
      const half2_t a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
      const half2_t a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
      const half2_t a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
      const half8_t a = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qop[m], sacc, 0, 0, 0);
    }
    // tokens past the end: score -inf, and their V bytes (never written, so
    // possibly NaN codes) cleared so that p = 0 meets a finite value
    const bool ragged = T + 16 > L;
    float s[4];
    float cmax = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float x = sacc[i] * sm;
      s[i] = T + 4 * j + i < L ? x : -__builtin_inff();
      cmax = fmaxf(cmax, s[i]);
    }
    if (ragged) {
      const int nv = min(max(L - T - 4 * j, 0), 4);
      const uint32_t mask = nv >= 4 ? 0xFFFFFFFFu : (1u << (8 * nv)) - 1u;
#pragma unroll
      for (int t = 0; t < VT; t++) R.vw[t] &= mask;
    }
    // a row's max can only pass m_run + slack where one of its lanes' own
    // maxima does, so the wave-wide test needs no cross-lane reduction; the
    // row max (over the row's 4 lanes) is formed only when some row moves
    if (__builtin_amdgcn_ballot_w64(cmax > m_run + kRescaleSlack) != 0) {
      cmax = max_xor16_xor32(cmax);
      const float m_new = cmax > m_run + kRescaleSlack ? cmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < VT; t++) oacc[t] *= alpha;
    }
    half4_t pop, pop_lo;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float e = __builtin_amdgcn_exp2f(s[i] - m_run);
      l_run += e;
      const _Float16 hi = (_Float16)e;
      if (DUP) {
        pop[i] = (_Float16)(e - lo_sel * (float)hi);
      } else {
        pop[i] = hi;
        pop_lo[i] = (_Float16)(e - (float)hi);
      }
    }
#pragma unroll
    for (int t = 0; t < VT; t++) {
      const half2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(R.vw[t], 1.0f, false);
      const half2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(R.vw[t], 1.0f, true);
      const half4_t a = {v0[0], v0[1], v1[0], v1[1]};
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pop, oacc[t], 0, 0, 0);
      if (!DUP) oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pop_lo, oacc[t], 0, 0, 0);
    }
  };

  constexpr int S1 = kWaves;
  if (cw0 < c1) {
    const int clast = cw0 + (c1 - 1 - cw0) / S1 * S1;
    const int dq = (32 * S1) / P, dr = (32 * S1) % P;
    Regs RA, RB;
    auto fc = walk.cursor_at(cw0);
    auto ref0 = walk.fetch(fc);
    walk.advance(fc, S1, clast, dq, dr);
    auto ref1 = walk.fetch(fc);
    walk.advance(fc, S1, clast, dq, dr);
    load(RA, ref0.pg.x, ref0.row0);
    for (int c = cw0; c <= clast; c += S1) {
      load(RB, ref0.pg.y, ref0.row1);
      __builtin_amdgcn_sched_barrier(0);
      compute(RA, 32 * c);
      __builtin_amdgcn_sched_barrier(0);
      const auto ref2 = walk.fetch(fc);
      walk.advance(fc, S1, clast, dq, dr);
      load(RA, ref1.pg.x, ref1.row0);  // the next chunk's first half (the last chunk again at the end)
      __builtin_amdgcn_sched_barrier(0);
      compute(RB, 32 * c + 16);
      __builtin_amdgcn_sched_barrier(0);
      ref0 = ref1;
      ref1 = ref2;
    }
  }

  // ---- partial results, as in the 4-bit kernel; O^T tile t row 4j + rr is
  // channel 16t + 4j + rr
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (DUP) {
#pragma unroll
    for (int t = 0; t < VT; t++) {
#pragma unroll
      for (int rr = 0; rr < 4; rr++) oacc[t][rr] = add_xor8(oacc[t][rr]);
    }
  }
  float* sm_o = smem;                    // [kWaves][G][D]: each wave's o
  float* sm_ml = smem + kWaves * G * D;  // [kWaves][G][2]
  if (n < G) {
    if (j == 0) {
      sm_ml[(wave * G + n) * 2] = m_run;
      sm_ml[(wave * G + n) * 2 + 1] = l_run;
    }
    float* dst = sm_o + (wave * G + n) * D + 4 * j;
#pragma unroll
    for (int t = 0; t < VT; t++) *(float4*)(dst + 16 * t) = make_float4(oacc[t][0], oacc[t][1], oacc[t][2], oacc[t][3]);
  }
  finish_partial<D>(sm_o, sm_ml, G, p.gs[1], po, ml);
}

// Merge the splits of one (sequence, query head): M = max m_s,
// o = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s, lse = (M + log2 sum) ln 2.
//
// Up to kMergePre splits: one wavefront per (sequence, query head, 64-channel
// block), lane = channel.  The partial o of every split are loaded together
// with the (m, l) pairs, so the merge costs one memory round trip; lane s
// holds the weight of split s (0 for an empty split, whose partial o is
// zero) and v_readlane broadcasts it.  Sums run over s = 0, 1, ... and over a
// fixed butterfly: the result is reproducible for a given split plan.
constexpr int kMergePre = 16;

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const DecodeParams p) {
  constexpr int NCB = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= (int64_t)p.batch * p.num_q_heads * NCB) return;  // whole wavefronts
  const int cb = (int)(unit % NCB);
  const int64_t bh = unit / NCB;
  const int h = (int)(bh % p.num_q_heads), b = (int)(bh / p.num_q_heads);
  const int G = p.group, g = h / G, n = h - g * G, S = p.num_splits;  // S <= kMergePre
  const int64_t part0 = ((int64_t)b * p.num_kv_heads + g) * S;
  const float* mlp = p.part_ml + (part0 * G + n) * 2;                // split s at mlp[s * 2G]
  const float* op = p.part_o + (part0 * G + n) * D + cb * 64 + lane;  // split s at op[s * G * D]
  const int64_t os = (int64_t)G * D, ms = 2 * G;

  float ov[kMergePre];
#pragma unroll
  for (int i = 0; i < kMergePre; i++) ov[i] = i < S ? op[i * os] : 0.0f;
  const float m0 = lane < S ? mlp[lane * ms] : -__builtin_inff();
  const float l0 = lane < S ? mlp[lane * ms + 1] : 0.0f;
  float M = m0;
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) M = fmaxf(M, __shfl_xor(M, k, 64));
  const float w = m0 == -__builtin_inff() ? 0.0f : exp2f(m0 - M);
  float den = w * l0, o = 0.0f;
#pragma unroll
  for (int i = 0; i < kMergePre; i++)
    if (i < S) o += as_f32(__builtin_amdgcn_readlane(as_u32(w), i)) * ov[i];
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) den += __shfl_xor(den, k, 64);
  o = den > 0.0f ? o / den : 0.0f;
  const int64_t oi = ((int64_t)b * p.num_q_heads + h) * D + cb * 64 + lane;
  if (p.out_bf16)
    ((uint16_t*)p.out)[oi] = (uint16_t)bf16x2_rne((float2_t){o, 0.0f});
  else
    ((float*)p.out)[oi] = o;
  if (p.lse != nullptr && cb == 0 && lane == 0)
    p.lse[(int64_t)b * p.num_q_heads + h] = den > 0.0f ? (M + log2f(den)) * kLn2 : -__builtin_inff();
}

// Merge for more than kMergePre splits: one workgroup per (sequence, query
// head, 64-channel block).  Its 256 threads
// scan the (m, l) pairs together and stage the split weights 2^(m_s - M) in
// LDS (0 for an empty split, whose partial o is zero); then 4 groups of 64
// threads accumulate interleaved splits for their channel, branch-free, and
// are summed in LDS.  Every sum runs in a fixed order: reproducible.
template <int D>
__global__ __launch_bounds__(256) void merge_wide_kernel(const DecodeParams p) {
  constexpr int CW = 64, SG = 4, NCB = D / CW, WTILE = 4096;
  const int cb = blockIdx.x % NCB, h = blockIdx.x / NCB, b = blockIdx.y;
  const int tid = threadIdx.x, sg = tid / CW, cl = tid % CW, c = cb * CW + cl;
  const int G = p.group, g = h / G, n = h % G, S = p.num_splits;
  const int64_t part0 = ((int64_t)b * p.num_kv_heads + g) * S;
  const float* mlp = p.part_ml + (part0 * G + n) * 2;  // split s at mlp[s * 2G]
  const float* op = p.part_o + (part0 * G + n) * D + c;  // split s at op[s * G * D]
  __shared__ float red[256];
  __shared__ float wts[WTILE];
  __shared__ float acc_s[SG][CW];

  float m = -__builtin_inff();
  for (int s = tid; s < S; s += 256) m = fmaxf(m, mlp[(int64_t)s * 2 * G]);
  red[tid] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();

  float den = 0.0f, o = 0.0f;
  for (int s0 = 0; s0 < S; s0 += WTILE) {
    const int ns = min(WTILE, S - s0);
    for (int s = tid; s < ns; s += 256) {
      const float ms = mlp[(int64_t)(s0 + s) * 2 * G];
      const float w = ms == -__builtin_inff() ? 0.0f : exp2f(ms - M);
      wts[s] = w;
      den += w * mlp[(int64_t)(s0 + s) * 2 * G + 1];
    }
    __syncthreads();
#pragma unroll 8
    for (int s = sg; s < ns; s += SG) o += wts[s] * op[(int64_t)(s0 + s) * G * D];
    __syncthreads();
  }
  red[tid] = den;
  acc_s[sg][cl] = o;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  den = red[0];
  if (sg != 0) return;
  o = acc_s[0][cl] + acc_s[1][cl] + acc_s[2][cl] + acc_s[3][cl];
  o = den > 0.0f ? o / den : 0.0f;
  const int64_t oi = ((int64_t)b * p.num_q_heads + h) * D + c;
  if (p.out_bf16)
    ((uint16_t*)p.out)[oi] = (uint16_t)bf16x2_rne((float2_t){o, 0.0f});
  else
    ((float*)p.out)[oi] = o;
  if (p.lse != nullptr && cb == 0 && cl == 0)
    p.lse[(int64_t)b * p.num_q_heads + h] = den > 0.0f ? (M + log2f(den)) * kLn2 : -__builtin_inff();
}

// ---------------------------------------------------------------- static scratch
// The split partials of kvq_decode_attention_noalloc live in this array (one
// copy per device, held until the process ends) instead of a caller
// workspace.  Host code never passes the array's name to a kernel -- on the
// host it is only a stand-in for the symbol -- but the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept.  Calls that overlap on one device share the array and
// race; no part of it needs to start at zero (an empty split writes zeros).
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kScratchMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// LDS of a decode workgroup: each wave's [G][D] o and its G (m, l) pairs.
static size_t decode_lds_bytes(int G, int head_dim) { return (size_t)kWaves * G * (head_dim + 2) * sizeof(float); }

// Above 64 KiB (16 query heads per KV head at head dim 256) the kernels need
// the larger dynamic-LDS limit: set once per device for every instantiation.
static hipError_t decode_lds_limit() {
  static std::once_flag once[kScratchMaxDevices];
  static hipError_t result[kScratchMaxDevices];
  const int bytes = (int)decode_lds_bytes(16, 256);
  const void* kernels[] = {
      (const void*)decode_kernel<256, FMT_NVFP4, true>, (const void*)decode_kernel<256, FMT_NVFP4, false>,
      (const void*)decode_kernel<256, FMT_INT4, true>,  (const void*)decode_kernel<256, FMT_INT4, false>,
      (const void*)decode_kernel<256, FMT_K8V4, true>,  (const void*)decode_kernel<256, FMT_K8V4, false>,
      (const void*)decode_kernel<128, FMT_NVFP4, true>, (const void*)decode_kernel<128, FMT_NVFP4, false>,
      (const void*)decode_kernel<128, FMT_INT4, true>,  (const void*)decode_kernel<128, FMT_INT4, false>,
      (const void*)decode_kernel<128, FMT_K8V4, true>,  (const void*)decode_kernel<128, FMT_K8V4, false>,
      (const void*)decode_fp8_kernel<256, true>,        (const void*)decode_fp8_kernel<256, false>,
      (const void*)decode_fp8_kernel<128, true>,        (const void*)decode_fp8_kernel<128, false>};
  auto set_all = [&]() {
    for (const void* k : kernels) {
      const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  };
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchMaxDevices) {
    (void)hipGetLastError();
    return set_all();
  }
  std::call_once(once[dev], [&] { result[dev] = set_all(); });
  return result[dev];
}

hipError_t launch_decode(const DecodeParams& p, int fmt, int head_dim, hipStream_t stream) {
  const dim3 grid(p.num_splits, p.num_kv_heads, p.batch), block(64 * kWaves);
  const size_t lds = decode_lds_bytes(p.group, head_dim);
  if (lds > 65536) {
    const hipError_t e = decode_lds_limit();
    if (e != hipSuccess) return e;
  }
  const int64_t munits = (int64_t)p.batch * p.num_q_heads * (head_dim / 64);
  const bool narrow = p.num_splits <= kMergePre;
  const dim3 mgrid = narrow ? dim3((unsigned)((munits + 3) / 4)) : dim3(p.num_q_heads * (head_dim / 64), p.batch);
  const bool dup = p.group <= 8;
#define KVQ_DECODE(D, F)                                                                        \
  do {                                                                                          \
    if (dup) hipLaunchKernelGGL((decode_kernel<D, F, true>), grid, block, lds, stream, p);      \
    else hipLaunchKernelGGL((decode_kernel<D, F, false>), grid, block, lds, stream, p);         \
  } while (0)
  if (fmt == FMT_FP8) {
    if (head_dim == 256) {
      if (dup) hipLaunchKernelGGL((decode_fp8_kernel<256, true>), grid, block, lds, stream, p);
      else hipLaunchKernelGGL((decode_fp8_kernel<256, false>), grid, block, lds, stream, p);
    } else {
      if (dup) hipLaunchKernelGGL((decode_fp8_kernel<128, true>), grid, block, lds, stream, p);
      else hipLaunchKernelGGL((decode_fp8_kernel<128, false>), grid, block, lds, stream, p);
    }
  } else if (head_dim == 256) {
    if (fmt == FMT_NVFP4) KVQ_DECODE(256, FMT_NVFP4);
    else if (fmt == FMT_K8V4) KVQ_DECODE(256, FMT_K8V4);
    else KVQ_DECODE(256, FMT_INT4);
  } else {
    if (fmt == FMT_NVFP4) KVQ_DECODE(128, FMT_NVFP4);
    else if (fmt == FMT_K8V4) KVQ_DECODE(128, FMT_K8V4);
    else KVQ_DECODE(128, FMT_INT4);
  }
  if (head_dim == 256) {
    if (narrow) hipLaunchKernelGGL((merge_kernel<256>), mgrid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((merge_wide_kernel<256>), mgrid, dim3(256), 0, stream, p);
  } else {
    if (narrow) hipLaunchKernelGGL((merge_kernel<128>), mgrid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((merge_wide_kernel<128>), mgrid, dim3(256), 0, stream, p);
  }
#undef KVQ_DECODE
  return hipGetLastError();
}

}  // namespace kvq
