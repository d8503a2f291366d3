// kvq_extend.hip -- extend (chunked-prefill) attention over the bf16 workspace.
//
// What it computes ("SGLang's 4-bit KV cache: the 56% is exact, the 1.78x is
// untested", Figure 2 caption: the chunked-prefill / extend path dequantizes
// the cached prefix into a reused workspace and attends over prefix plus
// current chunk): the workspace holds bf16 K and V rows for tokens
// [0, prefix_len + chunk_len) -- the prefix from kvq_dequant_prefix, then the
// chunk's own K/V -- and chunk query i (sequence position prefix_len + i)
// attends causally to keys 0 .. prefix_len + i.
//
// Structure: the (chunk token, query head) pairs of one KV head are flattened
// into query rows r = i * G + h; a workgroup of 4 wavefronts takes 64
// consecutive rows (16 per wavefront, the MFMA's column dimension) and walks
// the keys its rows can see in 32-token steps.  Each step's K rows and
// transposed V rows are staged once in LDS (double-buffered, the next step's
// global loads in flight in registers) and read by all 4 wavefronts:
//   QK  S^T[token][row] = K[token][ch] Q^T[ch][row] on v_mfma_f32_16x16x32_bf16
//       (bf16 K and q exactly, fp32 accumulation);
//   online softmax in base 2 per row, lazily rescaled as in decode;
//   PV  O^T[ch][row] += V^T[ch][token] P^T[token][row], P split into bf16
//       hi + lo parts (two MFMAs) so the product keeps ~16 bits of each p.
//
// Paged variant (SRC = the cache format): the same kernel reads the prefix
// straight from the 4-bit pages instead of a bf16 workspace -- the fused
// extend that needs no workspace -- and the chunk's own K/V from bf16 rows.
// Prefix codes are expanded to bf16 exactly while staged (NVFP4 e2m1 * e4m3;
// INT4 q) and the remaining factor of each token (NVFP4: the global scale;
// INT4: the token's scale; chunk tokens: 1) is staged per token and applied
// to its score (K) and to its probability in the PV product (V).
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kExtRows = 64;   // query rows per workgroup, 16 per wavefront
constexpr int kExtStep = 32;   // key tokens per step
static constexpr float kExtLog2e = 1.4426950408889634f;
static constexpr float kExtLn2 = 0.6931471805599453f;
static constexpr float kExtSlack = 8.0f;

// LDS strides chosen against bank conflicts (64 banks of 4 bytes): a K row
// is 4 banks off the previous one; a V^T row is 19 dwords long, so the
// 16-channel groups one wavefront writes (16 rows apart) start 48 banks apart
// (conflict-free writes) and an operand read spreads over the banks with at
// most 3 dwords per bank.
template <int D>
struct ExtLds {
  static constexpr int KP = 2 * D + 16;        // bytes per staged K row (token), padded
  static constexpr int VPD = kExtStep / 2 + 3; // dwords per staged V^T row (channel): 16 used + 3 pad
  static constexpr int KB = kExtStep * KP;
  static constexpr int VB = D * VPD * 4;
  static constexpr int BUF = KB + VB + 2 * kExtStep * 4;  // + per-token K and V factors
  static constexpr int TOTAL = 2 * BUF;
};

constexpr int kExtWorkspace = 0;  // SRC: every key from the bf16 workspace (else the cache format)

template <int D, int SRC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void extend_kernel(const ExtendParams p) {
  using Lds = ExtLds<D>;
  constexpr int KCH = D / 32, VT = D / 16;
  constexpr int KV16 = D / 64;       // 16-byte K vectors per thread and step
  constexpr int CPT = D / 16;        // V channels per thread and step (two tokens each)
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane >> 4, n = lane & 15;
  const int g = blockIdx.y;
  const int G = p.group;
  const int64_t nrows = (int64_t)p.chunk_len * G;
  const int64_t row0 = (int64_t)blockIdx.x * kExtRows;
  const int64_t Lk = (int64_t)p.prefix_len + p.chunk_len;

  // this lane's query row (column n of its wavefront's tile)
  const int64_t row = row0 + 16 * wave + n;
  const bool row_ok = row < nrows;
  const int irow = row_ok ? (int)(row / G) : p.chunk_len - 1;  // a padding row sees every key, q = 0
  const int h = g * G + (row_ok ? (int)(row % G) : 0);
  const int64_t lim = (int64_t)p.prefix_len + irow;            // last key the row sees

  // keys the workgroup needs: up to the last row's limit
  const int64_t last_row = min(row0 + kExtRows, nrows) - 1;
  const int64_t kmax = min(Lk - 1, (int64_t)p.prefix_len + last_row / G);
  const int nsteps = (int)(kmax / kExtStep) + 1;

  bf16x8_t qop[KCH];
  {
    const uint16_t* qrow = p.q + (int64_t)irow * p.q_stride + (int64_t)h * D + 8 * j;
#pragma unroll
    for (int m = 0; m < KCH; m++) {
      u32x4_t raw = ld_global<u32x4_t>(qrow + 32 * m);
      if (!row_ok) raw = (u32x4_t){0u, 0u, 0u, 0u};
      qop[m] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }
  const float sm = p.sm_scale * kExtLog2e;

  // ---- staging: thread t loads 16-byte vectors kseg*KV16 .. of K row krow, and
  // the V values of tokens 2(t%16), 2(t%16)+1, channels (t/16)*CPT ...  At head
  // dim 256 a quarter-wavefront covers 4 rows x 4 segments (distinct banks on
  // the LDS write, 256 contiguous bytes per row on the global read); at 128 it
  // covers 2 rows x 8 segments, already conflict-free.
  const int krow = D == 256 ? ((tid >> 2) & 3) + 4 * (tid >> 5) : tid >> 3;
  const int kseg = D == 256 ? (tid & 3) + 4 * ((tid >> 4) & 1) : tid & 7;
  const int vpair = tid & 15, vcb = tid >> 4;
  constexpr bool PAGED = SRC != kExtWorkspace;
  const int64_t Lp = p.prefix_len;
  // bf16 rows: the workspace holds every token; the paged variant's rows are the chunk's
  const int64_t row_base = PAGED ? Lp : 0;
  u32x4_t kreg[KV16], va[CPT / 8], vb[CPT / 8];
  // paged prefix tokens: raw codes and scale words, expanded in lstore
  u32x4_t kcode = {0u, 0u, 0u, 0u};
  uint32_t kscw = 0u, vcode_a[CPT / 8 * 2], vcode_b[CPT / 8 * 2], vscw_a = 0u, vscw_b = 0u;
  bool kpaged = false, vapaged = false, vbpaged = false;
  auto page_of = [&](int64_t t, int& off) -> const uint8_t* {
    const int64_t pi = t / p.page_size;
    off = (int)(t - pi * p.page_size);
    return p.pool + ((int64_t)p.pages[pi] * p.num_kv_heads + g) * p.slab;
  };
  auto gload = [&](int step) {
    const int64_t t0 = (int64_t)step * kExtStep;
    const int64_t tk = t0 + krow;
    kpaged = PAGED && tk < Lp;
    if (kpaged) {
      int off;
      const uint8_t* sl = page_of(tk, off);
      // elements kseg * D/8 .. : D/16 code bytes and D/128 scale bytes (NVFP4) or the row scale (INT4)
      if (D == 256) kcode = ld_global<u32x4_t>(sl + (int64_t)off * (D / 2) + kseg * (D / 16));
      else kcode.xy = ld_global<u32x2_t>(sl + (int64_t)off * (D / 2) + kseg * (D / 16));
      if (SRC == FMT_NVFP4)
        kscw = D == 256 ? ld_global<uint16_t>(sl + p.scales_off + (int64_t)off * (D / 16) + 2 * kseg)
                        : ld_global<uint8_t>(sl + p.scales_off + (int64_t)off * (D / 16) + kseg);
      else
        kscw = ld_global<uint32_t>(sl + p.scales_off + (int64_t)off * 4);
    } else {
      const uint16_t* kp = p.k + (tk - row_base) * p.kv_stride + (int64_t)g * D + kseg * (D / 8);
#pragma unroll
      for (int v = 0; v < KV16; v++)
        kreg[v] = tk < Lk ? ld_global<u32x4_t>(kp + 8 * v) : (u32x4_t){0u, 0u, 0u, 0u};
    }
    const int64_t ta = t0 + 2 * vpair, tb = ta + 1;
    vapaged = PAGED && ta < Lp;
    vbpaged = PAGED && tb < Lp;
#pragma unroll
    for (int half = 0; half < 2; half++) {
      const int64_t tv = half ? tb : ta;
      const bool pg = half ? vbpaged : vapaged;
      if (pg) {
        int off;
        const uint8_t* sl = page_of(tv, off) + p.half;
        // CPT channels from vcb * CPT: CPT/2 code bytes, one NVFP4 block scale (CPT == 16) or the row scale
        const uint8_t* cp = sl + (int64_t)off * (D / 2) + vcb * (CPT / 2);
        uint32_t* vc = half ? vcode_b : vcode_a;
        if (CPT == 16) {
          const u32x2_t w = ld_global<u32x2_t>(cp);
          vc[0] = w.x;
          vc[1] = w.y;
        } else {
          vc[0] = ld_global<uint32_t>(cp);
        }
        uint32_t sw;
        if (SRC == FMT_NVFP4)
          sw = ld_global<uint8_t>(sl + p.scales_off + (int64_t)off * (D / 16) + vcb * CPT / 16);
        else
          sw = ld_global<uint32_t>(sl + p.scales_off + (int64_t)off * 4);
        if (half) vscw_b = sw;
        else vscw_a = sw;
      } else {
        const uint16_t* pv = p.v + (tv - row_base) * p.kv_stride + (int64_t)g * D + vcb * CPT;
#pragma unroll
        for (int v = 0; v < CPT / 8; v++) {
          const u32x4_t x = tv < Lk ? ld_global<u32x4_t>(pv + 8 * v) : (u32x4_t){0u, 0u, 0u, 0u};
          if (half) vb[v] = x;
          else va[v] = x;
        }
      }
    }
  };
  // bf16 pairs of 8 codes (element 0 low): NVFP4 e2m1 * block scale, exact;
  // INT4 the integers q, exact
  auto expand8 = [&](uint32_t w, float s, uint32_t out[4]) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float2_t x;
      if (SRC == FMT_NVFP4) {
        switch (e) {
          case 0: x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
          case 1: x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
          case 2: x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
          default: x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
        }
        x[0] *= s;
        x[1] *= s;
      } else {
        x[0] = (float)((int)(w << (28 - 8 * e)) >> 28);
        x[1] = (float)((int)(w << (24 - 8 * e)) >> 28);
      }
      out[e] = bf16x2_rne(x);
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* base = lds + buf * Lds::BUF;
    float* kfac = (float*)(base + Lds::KB + Lds::VB);
    float* vfac = kfac + kExtStep;
    if (PAGED && kpaged) {
      // D/8 elements = KV16 16-byte bf16 vectors from D/32 code dwords
      const uint32_t cw[4] = {kcode.x, kcode.y, kcode.z, kcode.w};
#pragma unroll
      for (int v = 0; v < KV16; v++) {
        uint32_t o[4];
        const float s = SRC == FMT_NVFP4 ? e4m3_decode((kscw >> (8 * (v / 2))) & 0xFFu) : 1.0f;
        expand8(cw[v], s, o);
        kreg[v] = (u32x4_t){o[0], o[1], o[2], o[3]};
      }
    }
    if (PAGED && kseg == 0) kfac[krow] = kpaged ? (SRC == FMT_NVFP4 ? p.gs[0] : as_f32(kscw)) : 1.0f;
#pragma unroll
    for (int v = 0; v < KV16; v++)
      *(u32x4_t*)(base + krow * Lds::KP + kseg * (D / 4) + 16 * v) = kreg[v];
    if (PAGED) {
#pragma unroll
      for (int half = 0; half < 2; half++) {
        const bool pg = half ? vbpaged : vapaged;
        if (!pg) continue;
        const uint32_t* vc = half ? vcode_b : vcode_a;
        const uint32_t sw = half ? vscw_b : vscw_a;
        const float s = SRC == FMT_NVFP4 ? e4m3_decode(sw & 0xFFu) : 1.0f;
#pragma unroll
        for (int v = 0; v < CPT / 8; v++) {
          uint32_t o[4];
          expand8(vc[v], s, o);
          if (half) vb[v] = (u32x4_t){o[0], o[1], o[2], o[3]};
          else va[v] = (u32x4_t){o[0], o[1], o[2], o[3]};
        }
      }
      if (vcb == 0) {
        vfac[2 * vpair] = vapaged ? (SRC == FMT_NVFP4 ? p.gs[1] : as_f32(vscw_a)) : 1.0f;
        vfac[2 * vpair + 1] = vbpaged ? (SRC == FMT_NVFP4 ? p.gs[1] : as_f32(vscw_b)) : 1.0f;
      }
    }
    uint32_t* vt = (uint32_t*)(base + Lds::KB);
#pragma unroll
    for (int v = 0; v < CPT / 8; v++) {
      const uint32_t a4[4] = {va[v].x, va[v].y, va[v].z, va[v].w};
      const uint32_t b4[4] = {vb[v].x, vb[v].y, vb[v].z, vb[v].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int c = vcb * CPT + 8 * v + 2 * e;
        // (token a, token b) of channel c, then of channel c + 1
        vt[c * Lds::VPD + vpair] = byte_perm(b4[e], a4[e], 0x05040100u);
        vt[(c + 1) * Lds::VPD + vpair] = byte_perm(b4[e], a4[e], 0x07060302u);
      }
    }
  };

  float4_t oacc[VT];
#pragma unroll
  for (int t = 0; t < VT; t++) oacc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -__builtin_inff(), l_run = 0.0f;

  auto compute = [&](int buf, int64_t t0) {
    const uint8_t* kb = lds + buf * Lds::BUF;
    const uint32_t* vt = (const uint32_t*)(kb + Lds::KB);
    float4_t sacc[2];
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
      sacc[hh] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
      const uint8_t* krow_p = kb + (16 * hh + n) * Lds::KP + 16 * j;
#pragma unroll
      for (int m = 0; m < KCH; m++) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(krow_p + 64 * m));
        sacc[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[m], sacc[hh], 0, 0, 0);
      }
    }
    float s[8], vf[8];
    const float* kfac = (const float*)(kb + Lds::KB + Lds::VB);
    const float* vfac = kfac + kExtStep;
    float cmax = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int tok = 16 * (e / 4) + 4 * j + (e % 4);
      const int64_t kp = t0 + tok;
      float x = sacc[e / 4][e % 4] * sm;
      if (PAGED) {
        x *= kfac[tok];
        vf[e] = vfac[tok];
      }
      s[e] = kp <= lim ? x : -__builtin_inff();
      cmax = fmaxf(cmax, s[e]);
    }
    cmax = max_xor16_xor32(cmax);
    if (__builtin_amdgcn_ballot_w64(cmax > m_run + kExtSlack) != 0) {
      const float m_new = cmax > m_run + kExtSlack ? cmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < VT; t++) oacc[t] *= alpha;
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float p0 = __builtin_amdgcn_exp2f(s[e] - m_run), p1 = __builtin_amdgcn_exp2f(s[e + 1] - m_run);
      l_run += p0 + p1;
      if (PAGED) {  // the value factor of each token rides on its probability
        p0 *= vf[e];
        p1 *= vf[e + 1];
      }
      const uint32_t hw = bf16x2_rne((float2_t){p0, p1});
      const float h0 = as_f32(hw << 16), h1 = as_f32(hw & 0xFFFF0000u);
      hi[e / 2] = hw;
      lo[e / 2] = bf16x2_rne((float2_t){p0 - h0, p1 - h1});
    }
    const bf16x8_t phi = __builtin_bit_cast(bf16x8_t, (u32x4_t){hi[0], hi[1], hi[2], hi[3]});
    const bf16x8_t plo = __builtin_bit_cast(bf16x8_t, (u32x4_t){lo[0], lo[1], lo[2], lo[3]});
#pragma unroll
    for (int t = 0; t < VT; t++) {
      // channel 16t + n, tokens 4j..4j+3 and 16+4j..16+4j+3 (the order of P's k index)
      const uint32_t* vr = vt + (16 * t + n) * Lds::VPD + 2 * j;  // 4-byte aligned rows: dword reads
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, (u32x4_t){vr[0], vr[1], vr[8], vr[9]});
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi, oacc[t], 0, 0, 0);
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo, oacc[t], 0, 0, 0);
    }
  };

  gload(0);
  lstore(0);
  if (nsteps > 1) gload(1);
  __syncthreads();
  for (int st = 0; st < nsteps; st++) {
    compute(st & 1, (int64_t)st * kExtStep);
    if (st + 1 < nsteps) {
      lstore((st + 1) & 1);
      if (st + 2 < nsteps) gload(st + 2);
    }
    __syncthreads();
  }

  // ---- epilogue: each lane column is one query row
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!row_ok) return;
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  const int64_t obase = (int64_t)irow * p.out_stride + (int64_t)h * D + 4 * j;
#pragma unroll
  for (int t = 0; t < VT; t++) {
    const float o0 = oacc[t][0] * inv, o1 = oacc[t][1] * inv, o2 = oacc[t][2] * inv, o3 = oacc[t][3] * inv;
    if (p.out_bf16) {
      *(u32x2_t*)((uint16_t*)p.out + obase + 16 * t) =
          (u32x2_t){bf16x2_rne((float2_t){o0, o1}), bf16x2_rne((float2_t){o2, o3})};
    } else {
      *(float4*)((float*)p.out + obase + 16 * t) = make_float4(o0, o1, o2, o3);
    }
  }
  if (p.lse != nullptr && j == 0)
    p.lse[(int64_t)irow * p.lse_stride + h] = l_run > 0.0f ? (m_run + log2f(l_run)) * kExtLn2 : -__builtin_inff();
}

template <int D, int SRC>
static hipError_t launch_extend_t(const ExtendParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.chunk_len * p.group;
  const dim3 grid((unsigned)((rows + kExtRows - 1) / kExtRows), (unsigned)p.num_kv_heads), block(256);
  // the double-buffered staging (74 KB at head dim 256) is above HIP's default
  // 64 KB dynamic-LDS limit per workgroup; gfx950 has 160 KB per CU
  const hipError_t e = hipFuncSetAttribute((const void*)extend_kernel<D, SRC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, ExtLds<D>::TOTAL);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((extend_kernel<D, SRC>), grid, block, ExtLds<D>::TOTAL, stream, p);
  return hipGetLastError();
}

hipError_t launch_extend(const ExtendParams& p, int head_dim, int src_fmt, hipStream_t stream) {
  if (head_dim == 256) {
    if (src_fmt == FMT_NVFP4) return launch_extend_t<256, FMT_NVFP4>(p, stream);
    if (src_fmt == FMT_INT4) return launch_extend_t<256, FMT_INT4>(p, stream);
    return launch_extend_t<256, kExtWorkspace>(p, stream);
  }
  if (src_fmt == FMT_NVFP4) return launch_extend_t<128, FMT_NVFP4>(p, stream);
  if (src_fmt == FMT_INT4) return launch_extend_t<128, FMT_INT4>(p, stream);
  return launch_extend_t<128, kExtWorkspace>(p, stream);
}

}  // namespace kvq
