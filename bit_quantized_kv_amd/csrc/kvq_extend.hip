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
  static constexpr int BUF = KB + D * VPD * 4;
  static constexpr int TOTAL = 2 * BUF;
};

template <int D>
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
  u32x4_t kreg[KV16], va[CPT / 8], vb[CPT / 8];
  auto gload = [&](int step) {
    const int64_t t0 = (int64_t)step * kExtStep;
    const int64_t tk = t0 + krow;
    const uint16_t* kp = p.k + tk * p.kv_stride + (int64_t)g * D + kseg * (D / 8);
#pragma unroll
    for (int v = 0; v < KV16; v++) kreg[v] = tk < Lk ? ld_global<u32x4_t>(kp + 8 * v) : (u32x4_t){0u, 0u, 0u, 0u};
    const int64_t ta = t0 + 2 * vpair, tb = ta + 1;
    const uint16_t* pa = p.v + ta * p.kv_stride + (int64_t)g * D + vcb * CPT;
    const uint16_t* pb = pa + p.kv_stride;
#pragma unroll
    for (int v = 0; v < CPT / 8; v++) {
      va[v] = ta < Lk ? ld_global<u32x4_t>(pa + 8 * v) : (u32x4_t){0u, 0u, 0u, 0u};
      vb[v] = tb < Lk ? ld_global<u32x4_t>(pb + 8 * v) : (u32x4_t){0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* base = lds + buf * Lds::BUF;
#pragma unroll
    for (int v = 0; v < KV16; v++)
      *(u32x4_t*)(base + krow * Lds::KP + kseg * (D / 4) + 16 * v) = kreg[v];
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
    float s[8];
    float cmax = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int64_t kp = t0 + 16 * (e / 4) + 4 * j + (e % 4);
      const float x = sacc[e / 4][e % 4] * sm;
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
      const float p0 = __builtin_amdgcn_exp2f(s[e] - m_run), p1 = __builtin_amdgcn_exp2f(s[e + 1] - m_run);
      l_run += p0 + p1;
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

hipError_t launch_extend(const ExtendParams& p, int head_dim, hipStream_t stream) {
  const int64_t rows = (int64_t)p.chunk_len * p.group;
  const dim3 grid((unsigned)((rows + kExtRows - 1) / kExtRows), (unsigned)p.num_kv_heads), block(256);
  // the double-buffered staging (73 KB at head dim 256) is above HIP's default
  // 64 KB dynamic-LDS limit per workgroup; gfx950 has 160 KB per CU
  hipError_t e;
  if (head_dim == 256) {
    e = hipFuncSetAttribute((const void*)extend_kernel<256>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            ExtLds<256>::TOTAL);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((extend_kernel<256>), grid, block, ExtLds<256>::TOTAL, stream, p);
  } else {
    e = hipFuncSetAttribute((const void*)extend_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            ExtLds<128>::TOTAL);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((extend_kernel<128>), grid, block, ExtLds<128>::TOTAL, stream, p);
  }
  return hipGetLastError();
}

}  // namespace kvq
