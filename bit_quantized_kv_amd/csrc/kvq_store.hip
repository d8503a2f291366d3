// kvq_store.hip -- quantize-on-write and prefix dequantization for gfx950.
//
// Quantize-on-write follows the write path of "SGLang's 4-bit KV cache: the
// 56% is exact, the 1.78x is untested" (Figure 2 caption: prefill and decode
// quantize K/V and store them into the shared pool) for NVFP4, and the INT4
// write path of "KV cache in 4 bits: 8.8 instead of 4.7 full sessions on the
// same four RTX 5090s" ("What we changed").  Prefix dequantization is the
// extend path of the same Figure 2 caption, with a bf16 workspace.
//
// Both kernels stream, one workgroup per run of consecutive tokens of one
// (K|V, head) pair, with 16/32-byte vector accesses on consecutive lanes.
// Every rounding decision is an IEEE fp32 operation (correctly rounded
// quotients, no FMA contraction) or a gfx950 conversion instruction with the
// same rounding, so the packed bytes and the dequantized bf16 are bit-exact
// against a scalar implementation of the same rules.
#pragma clang fp contract(off)

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

template <typename T>
struct Row16;

template <>
struct Row16<float> {
  __device__ static void load(const void* p, float x[16]) {
    const u32x4_t* v = (const u32x4_t*)p;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const u32x4_t a = ld_stream<u32x4_t>(v + i);  // rows are read once: non-temporal
      x[4 * i + 0] = as_f32(a.x);
      x[4 * i + 1] = as_f32(a.y);
      x[4 * i + 2] = as_f32(a.z);
      x[4 * i + 3] = as_f32(a.w);
    }
  }
};

template <>
struct Row16<uint16_t> {  // bf16 bit patterns, widened exactly
  __device__ static void load(const void* p, float x[16]) {
    const u32x4_t* v = (const u32x4_t*)p;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const u32x4_t a = ld_stream<u32x4_t>(v + i);
      uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        x[8 * i + 2 * j] = as_f32(w[j] << 16);
        x[8 * i + 2 * j + 1] = as_f32(w[j] & 0xFFFF0000u);
      }
    }
  }
};

// Orthogonal Hadamard rotation of one row held as 16 elements per lane by
// the D/16 consecutive lanes of the row (lane b holds elements 16b..16b+15):
// the fast transform's stages h = 1, 2, 4, 8 inside the lane, then h = 16,
// 32, ... across lanes (partner lane b ^ (h/16)); each stage maps the pair
// (x_i, x_{i+h}) to (x_i + x_{i+h}, x_i - x_{i+h}) in fp32, and the scale
// 1/sqrt(D) is applied last -- the same operations, on the same operands, as
// a scalar loop over the stages, so the rotated row is bit-reproducible.
template <int D>
__device__ inline void hadamard_row(float x[16], int b, float scale) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      if (i & h) continue;
      const float a = x[i], c = x[i + h];
      x[i] = a + c;
      x[i + h] = a - c;
    }
  }
#pragma unroll
  for (int m = 1; m < D / 16; m <<= 1) {
    const bool upper = (b & m) != 0;
#pragma unroll
    for (int e = 0; e < 16; e++) {
      const float partner = lane_xor16(x[e], m);
      x[e] = upper ? partner - x[e] : x[e] + partner;
    }
  }
#pragma unroll
  for (int e = 0; e < 16; e++) x[e] *= scale;
}

// A workgroup takes kStoreTokens(D) = 256 / (D/16) consecutive input tokens of
// one (K|V, head) pair, blockIdx.y = kv * num_kv_heads + head; thread (i, b)
// quantizes block b (16 head-dim elements) of token t0 + i.  No 64-bit
// division: the token comes from blockIdx.x, the pair from blockIdx.y.
template <int D>
__device__ inline int64_t store_token(int tid) {
  return (int64_t)blockIdx.x * (256 / (D / 16)) + tid / (D / 16);
}

// True when the FMA-corrected quotient below is the correctly rounded x / S
// for every x: S = e4m3 * gs has at most 4 significant bits when gs is a
// power of two (an exhaustive check over every fp32 significand against each
// of the 8 E4M3 significands finds no difference), and the bounded exponent
// range keeps the residual exact.
__device__ inline bool fma_quotient_exact(float gs) {
  const uint32_t u = as_u32(gs);
  return (u & 0x807FFFFFu) == 0u && (u >> 23) - 103u <= 48u;  // gs = 2^k, -24 <= k <= 24
}

// y = RN(x / S) from r = RN(1 / S): q = RN(x r) is within an ulp of x / S,
// the residual x - q S is exact in an FMA, and one correction step rounds
// correctly (Markstein's division step).  Written as q - (q S - x) r so that
// x = -0 keeps its sign.
__device__ inline float fma_quotient(float x, float S, float r) {
  const float q = x * r;
  const float e = __builtin_fmaf(q, S, -x);
  return __builtin_fmaf(-e, r, q);
}

// Eight ratios -> one dword of E2M1 codes (element 0 in the low nibble) with
// the gfx950 conversion v_cvt_scalef32_pk_fp4_f32 at scale 1: round to
// nearest, ties to the even code, saturation at 6, the sign kept (also for
// zeros and denormals).  Checked exhaustively against a scalar encoder of
// that rule over every non-NaN fp32 input.
__device__ inline uint32_t e2m1_pack8(const float* y) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
}

// NVFP4 of one 16-element block under the global scale gs: the E4M3 block
// scale code and the two words of E2M1 codes (element 0 in the low nibble).
__device__ inline void nvfp4_block(const float x[16], float gs, uint32_t& w0, uint32_t& w1, uint32_t& cs) {
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; e++) amax = fmaxf(amax, __builtin_fabsf(x[e]));
  const float den = 6.0f * gs;
  const float s_raw = amax / den;
  cs = e4m3_encode(s_raw);
  const float S = e4m3_decode(cs) * gs;

  float y[16];
  if (S != 0.0f && s_raw <= 448.0f && fma_quotient_exact(gs)) {
    const float r = 1.0f / S;
#pragma unroll
    for (int e = 0; e < 16; e++) y[e] = fma_quotient(x[e], S, r);
  } else {
    // general global scale, a saturated block scale, or S = 0 (codes 0 below)
#pragma unroll
    for (int e = 0; e < 16; e++) y[e] = x[e] / S;
  }
  w0 = e2m1_pack8(y);
  w1 = e2m1_pack8(y + 8);
  if (S == 0.0f) w0 = w1 = 0u;
}

// FP8 E4M3 of 16 values with a per-tensor scale s: code = E4M3(fp32(x / s))
// with the sign kept, saturating at 448; four words, element 0 in the low byte.
// The quotient is IEEE division; the code comes from gfx950's
// v_cvt_pk_fp8_f32 after a clamp to [-448, 448], which matches that rule for
// every fp32 input (round to nearest, ties to the even code, the sign kept;
// checked exhaustively), two codes per instruction.
__device__ inline void fp8_block(const float x[16], float s, uint32_t w[4]) {
  float y[16];
#pragma unroll
  for (int e = 0; e < 16; e++) y[e] = __builtin_amdgcn_fmed3f(x[e] / s, -448.0f, 448.0f);
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * k], y[4 * k + 1], 0, false);
    w[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * k + 2], y[4 * k + 3], lo, true);
  }
}

template <int D, typename TIn>
__global__ __launch_bounds__(256) void nvfp4_store_kernel(StoreParams p) {
  constexpr int NB = D / 16;
  const int kv = (int)blockIdx.y >= p.num_kv_heads ? 1 : 0;
  const int g = (int)blockIdx.y - kv * p.num_kv_heads;
  const int b = threadIdx.x % NB;
  const int64_t i = store_token<D>(threadIdx.x);
  if (i >= p.num_tokens) return;
  // the input row and the slot are loaded together; a skipped token (slot < 0)
  // is quantized and dropped
  float x[16];
  const TIn* src = (const TIn*)(kv ? p.v : p.k) + i * p.in_stride + (int64_t)g * D + 16 * b;
  Row16<TIn>::load(src, x);
  if (p.rotate) hadamard_row<D>(x, b, p.rot_scale);
  const int32_t slot = p.slots[i];
  uint32_t w0, w1, cs;
  nvfp4_block(x, p.gs[kv], w0, w1, cs);
  if (slot < 0) return;

  const int64_t page = slot / p.page_size;
  const int64_t off = slot % p.page_size;
  uint8_t* half = p.pool + (page * p.num_kv_heads + g) * p.slab + kv * p.half;
  *(uint2*)(half + off * (D / 2) + 8 * b) = make_uint2(w0, w1);
  half[p.scales_off + off * NB + b] = (uint8_t)cs;
}

// FP8 E4M3 with one FP32 scale per tensor (the comparator format): K rows
// are stored by token (D bytes), V by channel (the slab's V section holds D
// rows of page_size bytes).  code = E4M3(fp32(x / s)) with the sign kept,
// saturating at 448.  Thread (i, b) holds the 16 codes of elements 16b ..
// 16b + 15 of token i: a K row segment, one 16-byte store.  V: when the
// workgroup's tokens come in runs of 16 that fill 16 consecutive slots of
// one page from a multiple of 16 (chunked prefill into fresh pages), each
// run is a 16-byte-aligned 16-byte segment of every channel row; the codes
// go through LDS (token-major in, channel-major out) and each thread writes
// one channel's segment with a single 16-byte store.  Other workgroups
// (single tokens, skipped slots, unaligned runs) store V byte by byte.
template <int D, typename TIn>
__global__ __launch_bounds__(256) void fp8_store_kernel(StoreParams p) {
  constexpr int NB = D / 16, TOK = 256 / NB;  // tokens per workgroup: 16 (D 256) or 32 (D 128)
  __shared__ __attribute__((aligned(16))) uint8_t tile[TOK * D];
  const int kv = (int)blockIdx.y >= p.num_kv_heads ? 1 : 0;
  const int g = (int)blockIdx.y - kv * p.num_kv_heads;
  const int b = threadIdx.x % NB, il = threadIdx.x / NB;
  const int64_t i = store_token<D>(threadIdx.x);
  const bool valid = i < p.num_tokens;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  int32_t slot = -1;
  if (valid) {
    float x[16];
    Row16<TIn>::load((const TIn*)(kv ? p.v : p.k) + i * p.in_stride + (int64_t)g * D + 16 * b, x);
    if (p.rotate) hadamard_row<D>(x, b, p.rot_scale);
    slot = p.slots[i];
    fp8_block(x, p.gs[kv], w);
  }
  if (kv == 0) {
    if (slot < 0) return;
    const int64_t page = slot / p.page_size;
    const int off = slot % p.page_size;
    uint8_t* base = p.pool + (page * p.num_kv_heads + g) * p.slab;
    *(uint4*)(base + (int64_t)off * D + 16 * b) = make_uint4(w[0], w[1], w[2], w[3]);
    return;
  }
  // V (a workgroup-uniform branch): tile or scatter for the whole workgroup
  const int run0 = il & ~15;  // first token of this thread's run of 16, in the workgroup
  const int64_t i0 = (int64_t)blockIdx.x * TOK + run0;
  const int32_t first = i0 < p.num_tokens ? p.slots[i0] : -1;
  const bool in_run = valid && first >= 0 && (first & 15) == 0 && slot == first + (il - run0);
  const bool tiled = (p.page_size & 15) == 0 && __syncthreads_and(in_run);
  if (tiled) {
    *(uint4*)(tile + il * D + 16 * b) = make_uint4(w[0], w[1], w[2], w[3]);
    __syncthreads();
    // thread t writes channel c = t % D of run t / D (the workgroup's runs
    // are TOK / 16 = 256 / D, so every thread has one)
    const int c = threadIdx.x % D, run = threadIdx.x / D;
    const int32_t fs = p.slots[(int64_t)blockIdx.x * TOK + 16 * run];
    uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 16; k++) o[k / 4] |= (uint32_t)tile[(16 * run + k) * D + c] << (8 * (k % 4));
    const int64_t page = fs / p.page_size;
    const int off = fs % p.page_size;
    uint8_t* vrow = p.pool + (page * p.num_kv_heads + g) * p.slab + (int64_t)p.page_size * D +
                    (int64_t)c * p.page_size + off;
    *(uint4*)vrow = make_uint4(o[0], o[1], o[2], o[3]);
    return;
  }
  if (slot < 0) return;
  const int64_t page = slot / p.page_size;
  const int off = slot % p.page_size;
  uint8_t* col = p.pool + (page * p.num_kv_heads + g) * p.slab + (int64_t)p.page_size * D + (int64_t)(16 * b) * p.page_size + off;
#pragma unroll
  for (int e = 0; e < 16; e++) col[(int64_t)e * p.page_size] = (uint8_t)(w[e / 4] >> (8 * (e % 4)));
}

// FP8 keys with NVFP4 values: K rows as in the FP8 format (by token, D bytes,
// per-tensor scale gs[0]), V rows as in NVFP4 (global scale gs[1]) in the
// slab's V section.  The K|V choice is per workgroup (grid y).
template <int D, typename TIn>
__global__ __launch_bounds__(256) void k8v4_store_kernel(StoreParams p) {
  constexpr int NB = D / 16;
  const int kv = (int)blockIdx.y >= p.num_kv_heads ? 1 : 0;
  const int g = (int)blockIdx.y - kv * p.num_kv_heads;
  const int b = threadIdx.x % NB;
  const int64_t i = store_token<D>(threadIdx.x);
  if (i >= p.num_tokens) return;
  float x[16];
  Row16<TIn>::load((const TIn*)(kv ? p.v : p.k) + i * p.in_stride + (int64_t)g * D + 16 * b, x);
  if (p.rotate) hadamard_row<D>(x, b, p.rot_scale);
  const int32_t slot = p.slots[i];
  uint32_t w[4], cs = 0u;
  if (kv == 0) fp8_block(x, p.gs[0], w);
  else nvfp4_block(x, p.gs[1], w[0], w[1], cs);
  if (slot < 0) return;
  const int64_t page = slot / p.page_size;
  const int64_t off = slot % p.page_size;
  uint8_t* base = p.pool + (page * p.num_kv_heads + g) * p.slab;
  if (kv == 0) {
    *(uint4*)(base + off * D + 16 * b) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    uint8_t* vsec = base + p.half;
    *(uint2*)(vsec + off * (D / 2) + 8 * b) = make_uint2(w[0], w[1]);
    vsec[p.scales_off + off * NB + b] = (uint8_t)cs;
  }
}

// INT4 rounding of a quotient near a half-integer: rint(RN(x / s)) when
// x / s lies within 2^-19 + 2^-20 of the half-integer h, without a division.
// The residual d = x - h s is exact in one FMA (a multiple of 2^(e - 24) for
// s in [2^e, 2^(e+1)), below 2^(e - 17) in magnitude: at most 7 significant
// bits).  RN(x / s) = h exactly when |x / s - h| <= ulp(h) / 2 -- h = k + 1/2
// has a zero last significand bit, so a midpoint rounds to h -- i.e. when
// |d| <= s ulp(h) / 2, with the smaller ulp of the binade below on the side
// toward zero of a power-of-two |h| (0.5); rint(h) is then the even one of
// floor(h), ceil(h).  Otherwise RN(x / s) is on the side of h that d's sign
// gives.
__device__ inline float int4_near_half(float x, float s, float h) {
  const float d = __builtin_fmaf(-h, s, x);
  const float ah = __builtin_fabsf(h);
  const int e = __builtin_amdgcn_frexp_expf(ah) - 1;  // ah in [2^e, 2^(e+1))
  const bool toward_zero = (d < 0.0f) == (h > 0.0f);
  const bool pow2 = ah == __builtin_ldexpf(1.0f, e);
  const float half_ulp_s = __builtin_ldexpf(s, e - 24 - ((toward_zero && pow2) ? 1 : 0));
  const float lo = __builtin_floorf(h), hi = lo + 1.0f;
  if (__builtin_fabsf(d) <= half_ulp_s) return ((int)lo & 1) ? hi : lo;
  return d > 0.0f ? hi : lo;
}

// INT4: the D/16 threads of one row reduce the row amax with DPP lane
// exchanges; s = RN(amax / 7) and q = clamp(rint(RN(x / s)), -7, 7).  The
// quotient is taken as y = RN(x RN(1 / s)): both roundings are relative
// errors below 2^-24 and |x / s| <= 7 (1 + 2^-23), so |y - x/s| < 2^-20, and
// RN(x / s) is within 2^-21 of x / s: where y lies farther than 2^-19 from
// every half-integer, rint(y) = rint(RN(x / s)).  rint(y) comes from adding
// 1.5 * 2^23 (round to nearest even), whose low mantissa bits then hold the
// integer in two's complement -- the nibble itself.  An element closer to a
// half-integer (bf16 inputs make exact ratios such as x = amax / 2 common)
// is decided by int4_near_half; a row with s below 2^-100 takes IEEE
// division.
template <int D, typename TIn>
__global__ __launch_bounds__(256) void int4_store_kernel(StoreParams p) {
  constexpr int NB = D / 16;
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  const int kv = (int)blockIdx.y >= p.num_kv_heads ? 1 : 0;
  const int g = (int)blockIdx.y - kv * p.num_kv_heads;
  const int b = threadIdx.x % NB;
  const int64_t i = store_token<D>(threadIdx.x);
  if (i >= p.num_tokens) return;  // whole rows only: a row's NB lanes share i
  float x[16];
  const TIn* src = (const TIn*)(kv ? p.v : p.k) + i * p.in_stride + (int64_t)g * D + 16 * b;
  Row16<TIn>::load(src, x);
  if (p.rotate) hadamard_row<D>(x, b, p.rot_scale);
  const int32_t slot = p.slots[i];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; e++) amax = fmaxf(amax, __builtin_fabsf(x[e]));
#pragma unroll
  for (int m = 1; m < NB; m <<= 1) amax = fmaxf(amax, lane_xor16(amax, m));
  const float s = amax / 7.0f;
  uint32_t w0 = 0, w1 = 0;
  if (s != 0.0f) {
    uint32_t nib[16];
    if (s >= 0x1p-100f) {
      const float r = 1.0f / s;
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const float y = x[e] * r;
        const float t = y + kMagic;
        const float n = t - kMagic;
        nib[e] = as_u32(t);
        if (__builtin_fabsf(y - n) >= 0.5f - 0x1p-19f) {
          const float q = int4_near_half(x[e], s, n + (y > n ? 0.5f : -0.5f));
          nib[e] = as_u32(__builtin_amdgcn_fmed3f(q, -7.0f, 7.0f) + kMagic);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; e++)
        nib[e] = as_u32(__builtin_amdgcn_fmed3f(__builtin_rintf(x[e] / s), -7.0f, 7.0f) + kMagic);
    }
#pragma unroll
    for (int e = 0; e < 8; e++) {
      w0 |= (nib[e] & 0xFu) << (4 * e);
      w1 |= (nib[e + 8] & 0xFu) << (4 * e);
    }
  }
  if (slot < 0) return;
  const int64_t page = slot / p.page_size;
  const int64_t off = slot % p.page_size;
  uint8_t* half = p.pool + (page * p.num_kv_heads + g) * p.slab + kv * p.half;
  *(uint2*)(half + off * (D / 2) + 8 * b) = make_uint2(w0, w1);
  if (b == 0) *(float*)(half + p.scales_off + off * 4) = s;
}

// Global-scale calibration: the running absolute maximum of a layer's K and
// V over prefill rows.  Grid (up to kAmaxWorkgroups, K|V): the workgroups walk
// the (token, head) rows grid-stride, four row runs at a time with their loads
// in flight together; a workgroup adds its maximum with one atomic max on the
// fp32 bit pattern of running[kv] (which orders like the value for
// non-negative numbers), and only when it exceeds the value it reads there,
// so that few of the atomics -- which serialize on one address -- happen.
constexpr int kAmaxWorkgroups = 1024;

template <int D, typename TIn>
__global__ __launch_bounds__(256) void amax_kernel(StoreParams p, float* running) {
  constexpr int NB = D / 16, RPW = 256 / NB;
  const int kv = blockIdx.y;
  const int b = threadIdx.x % NB;
  const int64_t rows = (int64_t)p.num_tokens * p.num_kv_heads;
  const int64_t stride = (int64_t)gridDim.x * RPW;
  const TIn* src = (const TIn*)(kv ? p.v : p.k) + 16 * b;
  float amax = 0.0f;
  // a run past the end re-reads the last row, which leaves a maximum unchanged
  for (int64_t r0 = (int64_t)blockIdx.x * RPW + threadIdx.x / NB; r0 < rows; r0 += 4 * stride) {
    float x[4][16];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int64_t r = min(r0 + u * stride, rows - 1);
      const int64_t i = r / p.num_kv_heads;
      const int g = (int)(r - i * p.num_kv_heads);
      Row16<TIn>::load(src + i * p.in_stride + (int64_t)g * D, x[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      if (p.rotate) hadamard_row<D>(x[u], b, p.rot_scale);  // a rotated cache stores rotated rows
#pragma unroll
      for (int e = 0; e < 16; e++) amax = fmaxf(amax, __builtin_fabsf(x[u][e]));
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    // the running maximum only grows, so a workgroup whose maximum does not
    // exceed a (possibly stale) read of it has nothing to add
    if (m > __builtin_nontemporal_load(running + kv)) atomicMax((unsigned int*)(running + kv), as_u32(m));
  }
}

// gs = fp32(amax / (6 * 448)) for K and V (1 for an all-zero tensor), so the
// largest block scale of the calibrated data is E4M3's largest value.
__global__ void global_scale_kernel(const float* running, float* gs) {
  const int i = threadIdx.x;
  if (i < 2) gs[i] = running[i] > 0.0f ? running[i] / 2688.0f : 1.0f;
}

hipError_t launch_calibrate_amax(const StoreParams& p, int head_dim, int in_bf16, float* running,
                                 hipStream_t stream) {
  const int rpw = 256 / (head_dim / 16);
  const int64_t runs = ((int64_t)p.num_tokens * p.num_kv_heads + rpw - 1) / rpw;
  const dim3 grid((unsigned)(runs < kAmaxWorkgroups ? runs : kAmaxWorkgroups), 2u), block(256);
  if (head_dim == 256) {
    if (in_bf16) hipLaunchKernelGGL((amax_kernel<256, uint16_t>), grid, block, 0, stream, p, running);
    else hipLaunchKernelGGL((amax_kernel<256, float>), grid, block, 0, stream, p, running);
  } else {
    if (in_bf16) hipLaunchKernelGGL((amax_kernel<128, uint16_t>), grid, block, 0, stream, p, running);
    else hipLaunchKernelGGL((amax_kernel<128, float>), grid, block, 0, stream, p, running);
  }
  return hipGetLastError();
}

hipError_t launch_global_scale(const float* running, float* gs, hipStream_t stream) {
  hipLaunchKernelGGL(global_scale_kernel, dim3(1), dim3(64), 0, stream, running, gs);
  return hipGetLastError();
}

// Standalone rotation of rows (queries before decode over a rotated cache,
// and the decode output back): thread per 16-element block, rows of D/16
// consecutive lanes.
template <int D, typename TIn, bool OUT_BF16>
__global__ __launch_bounds__(256) void hadamard_kernel(RotateParams p) {
  constexpr int NB = D / 16;
  const int b = threadIdx.x % NB;
  const int64_t row = (int64_t)blockIdx.x * (256 / NB) + threadIdx.x / NB;
  if (row >= p.rows) return;  // whole rows
  float x[16];
  Row16<TIn>::load((const TIn*)p.in + row * p.in_stride + 16 * b, x);
  hadamard_row<D>(x, b, p.scale);
  if (OUT_BF16) {
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; e++) w[e] = bf16x2_rne((float2_t){x[2 * e], x[2 * e + 1]});
    uint4* dst = (uint4*)((uint16_t*)p.out + row * p.out_stride + 16 * b);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    float4* dst = (float4*)((float*)p.out + row * p.out_stride + 16 * b);
#pragma unroll
    for (int e = 0; e < 4; e++) dst[e] = make_float4(x[4 * e], x[4 * e + 1], x[4 * e + 2], x[4 * e + 3]);
  }
}

hipError_t launch_hadamard(const RotateParams& p, int head_dim, int in_bf16, int out_bf16, hipStream_t stream) {
  const int rpw = 256 / (head_dim / 16);
  const dim3 grid((unsigned)((p.rows + rpw - 1) / rpw)), block(256);
#define KVQ_ROT(D)                                                                                         \
  do {                                                                                                     \
    if (in_bf16 && out_bf16) hipLaunchKernelGGL((hadamard_kernel<D, uint16_t, true>), grid, block, 0, stream, p); \
    else if (in_bf16) hipLaunchKernelGGL((hadamard_kernel<D, uint16_t, false>), grid, block, 0, stream, p);     \
    else if (out_bf16) hipLaunchKernelGGL((hadamard_kernel<D, float, true>), grid, block, 0, stream, p);        \
    else hipLaunchKernelGGL((hadamard_kernel<D, float, false>), grid, block, 0, stream, p);                     \
  } while (0)
  if (head_dim == 256) KVQ_ROT(256);
  else KVQ_ROT(128);
#undef KVQ_ROT
  return hipGetLastError();
}

// Prefix dequantization.  A workgroup expands kDequantTokens = 64 consecutive
// tokens (four 16-token groups, each inside one page since the page size is a
// multiple of 16) of one (K|V, head) pair, blockIdx.y = kv * num_kv_heads +
// head.  Thread (row r, column c) expands code dword c (elements 8c..8c+7)
// of rows r, r + RPP, ... and writes 16 bytes of bf16 per row, so a row of
// D elements is one contiguous 2D-byte store across D/8 lanes.
//   NVFP4: bf16_rne(fp32(fp32(e2m1 * e4m3) * gs)): the E2M1 values come from
//   v_cvt_scalef32_pk_f32_fp4 (exact), the product with the E4M3 scale is
//   exact, the gs product rounds once, v_cvt_pk_bf16_f32 rounds to nearest
//   even.  INT4: bf16_rne(fp32(q * s)).
constexpr int kDequantTokens = 64;

template <int D, int FMT, bool TAIL>
__device__ inline void dequant_rows(const DequantParams& p, int kv, int g, int t0) {
  constexpr int CPR = D / 8;               // code dwords per row
  constexpr int RPP = 256 / CPR;           // rows per pass: 8 (D 256) or 16 (D 128)
  constexpr int NI = kDequantTokens / RPP; // rows per thread
  constexpr int NB = D / 16;
  const int c = threadIdx.x % CPR, r = threadIdx.x / CPR;
  const uint8_t* pool = p.pool + (int64_t)g * p.slab + kv * p.half;
  const int64_t page_bytes = (int64_t)p.num_kv_heads * p.slab;
  uint32_t w[NI];
  uint32_t sc[NI];  // NVFP4: E4M3 byte; INT4: fp32 scale bits
  // position of the workgroup's first 16-token group in the page table
  int pidx = t0 / p.page_size, poff = t0 - pidx * p.page_size;
#pragma unroll
  for (int k = 0; k < NI; k++) {
    // row r + RPP k lies in 16-token group (RPP k) / 16 (r < RPP)
    constexpr int kGrpStep = RPP >= 16 ? 1 : 16 / RPP;  // rows k sharing a group
    if (k > 0 && k % kGrpStep == 0) {
      poff += 16;
      if (poff >= p.page_size) {
        poff -= p.page_size;
        pidx += 1;
      }
    }
    const int rr = r + RPP * k - 16 * (k / kGrpStep);  // row inside the group
    const uint8_t* half;
    int off;
    if (TAIL) {
      const int t = t0 + r + RPP * k;
      if (t >= p.prefix_len) continue;
      half = pool + (int64_t)p.pages[t / p.page_size] * page_bytes;
      off = t % p.page_size;
    } else {
      half = pool + (int64_t)p.pages[pidx] * page_bytes;
      off = poff + rr;
    }
    w[k] = ld_stream<uint32_t>(half + (uint32_t)(off * (D / 2) + 4 * c));
    if (FMT == FMT_NVFP4)
      sc[k] = ld_stream<uint8_t>(half + (uint32_t)(p.scales_off + off * NB + (c >> 1)));
    else
      sc[k] = ld_stream<uint32_t>(half + (uint32_t)(p.scales_off + off * 4));
  }
  const float gs = FMT == FMT_NVFP4 ? p.gs[kv] : 1.0f;
  uint16_t* out = (kv ? p.v_out : p.k_out) + (int64_t)g * D + 8 * c;
#pragma unroll
  for (int k = 0; k < NI; k++) {
    const int t = t0 + r + RPP * k;
    if (TAIL && t >= p.prefix_len) continue;
    uint32_t o[4];
    if (FMT == FMT_NVFP4) {
      const float s = e4m3_decode(sc[k]);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        float2_t v;
        switch (e) {
          case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], 1.0f, 0); break;
          case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], 1.0f, 1); break;
          case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], 1.0f, 2); break;
          default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], 1.0f, 3); break;
        }
        v[0] = (v[0] * s) * gs;
        v[1] = (v[1] * s) * gs;
        o[e] = bf16x2_rne(v);
      }
    } else {
      const float s = as_f32(sc[k]);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        float2_t v;
        // sign-extended nibbles 2e, 2e + 1 (v_bfe_i32)
        v[0] = (float)((int)(w[k] << (28 - 8 * e)) >> 28) * s;
        v[1] = (float)((int)(w[k] << (24 - 8 * e)) >> 28) * s;
        o[e] = bf16x2_rne(v);
      }
    }
    // uniform row base plus a 32-bit lane offset
    uint16_t* row = out + (int64_t)(t0 + RPP * k) * p.out_stride;
    *(u32x4_t*)(row + (uint32_t)(r * p.out_stride)) = (u32x4_t){o[0], o[1], o[2], o[3]};
  }
}

template <int D, int FMT>
__global__ __launch_bounds__(256) void dequant_prefix_kernel(DequantParams p) {
  const int kv = (int)blockIdx.y >= p.num_kv_heads ? 1 : 0;
  const int g = (int)blockIdx.y - kv * p.num_kv_heads;
  const int t0 = (int)blockIdx.x * kDequantTokens;
  if (t0 + kDequantTokens <= p.prefix_len)
    dequant_rows<D, FMT, false>(p, kv, g, t0);
  else
    dequant_rows<D, FMT, true>(p, kv, g, t0);
}

hipError_t launch_quantize_store(const StoreParams& p, int fmt, int head_dim, int in_bf16, hipStream_t stream) {
  const int tpw = 256 / (head_dim / 16);
  const dim3 grid((unsigned)((p.num_tokens + tpw - 1) / tpw), (unsigned)(2 * p.num_kv_heads)), block(256);
#define KVQ_STORE(D, T)                                                            \
  do {                                                                             \
    if (fmt == FMT_NVFP4)                                                          \
      hipLaunchKernelGGL((nvfp4_store_kernel<D, T>), grid, block, 0, stream, p);   \
    else if (fmt == FMT_INT4)                                                      \
      hipLaunchKernelGGL((int4_store_kernel<D, T>), grid, block, 0, stream, p);    \
    else if (fmt == FMT_K8V4)                                                      \
      hipLaunchKernelGGL((k8v4_store_kernel<D, T>), grid, block, 0, stream, p);    \
    else                                                                           \
      hipLaunchKernelGGL((fp8_store_kernel<D, T>), grid, block, 0, stream, p);     \
  } while (0)
  if (head_dim == 256) {
    if (in_bf16) KVQ_STORE(256, uint16_t); else KVQ_STORE(256, float);
  } else {
    if (in_bf16) KVQ_STORE(128, uint16_t); else KVQ_STORE(128, float);
  }
#undef KVQ_STORE
  return hipGetLastError();
}

hipError_t launch_dequant_prefix(const DequantParams& p, int fmt, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)((p.prefix_len + kDequantTokens - 1) / kDequantTokens), (unsigned)(2 * p.num_kv_heads));
  const dim3 block(256);
  if (head_dim == 256) {
    if (fmt == FMT_NVFP4) hipLaunchKernelGGL((dequant_prefix_kernel<256, FMT_NVFP4>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((dequant_prefix_kernel<256, FMT_INT4>), grid, block, 0, stream, p);
  } else {
    if (fmt == FMT_NVFP4) hipLaunchKernelGGL((dequant_prefix_kernel<128, FMT_NVFP4>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((dequant_prefix_kernel<128, FMT_INT4>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace kvq
