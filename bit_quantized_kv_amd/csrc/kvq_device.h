// kvq_device.h -- device-side types and codecs shared by the gfx950 kernels.
//
// Formats (see include/kvq.h): NVFP4 = E2M1 elements, one OCP E4M3 scale per
// 16 head-dim elements of a token row, FP32 per-layer global scale; INT4 =
// symmetric -7..7 two's-complement nibbles with one FP32 scale per token and
// head.  Even element in the low nibble.  FP8 (the comparator) = one OCP E4M3
// byte per value with one FP32 scale per tensor, V stored by channel.  K8V4 =
// FP8 keys (by token, per-tensor scale) with NVFP4 values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

enum { FMT_NVFP4 = 1, FMT_INT4 = 2, FMT_FP8 = 3, FMT_K8V4 = 4 };

// Byte layout of one slab (one page of one KV head).
struct SlabLayout {
  int64_t code_row;    // bytes per row of codes (head_dim / 2)
  int64_t scale_row;   // bytes per row of scales (head_dim / 16, or 4)
  int64_t half;        // bytes of the K half (codes + scales)
  int64_t scales_off;  // offset of the scales within a half
  int64_t slab;        // bytes of the whole slab
};

__host__ __device__ inline SlabLayout slab_layout(int fmt, int page_size, int head_dim) {
  SlabLayout s;
  if (fmt == FMT_K8V4) {
    // [K: page_size rows x head_dim bytes][V codes: page_size x head_dim/2][V scales]
    s.code_row = head_dim / 2;  // of the V section
    s.scale_row = head_dim / 16;
    s.half = (int64_t)page_size * head_dim;             // offset of the V section
    s.scales_off = (int64_t)page_size * s.code_row;     // within the V section
    s.slab = s.half + (int64_t)page_size * (s.code_row + s.scale_row);
    return s;
  }
  if (fmt == FMT_FP8) {
    // [K: page_size rows x head_dim bytes][V: head_dim rows x page_size bytes]
    s.code_row = head_dim;
    s.scale_row = 0;
    s.scales_off = (int64_t)page_size * head_dim;
    s.half = (int64_t)page_size * head_dim;
    s.slab = 2 * s.half;
    return s;
  }
  s.code_row = head_dim / 2;
  s.scale_row = fmt == FMT_NVFP4 ? head_dim / 16 : 4;
  s.scales_off = (int64_t)page_size * s.code_row;
  s.half = (int64_t)page_size * (s.code_row + s.scale_row);
  s.slab = 2 * s.half;
  return s;
}

// ---------------------------------------------------------------- global loads
// Loads through an explicitly global (address space 1) pointer, so the
// compiler emits global_load rather than flat_load (flat loads also count
// against the scalar/LDS counter and would serialize the prefetch).
// T is a scalar or a clang ext_vector type.
template <typename T>
__device__ inline T ld_global(const void* ptr) {
  return *(const __attribute__((address_space(1))) T*)ptr;
}

// The same load with the non-temporal cache policy (global_load ... nt), for
// data read once per call (cache pages, the bulk rows of a store): measured
// on MI355X, a plain 4 GiB read runs at 7.07 TB/s with it against 6.36 TB/s
// without.
template <typename T>
__device__ inline T ld_stream(const void* ptr) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) T*)ptr);
}

// Cache-policy operand of the raw buffer loads for the same once-read data:
// bit 1 is "nt" on gfx950 (7.14 TB/s on a 4 GiB buffer read against 6.41
// TB/s with no bits set), bit 0 "sc0" (with nt: 7.21 TB/s).
constexpr int kLoadStream = 3;

// ---------------------------------------------------------------- bit casts
__device__ inline uint32_t as_u32(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ inline float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ inline uint32_t h2_as_u32(half2_t x) { return __builtin_bit_cast(uint32_t, x); }
__device__ inline half2_t u32_as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }

// (x & mask) | (y & ~mask): one v_bfi_b32.
__device__ inline uint32_t bitfield_insert(uint32_t mask, uint32_t x, uint32_t y) {
  return (x & mask) | (y & ~mask);
}

// Byte permute of {hi, lo} (v_perm_b32): selector byte i picks byte sel_i of
// the 8-byte value (lo = bytes 0..3, hi = bytes 4..7); 0x0C yields 0x00.
__device__ inline uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Value of lane I of each quad (DPP quad_perm broadcast, no LDS traffic).
template <int I>
__device__ inline uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, I * 0x55, 0xF, 0xF, false);
}

// x of lane l ^ m (m = 1, 2, 4 or 8) within the lane's 16-lane row, with
// DPP moves only (no LDS round trip): quad permutations for 1 and 2, a
// half-row mirror followed by a quad reversal for 4, a row rotation by 8
// for 8.  m must be a compile-time constant after unrolling.
__device__ inline float lane_xor16(float x, int m) {
  const int v = (int)as_u32(x);
  int r;
  if (m == 1)
    r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  else if (m == 2)
    r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  else if (m == 4)
    r = __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false), 0x1B, 0xF, 0xF, false);
  else
    r = __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);
  return as_f32((uint32_t)r);
}

// max over lanes {l, l^16, l^32, l^48} with the gfx950 lane-swap instructions
// (VALU only, no LDS round trip).
__device__ inline float max_xor16_xor32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  x = fmaxf(as_f32(a[0]), as_f32(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return fmaxf(as_f32(b[0]), as_f32(b[1]));
}

// ---------------------------------------------------------------- encoders

// Two fp32 -> two bf16 (element 0 in the low half), round to nearest even,
// denormals kept: one v_cvt_pk_bf16_f32.
__device__ inline uint32_t bf16x2_rne(float2_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Non-negative fp32 -> E4M3 (OCP) code: round to nearest, ties to even,
// saturating at 448 (0x7E).  Integer rounding of the fp32 significand for the
// normal range; the subnormal range (below 2^-6) is a multiple of 2^-9 and is
// rounded with rint(s * 2^9), which is exact scaling followed by RNE.
__device__ inline uint32_t e4m3_encode(float s) {
  if (s != s) return 0x7Fu;
  if (!(s < 448.0f)) return 0x7Eu;
  uint32_t u = as_u32(s);
  int e = (int)(u >> 23) - 127;
  if (e >= -6) {
    uint32_t mant = u & 0x7FFFFFu;
    uint32_t q = mant >> 20;
    uint32_t rem = mant & 0xFFFFFu;
    uint32_t code = ((uint32_t)(e + 7) << 3) | q;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) code += 1;
    return code;
  }
  return (uint32_t)__builtin_rintf(s * 512.0f);
}

// E4M3 code -> fp32 (exact).  Hardware OCP E4M3 conversion (v_cvt_pk_f32_fp8).
__device__ inline float e4m3_decode(uint32_t code) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(code, false)[0];
}

// ---------------------------------------------------------------- decoders for the attention kernels

// E4M3 code byte(s) -> fp16 value * 2^-8: the 7 exponent/mantissa bits moved
// up by 7 land on fp16's exponent/mantissa with an exponent offset of 8
// (subnormals included), exact.  The sign bit (always 0 for a stored scale)
// is dropped so even corrupt bytes give finite values.
__device__ inline uint32_t e4m3_to_h_x2m8(uint32_t b) { return (b & 0x7Fu) << 7; }

// The same for two code bytes at bytes 0 and 2 of x (bytes 1 and 3 zero):
// both fp16 halves in one shift and one mask.
__device__ inline uint32_t e4m3_to_h_x2m8_pair(uint32_t x) { return (x << 7) & 0x3F803F80u; }

// Two E2M1 nibbles (byte `sel` of w: low nibble -> element 0, high -> element
// 1) as exact fp16 values times 2^8 (v_cvt_scalef32_pk_f16_fp4; that
// instruction applies only the exponent of its scale operand, so the 2^8 is
// free and exact).  Paired with scales from e4m3_to_h_x2m8 the product is the
// exact e2m1 * e4m3.
template <int SEL>
__device__ inline half2_t e2m1x2_to_h2_x256(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, SEL);
}

// Two-nibble INT4 pairs: the two's-complement nibbles at positions p and
// p + 4 of w become fp16 (q_p, q_{p+4}) exactly.  Each nibble u lands in the
// low mantissa bits of 1024 (0x6400) with its sign bit flipped (the XOR with
// 0x0008 turns u into q + 8), then 1032 is subtracted: mask, bias and the
// 0x6400 fill are one AND + XOR (a single v_bitop3), so no separate pass over
// the word is needed.
template <int P>
__device__ inline half2_t int4x2_to_h2(uint32_t w) {
  uint32_t t = ((w >> (4 * P)) & 0x000F000Fu) ^ 0x64086408u;
  return u32_as_h2(t) - (half2_t){(_Float16)1032.0f, (_Float16)1032.0f};
}

// The same for the nibbles at positions 1 and 5 without a shift: left in
// place they land 4 bits up in the mantissa of 1024 (the XOR with 0x0080
// flips their sign bit), so the result is (16 q_1, 16 q_5), exact; the caller
// undoes the factor 16 where it is cheap (the query, the output).  With the
// word shifted right by 8 once, int4x2_to_h2<0> and this serve positions 2, 6
// and 3, 7: one shift per word instead of three.
__device__ inline half2_t int4x2_hi_to_h2_x16(uint32_t w) {
  uint32_t t = (w & 0x00F000F0u) ^ 0x64806480u;
  return u32_as_h2(t) - (half2_t){(_Float16)1152.0f, (_Float16)1152.0f};
}

}  // namespace kvq
