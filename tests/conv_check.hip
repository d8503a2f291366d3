// conv_check.hip -- exhaustive checks of the gfx950 conversion instructions
// that the library's bit-exact paths rest on (test infrastructure only; built
// by the package build into tests/libkvq_convcheck.so and driven by
// tests/test_gpu_conversions.py).
//
// Each check runs the instruction, through the same compiler builtin the
// library uses, over every input of its domain and compares it with a
// reference rule written here from the format definitions ("SGLang's 4-bit KV
// cache: the 56% is exact, the 1.78x is untested", section "The 56% survives
// its own scale, and names the block size": E2M1 elements, E4M3 block
// scales):
//   - v_cvt_scalef32_pk_fp4_f32 at scale 1 (the NVFP4 element encoder):
//     every fp32 bit pattern but NaN, in both nibbles and all four byte
//     positions, against round-to-nearest with ties to the even code,
//     saturation at 6 and the sign kept;
//   - v_cvt_pk_bf16_f32 (the bf16 output and prefix-dequant rounding): every
//     fp32 bit pattern but NaN, in both halves, against integer
//     round-to-nearest-even of the bit pattern;
//   - v_cvt_scalef32_pk_f16_fp4 at scale 2^8 and v_cvt_scalef32_pk_f32_fp4 at
//     scale 1 (the 4-bit decoders): all 256 code bytes in all four byte
//     positions, against the E2M1 value set;
//   - v_cvt_pk_f32_fp8 and v_cvt_scalef32_pk_f16_fp8 at scale 1 (E4M3 scale
//     and FP8 value decoders): all 256 codes in both byte halves, against the
//     OCP E4M3 definition (0x7F and 0xFF NaN);
//   - v_cvt_pk_fp8_f32 after a clamp to [-448, 448] (the FP8 value encoder):
//     every fp32 bit pattern but NaN, in both bytes of both halves of the
//     word, against round-to-nearest with ties to the even code, saturation
//     at 448 and the sign kept.
// A sweep writes, per workgroup, the number of mismatches and the smallest
// mismatching input (0xFFFFFFFF if none); nothing is atomic.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

namespace {

constexpr int kThreads = 256;
constexpr int kWorkgroups = 16384;                   // x 256 threads x 1024 inputs = 2^32
constexpr int kPerThread = 1024;
constexpr uint32_t kStride = (uint32_t)kThreads * kWorkgroups;

__device__ inline float bits_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ inline uint32_t f_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ inline bool is_nan_bits(uint32_t u) { return (u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu); }

// E2M1 code of r: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; the midpoints
// .25, 1.25, 2.5 and 5 go to the even code below, .75, 1.75 and 3.5 to the
// even code above; 6 and beyond (and infinity) saturate to code 7; the sign
// bit of r is kept (so -0 and negative tiny values give 0x8).
__device__ inline uint32_t e2m1_ref(uint32_t u) {
  const float a = bits_f(u & 0x7FFFFFFFu);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return c | ((u >> 28) & 8u);
}

// bf16 bit pattern of fp32 bits u (not NaN): round to nearest, ties to even,
// on the integer pattern (overflow carries into the exponent, i.e. to inf).
__device__ inline uint32_t bf16_ref(uint32_t u) { return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16; }

__device__ inline float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float mag = e == 0 ? 0.5f * (float)m : (float)(1u << (e - 1)) * (1.0f + 0.5f * (float)m);
  return (c & 8u) ? -mag : mag;
}

__device__ inline float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 15 && m == 7) return __builtin_nanf("");
  const float mag = e == 0 ? (float)m * 0x1p-9f : (1.0f + (float)m / 8.0f) * __builtin_ldexpf(1.0f, (int)e - 7);
  return (c & 0x80u) ? -mag : mag;
}

__device__ inline bool same_value(float got, float want) {
  if (want != want) return got != got;
  return f_bits(got) == f_bits(want);  // also tells -0 from +0
}

// Workgroup result: mismatch count and smallest mismatching input.
__device__ inline void finish(uint32_t bad, uint32_t first, uint32_t* count, uint32_t* first_out) {
  __shared__ uint32_t s_bad[kThreads], s_first[kThreads];
  s_bad[threadIdx.x] = bad;
  s_first[threadIdx.x] = first;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      s_bad[threadIdx.x] += s_bad[threadIdx.x + w];
      s_first[threadIdx.x] = min(s_first[threadIdx.x], s_first[threadIdx.x + w]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    count[blockIdx.x] = s_bad[0];
    first_out[blockIdx.x] = s_first[0];
  }
}

// Every fp32 input u but NaN: as the low element (byte position u % 4, the
// other bytes of the old word kept) and as the high element of the pair.
__global__ __launch_bounds__(kThreads) void fp4_encode_sweep(uint32_t* count, uint32_t* first_out) {
  uint32_t bad = 0, first = 0xFFFFFFFFu;
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  const float partner = 3.0f;  // code 5
  for (int i = 0; i < kPerThread; i++) {
    const uint32_t u = t + (uint32_t)i * kStride;
    if (is_nan_bits(u)) continue;
    const uint32_t want = e2m1_ref(u);
    const uint32_t old = 0xA5C3E1F0u;
    uint32_t w_lo, w_hi;
    switch (u & 3u) {
      case 0:
        w_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, bits_f(u), partner, 1.0f, 0);
        w_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, partner, bits_f(u), 1.0f, 0);
        break;
      case 1:
        w_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, bits_f(u), partner, 1.0f, 1);
        w_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, partner, bits_f(u), 1.0f, 1);
        break;
      case 2:
        w_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, bits_f(u), partner, 1.0f, 2);
        w_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, partner, bits_f(u), 1.0f, 2);
        break;
      default:
        w_lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, bits_f(u), partner, 1.0f, 3);
        w_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, partner, bits_f(u), 1.0f, 3);
        break;
    }
    const int sh = 8 * (int)(u & 3u);
    const uint32_t keep = ~(0xFFu << sh);
    const bool ok = (w_lo & keep) == (old & keep) && (w_hi & keep) == (old & keep) &&
                    ((w_lo >> sh) & 0xFFu) == (want | (5u << 4)) && ((w_hi >> sh) & 0xFFu) == (5u | (want << 4));
    if (!ok) {
      bad++;
      first = min(first, u);
    }
  }
  finish(bad, first, count, first_out);
}

// Every fp32 input u but NaN, in the low and in the high half of the pair.
__global__ __launch_bounds__(kThreads) void bf16_round_sweep(uint32_t* count, uint32_t* first_out) {
  uint32_t bad = 0, first = 0xFFFFFFFFu;
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  const float partner = -1.5f;  // 0xBFC0
  for (int i = 0; i < kPerThread; i++) {
    const uint32_t u = t + (uint32_t)i * kStride;
    if (is_nan_bits(u)) continue;
    const uint32_t want = bf16_ref(u);
    const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){bits_f(u), partner}, bf16x2_t));
    const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){partner, bits_f(u)}, bf16x2_t));
    if (a != (want | (0xBFC0u << 16)) || b != (0xBFC0u | (want << 16))) {
      bad++;
      first = min(first, u);
    }
  }
  finish(bad, first, count, first_out);
}

// All 256 code bytes x 4 byte positions (one thread each): the two nibbles of
// byte `sel` decoded by the fp16 (scale 2^8) and fp32 (scale 1) conversions.
__global__ __launch_bounds__(kThreads) void fp4_decode_sweep(uint32_t* count, uint32_t* first_out) {
  uint32_t bad = 0, first = 0xFFFFFFFFu;
  for (uint32_t k = threadIdx.x; k < 1024; k += kThreads) {
    const uint32_t byte = k & 0xFFu, sel = k >> 8;
    const uint32_t w = 0x96969696u ^ (0x96u << (8 * sel)) ^ (byte << (8 * sel));
    half2_t h;
    float2_t f;
    switch (sel) {
      case 0:
        h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0);
        f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
        break;
      case 1:
        h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1);
        f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
        break;
      case 2:
        h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2);
        f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
        break;
      default:
        h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3);
        f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
        break;
    }
    const float v0 = e2m1_value(byte & 15u), v1 = e2m1_value(byte >> 4);
    const bool ok = same_value((float)h[0], v0 * 256.0f) && same_value((float)h[1], v1 * 256.0f) &&
                    same_value(f[0], v0) && same_value(f[1], v1);
    if (!ok) {
      bad++;
      first = min(first, k);
    }
  }
  finish(bad, first, count, first_out);
}

// All 256 E4M3 codes in the low and the high byte of a word's lower half:
// v_cvt_pk_f32_fp8 (both results) and v_cvt_scalef32_pk_f16_fp8 at scale 1.
__global__ __launch_bounds__(kThreads) void fp8_decode_sweep(uint32_t* count, uint32_t* first_out) {
  uint32_t bad = 0, first = 0xFFFFFFFFu;
  const uint32_t c = threadIdx.x;  // 256 threads: one code each
  const uint32_t partner = 0x38u;  // 1.0
  for (int pos = 0; pos < 2; pos++) {
    const uint32_t w = pos == 0 ? (c | (partner << 8) | 0x4C3A0000u) : (partner | (c << 8) | 0x4C3A0000u);
    const float2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const half2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    const float want = e4m3_value(c);
    const float got_f = pos == 0 ? f[0] : f[1], other_f = pos == 0 ? f[1] : f[0];
    const float got_h = (float)(pos == 0 ? h[0] : h[1]), other_h = (float)(pos == 0 ? h[1] : h[0]);
    const bool ok = same_value(got_f, want) && same_value(got_h, want) && other_f == 1.0f && other_h == 1.0f;
    if (!ok) {
      bad++;
      first = min(first, c | ((uint32_t)pos << 8));
    }
  }
  finish(bad, first, count, first_out);
}

// E4M3 code of fp32 bits u (not NaN), the rule of the FP8 values: the sign
// bit kept; magnitudes of 448 and beyond (and infinity) saturate to 448
// (0x7E); normal results (>= 2^-6) keep 3 mantissa bits, rounded to nearest
// with ties to the even code (a carry moves into the exponent); below 2^-6
// the subnormal codes m 2^-9, m = rint(|x| 2^9), ties to even.
__device__ inline uint32_t e4m3_ref(uint32_t u) {
  const uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
  uint32_t c;
  if (bits_f(a) >= 448.0f) {
    c = 0x7Eu;
  } else if (bits_f(a) >= 0x1p-6f) {
    const uint32_t e = (a >> 23) - 127u + 7u, m = a & 0x7FFFFFu;
    const uint32_t q = m >> 20, rem = m & 0xFFFFFu;
    c = (e << 3) + q + ((rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u);
  } else {
    c = (uint32_t)__builtin_rintf(bits_f(a) * 512.0f);  // exact scaling; rint ties to even
  }
  return c | sign;
}

// Every fp32 input u but NaN, clamped to [-448, 448] as the library clamps
// before converting, in byte 0 and 1 of the low half and byte 2 and 3 of the
// high half (the other byte of the pair holds 1.0, code 0x38; the other half
// of the old word is kept).
__global__ __launch_bounds__(kThreads) void fp8_encode_sweep(uint32_t* count, uint32_t* first_out) {
  uint32_t bad = 0, first = 0xFFFFFFFFu;
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  const float partner = 1.0f;
  const uint32_t old = 0xC3A5E15Au;
  for (int i = 0; i < kPerThread; i++) {
    const uint32_t u = t + (uint32_t)i * kStride;
    if (is_nan_bits(u)) continue;
    const uint32_t want = e4m3_ref(u);
    const float y = __builtin_amdgcn_fmed3f(bits_f(u), -448.0f, 448.0f);
    const uint32_t lo0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, partner, (int)old, false);
    const uint32_t lo1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(partner, y, (int)old, false);
    const uint32_t hi0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, partner, (int)old, true);
    const uint32_t hi1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(partner, y, (int)old, true);
    const bool ok = lo0 == ((old & 0xFFFF0000u) | want | (0x38u << 8)) &&
                    lo1 == ((old & 0xFFFF0000u) | 0x38u | (want << 8)) &&
                    hi0 == ((old & 0xFFFFu) | (want << 16) | (0x38u << 24)) &&
                    hi1 == ((old & 0xFFFFu) | (0x38u << 16) | (want << 24));
    if (!ok) {
      bad++;
      first = min(first, u);
    }
  }
  finish(bad, first, count, first_out);
}

}  // namespace

// Each entry runs one sweep on `stream` and writes per-workgroup results into
// count[] and first[] (device uint32 arrays of kvqc_workgroups(which) entries).
// which: 0 fp4 encode, 1 bf16 rounding, 2 fp4 decode, 3 fp8 decode, 4 fp8 encode.
extern "C" int kvqc_workgroups(int which) { return which <= 1 || which == 4 ? kWorkgroups : 1; }

extern "C" int kvqc_run(int which, uint32_t* count, uint32_t* first, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (which) {
    case 0: hipLaunchKernelGGL(fp4_encode_sweep, dim3(kWorkgroups), dim3(kThreads), 0, s, count, first); break;
    case 1: hipLaunchKernelGGL(bf16_round_sweep, dim3(kWorkgroups), dim3(kThreads), 0, s, count, first); break;
    case 2: hipLaunchKernelGGL(fp4_decode_sweep, dim3(1), dim3(kThreads), 0, s, count, first); break;
    case 3: hipLaunchKernelGGL(fp8_decode_sweep, dim3(1), dim3(kThreads), 0, s, count, first); break;
    case 4: hipLaunchKernelGGL(fp8_encode_sweep, dim3(kWorkgroups), dim3(kThreads), 0, s, count, first); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}
