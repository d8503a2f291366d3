// kvq_store.hip -- quantize-on-write and prefix dequantization for gfx950.
//
// Quantize-on-write follows the write path of "SGLang's 4-bit KV cache: the
// 56% is exact, the 1.78x is untested" (Figure 2 caption: prefill and decode
// quantize K/V and store them into the shared pool) for NVFP4, and the INT4
// write path of "KV cache in 4 bits: 8.8 instead of 4.7 full sessions on the
// same four RTX 5090s" ("What we changed").  Prefix dequantization is the
// extend path of the same Figure 2 caption, with a bf16 workspace.
//
// Both kernels stream: one thread per 16-element block of a (token, head,
// K|V) row, 16/32-byte vector loads and stores, consecutive threads on
// consecutive blocks so every wavefront touches contiguous memory.  Every
// rounding decision is made in IEEE fp32 (correctly rounded division, no FMA
// contraction), so the packed bytes are bit-exact against a scalar
// implementation of the same rules.
#pragma clang fp contract(off)

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

template <typename T>
struct Row16;

template <>
struct Row16<float> {
  __device__ static void load(const void* p, float x[16]) {
    const float4* v = (const float4*)p;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float4 a = v[i];
      x[4 * i + 0] = a.x;
      x[4 * i + 1] = a.y;
      x[4 * i + 2] = a.z;
      x[4 * i + 3] = a.w;
    }
  }
};

template <>
struct Row16<uint16_t> {  // bf16 bit patterns, widened exactly
  __device__ static void load(const void* p, float x[16]) {
    const uint4* v = (const uint4*)p;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      uint4 a = v[i];
      uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        x[8 * i + 2 * j] = as_f32(w[j] << 16);
        x[8 * i + 2 * j + 1] = as_f32(w[j] & 0xFFFF0000u);
      }
    }
  }
};

// Thread t handles block b = t % (D/16) of row (token i, K|V, head g), rows
// ordered token-major so a wavefront reads a contiguous span of each token.
template <int D, typename TIn>
__global__ __launch_bounds__(256) void nvfp4_store_kernel(StoreParams p) {
  constexpr int NB = D / 16;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.num_tokens * 2 * p.num_kv_heads * NB;
  if (tid >= total) return;
  const int b = (int)(tid % NB);
  const int64_t row = tid / NB;
  const int g = (int)(row % p.num_kv_heads);
  const int kv = (int)((row / p.num_kv_heads) & 1);
  const int64_t i = row / (2 * p.num_kv_heads);
  const int32_t slot = p.slots[i];
  if (slot < 0) return;

  float x[16];
  const TIn* src = (const TIn*)(kv ? p.v : p.k) + i * p.in_stride + (int64_t)g * D + 16 * b;
  Row16<TIn>::load(src, x);

  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; e++) {
    float a = __builtin_fabsf(x[e]);
    amax = a > amax ? a : amax;
  }
  const float gs = p.gs[kv];
  const float den = 6.0f * gs;
  const float s_raw = amax / den;
  const uint32_t cs = e4m3_encode(s_raw);
  const float S = e4m3_decode(cs) * gs;

  uint32_t w0 = 0, w1 = 0;
  if (S != 0.0f) {
#pragma unroll
    for (int e = 0; e < 8; e++) w0 |= e2m1_encode(x[e] / S) << (4 * e);
#pragma unroll
    for (int e = 0; e < 8; e++) w1 |= e2m1_encode(x[8 + e] / S) << (4 * e);
  }
  const int64_t page = slot / p.page_size;
  const int64_t off = slot % p.page_size;
  uint8_t* half = p.pool + (page * p.num_kv_heads + g) * p.slab + kv * p.half;
  *(uint2*)(half + off * (D / 2) + 8 * b) = make_uint2(w0, w1);
  half[p.scales_off + off * NB + b] = (uint8_t)cs;
}

// INT4: the D/16 threads of one row reduce the row amax with lane shuffles.
template <int D, typename TIn>
__global__ __launch_bounds__(256) void int4_store_kernel(StoreParams p) {
  constexpr int NB = D / 16;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.num_tokens * 2 * p.num_kv_heads * NB;
  if (tid >= total) return;  // whole rows only: total is a multiple of NB
  const int b = (int)(tid % NB);
  const int64_t row = tid / NB;
  const int g = (int)(row % p.num_kv_heads);
  const int kv = (int)((row / p.num_kv_heads) & 1);
  const int64_t i = row / (2 * p.num_kv_heads);
  const int32_t slot = p.slots[i];
  if (slot < 0) return;  // uniform over the row's lanes

  float x[16];
  const TIn* src = (const TIn*)(kv ? p.v : p.k) + i * p.in_stride + (int64_t)g * D + 16 * b;
  Row16<TIn>::load(src, x);
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; e++) {
    float a = __builtin_fabsf(x[e]);
    amax = a > amax ? a : amax;
  }
#pragma unroll
  for (int m = 1; m < NB; m <<= 1) {
    float o = __shfl_xor(amax, m, NB);
    amax = o > amax ? o : amax;
  }
  const float s = amax / 7.0f;
  uint32_t w0 = 0, w1 = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int e = 0; e < 16; e++) {
      float r = __builtin_rintf(x[e] / s);
      r = r > 7.0f ? 7.0f : (r < -7.0f ? -7.0f : r);
      uint32_t nib = (uint32_t)(int)r & 0xFu;
      if (e < 8)
        w0 |= nib << (4 * e);
      else
        w1 |= nib << (4 * (e - 8));
    }
  }
  const int64_t page = slot / p.page_size;
  const int64_t off = slot % p.page_size;
  uint8_t* half = p.pool + (page * p.num_kv_heads + g) * p.slab + kv * p.half;
  *(uint2*)(half + off * (D / 2) + 8 * b) = make_uint2(w0, w1);
  if (b == 0) *(float*)(half + p.scales_off + off * 4) = s;
}

// Prefix dequantization: thread per 16-element block, writing 32 bytes of
// bf16.  NVFP4 value fp32(e2m1 * e4m3) is exact; one fp32 multiply by gs; bf16
// round-to-nearest-even.  INT4 value fp32(q * s).
template <int D, int FMT>
__global__ __launch_bounds__(256) void dequant_prefix_kernel(DequantParams p) {
  constexpr int NB = D / 16;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.prefix_len * 2 * p.num_kv_heads * NB;
  if (tid >= total) return;
  const int b = (int)(tid % NB);
  const int64_t row = tid / NB;
  const int g = (int)(row % p.num_kv_heads);
  const int kv = (int)((row / p.num_kv_heads) & 1);
  const int64_t t = row / (2 * p.num_kv_heads);
  const int64_t page = p.pages[t / p.page_size];
  const int64_t off = t % p.page_size;
  const uint8_t* half = p.pool + (page * p.num_kv_heads + g) * p.slab + kv * p.half;
  const uint2 w = *(const uint2*)(half + off * (D / 2) + 8 * b);
  uint32_t outw[8];
  if (FMT == FMT_NVFP4) {
    const float sc = e4m3_decode(half[p.scales_off + off * NB + b]);
    const float gs = p.gs[kv];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      uint32_t word = e < 8 ? w.x : w.y;
      int sh = 4 * (e & 7);
      uint32_t c0 = (word >> sh) & 15u, c1 = (word >> (sh + 4)) & 15u;
      float v0 = e2m1_magnitude(c0 & 7u) * sc, v1 = e2m1_magnitude(c1 & 7u) * sc;
      v0 = (c0 & 8u) ? -v0 : v0;
      v1 = (c1 & 8u) ? -v1 : v1;
      outw[e / 2] = (uint32_t)f32_to_bf16_rne(v0 * gs) | ((uint32_t)f32_to_bf16_rne(v1 * gs) << 16);
    }
  } else {
    const float s = *(const float*)(half + p.scales_off + off * 4);
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      uint32_t word = e < 8 ? w.x : w.y;
      int sh = 4 * (e & 7);
      int q0 = (int)(((word >> sh) & 15u) ^ 8u) - 8, q1 = (int)(((word >> (sh + 4)) & 15u) ^ 8u) - 8;
      outw[e / 2] = (uint32_t)f32_to_bf16_rne((float)q0 * s) | ((uint32_t)f32_to_bf16_rne((float)q1 * s) << 16);
    }
  }
  uint16_t* dst = (kv ? p.v_out : p.k_out) + t * p.out_stride + (int64_t)g * D + 16 * b;
  ((uint4*)dst)[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
  ((uint4*)dst)[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
}

static inline unsigned grid_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

hipError_t launch_quantize_store(const StoreParams& p, int fmt, int head_dim, int in_bf16, hipStream_t stream) {
  const int64_t threads = (int64_t)p.num_tokens * 2 * p.num_kv_heads * (head_dim / 16);
  const dim3 grid(grid_for(threads)), block(256);
#define KVQ_STORE(D, T)                                                            \
  do {                                                                             \
    if (fmt == FMT_NVFP4)                                                          \
      hipLaunchKernelGGL((nvfp4_store_kernel<D, T>), grid, block, 0, stream, p);   \
    else                                                                           \
      hipLaunchKernelGGL((int4_store_kernel<D, T>), grid, block, 0, stream, p);    \
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
  const int64_t threads = (int64_t)p.prefix_len * 2 * p.num_kv_heads * (head_dim / 16);
  const dim3 grid(grid_for(threads)), block(256);
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
