// kvq_launch.h -- kernel parameter blocks and launchers (internal to libkvq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Wavefronts per decode workgroup: each takes every kDecodeWaves-th 32-token
// chunk of the workgroup's split, and the workgroup merges them in LDS.
constexpr int kDecodeWaves = 4;

// Size of the static device scratch that kvq_decode_attention_noalloc uses in
// place of a caller workspace (16 MiB per device), and the devices it tracks.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
constexpr int kScratchMaxDevices = 64;

struct StoreParams {
  uint8_t* pool;
  const float* gs;  // {gs_K, gs_V} (NVFP4 global / FP8 per-tensor scales)
  const void* k;
  const void* v;
  const int32_t* slots;
  int64_t in_stride;  // elements between tokens
  int64_t slab, half, scales_off;
  int32_t num_tokens, page_size, num_kv_heads;
  int32_t rotate;     // Hadamard-rotate each row before quantizing
  float rot_scale;    // fp32(1 / sqrt(head_dim))
};

struct RotateParams {
  const void* in;
  void* out;
  int64_t in_stride, out_stride;  // elements between rows
  int32_t rows;
  float scale;  // fp32(1 / sqrt(head_dim))
};

struct DequantParams {
  const uint8_t* pool;
  const float* gs;
  const int32_t* pages;
  uint16_t* k_out;
  uint16_t* v_out;
  int64_t out_stride;
  int64_t slab, half, scales_off;
  int32_t prefix_len, page_size, num_kv_heads;
};

struct DecodeParams {
  const uint8_t* pool;
  const float* gs;
  const uint16_t* q;  // bf16 [B][Hq][D]
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* part_o;   // [B][Hkv][S][G][D]
  float* part_ml;  // [B][Hkv][S][G][2]
  void* out;
  float* lse;
  int64_t slab, half, scales_off;
  float sm_scale;
  int32_t max_pages, batch, num_kv_heads, num_q_heads, group, page_size;
  int32_t num_splits, chunks_per_split;
  int32_t out_bf16;
};

struct ExtendParams {
  const uint16_t* q;  // bf16 [chunk_len][q_stride], head h at h * head_dim
  const uint16_t* k;  // bf16: workspace [prefix_len + chunk_len][kv_stride], or (paged) the chunk's rows
  const uint16_t* v;
  void* out;          // [chunk_len][out_stride], bf16 or fp32
  float* lse;         // [chunk_len][lse_stride] or null
  int64_t q_stride, kv_stride, out_stride, lse_stride;
  float sm_scale;
  int32_t prefix_len, chunk_len, num_q_heads, num_kv_heads, group, out_bf16;
  // paged prefix (the 4-bit cache read directly; unused for the workspace variant)
  const uint8_t* pool;
  const float* gs;
  const int32_t* pages;
  int64_t slab, half, scales_off;
  int32_t page_size;
};

hipError_t launch_quantize_store(const StoreParams& p, int fmt, int head_dim, int in_bf16, hipStream_t stream);
hipError_t launch_dequant_prefix(const DequantParams& p, int fmt, int head_dim, hipStream_t stream);
hipError_t launch_calibrate_amax(const StoreParams& p, int head_dim, int in_bf16, float* running, hipStream_t stream);
hipError_t launch_global_scale(const float* running, float* gs, hipStream_t stream);
hipError_t launch_hadamard(const RotateParams& p, int head_dim, int in_bf16, int out_bf16, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int fmt, int head_dim, hipStream_t stream);
// Device address of the current device's static decode scratch
// (kDecodeScratchBytes), looked up on the first call per device.
hipError_t decode_scratch(void** ptr);
hipError_t launch_extend(const ExtendParams& p, int head_dim, int src_fmt, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int workgroups, hipStream_t stream);
hipError_t launch_stream_write(void* buf, int64_t bytes, uint32_t value, int workgroups, hipStream_t stream);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, int workgroups, hipStream_t stream);
hipError_t launch_mfma_rate(int lds_fed, int iters, int workgroups, uint32_t* sink, hipStream_t stream);

}  // namespace kvq
