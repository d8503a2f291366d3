"""bit_quantized_kv_amd -- a 4-bit paged KV cache (NVFP4 and INT4 per-token-head)
for MI355X: HIP kernels for gfx950 behind the C ABI in include/kvq.h, with a
thin ctypes binding (``bit_quantized_kv_amd.kvq``)."""

__all__ = ["kvq", "inputs", "build"]
