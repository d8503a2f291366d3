"""Python binding of libkvq (ctypes): argument marshalling only.

Every function here has the name of the C entry point it calls (include/kvq.h)
and does no arithmetic of the method: torch supplies device memory and the
current HIP stream, the kernels do the work.  If libkvq.so has not been built
the first call raises -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

NVFP4 = 1
INT4_TOKHEAD = 2
FP8_E4M3 = 3  # the per-tensor FP8 comparator format
K8V4 = 4  # FP8 keys (per-tensor scale) with NVFP4 values
DT_F32 = 0
DT_BF16 = 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")
_lib = None


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})"
                         + (f", hipError {lib().kvq_last_hip_error()}" if status == -6 else ""))
        self.status = status


class kvq_cache(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("pool", ctypes.c_void_p),
        ("global_scale", ctypes.c_void_p),
        ("flags", ctypes.c_int32),
    ]


FLAG_HADAMARD = 1  # rows Hadamard-rotated before quantization


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libkvq.so is not built ({LIB_PATH}); run `python -m bit_quantized_kv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    C = ctypes.POINTER(kvq_cache)
    sig = {
        "kvq_slab_bytes": (sz, [i32, i32, i32]),
        "kvq_quantize_store": (i32, [C, P, P, i32, i64, P, i32, P]),
        "kvq_decode_num_splits": (i32, [C, i32, i32, i32, ctypes.POINTER(i32)]),
        "kvq_decode_workspace_size": (i32, [C, i32, i32, i32, i32, ctypes.POINTER(sz)]),
        "kvq_decode_attention": (i32, [C, P, i32, P, i32, P, i32, i32, f32, i32, P, i32, P, P, sz, P]),
        "kvq_decode_attention_noalloc": (i32, [C, P, i32, P, i32, P, i32, i32, f32, i32, P, i32, P, P]),
        "kvq_dequant_prefix": (i32, [C, P, i32, P, P, i64, P]),
        "kvq_stream_read": (i32, [P, sz, P, i32, P]),
        "kvq_stream_write": (i32, [P, sz, ctypes.c_uint32, i32, P]),
        "kvq_stream_copy": (i32, [P, P, sz, i32, P]),
        "kvq_mfma_rate": (i32, [i32, i32, i32, P, P]),
        "kvq_calibrate_amax": (i32, [C, P, P, i32, i64, i32, P, P]),
        "kvq_calibrate_global_scale": (i32, [C, P, P]),
        "kvq_hadamard_rotate": (i32, [P, i32, i64, P, i32, i64, i32, i32, P]),
        "kvq_extend_attention": (i32, [P, i64, i32, P, P, i64, i32, i32, i32, i32, f32, P, i32, i64, P, P]),
        "kvq_extend_attention_paged": (i32, [C, P, i32, P, i64, i32, P, P, i64, i32, f32, P, i32, i64, P, P]),
        "kvq_status_string": (ctypes.c_char_p, [i32]),
        "kvq_last_hip_error": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().kvq_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise KvqError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def kvq_slab_bytes(fmt: int, page_size: int, head_dim: int) -> int:
    return int(lib().kvq_slab_bytes(fmt, page_size, head_dim))


class Cache:
    """One layer's paged cache: a device uint8 pool
    [num_pages][num_kv_heads][slab] and the device float[2] scales {K, V}
    (NVFP4 global scales, FP8 per-tensor scales; unused for INT4)."""

    def __init__(self, fmt: int, num_pages: int, page_size: int, num_kv_heads: int, head_dim: int,
                 device="cuda", global_scale=(1.0, 1.0), pool: torch.Tensor | None = None, rotated: bool = False):
        self.fmt, self.num_pages, self.page_size = fmt, num_pages, page_size
        self.flags = FLAG_HADAMARD if rotated else 0
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.slab = kvq_slab_bytes(fmt, page_size, head_dim)
        if pool is None:
            pool = torch.empty((num_pages, num_kv_heads, self.slab), dtype=torch.uint8, device=device)
        self.pool = pool
        self.global_scale = torch.tensor(list(global_scale), dtype=torch.float32, device=pool.device)

    def desc(self) -> kvq_cache:
        return kvq_cache(self.fmt, self.num_pages, self.page_size, self.num_kv_heads, self.head_dim,
                         self.pool.data_ptr(), self.global_scale.data_ptr(), self.flags)


def _desc(cache):
    return ctypes.byref(cache.desc()) if isinstance(cache, Cache) else ctypes.byref(cache)


def kvq_quantize_store(cache: Cache, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, stream=None):
    """k, v: [n_tok][Hkv][D] (or [n_tok][>= Hkv*D] rows) fp32 or bf16 on the
    device, rows with unit stride inside a token; slot_mapping int32 [n_tok]."""
    n = slot_mapping.shape[0]
    dt = {torch.float32: DT_F32, torch.bfloat16: DT_BF16}[k.dtype]
    assert v.dtype == k.dtype and k.stride(0) == v.stride(0) and slot_mapping.dtype == torch.int32
    d = cache.desc()
    _check("kvq_quantize_store", lib().kvq_quantize_store(ctypes.byref(d), _ptr(k), _ptr(v), dt, k.stride(0),
                                                          _ptr(slot_mapping), n, _stream(stream)))


def kvq_decode_num_splits(cache: Cache, batch: int, num_q_heads: int, max_seq_len: int) -> int:
    out = ctypes.c_int32(0)
    d = cache.desc()
    _check("kvq_decode_num_splits", lib().kvq_decode_num_splits(ctypes.byref(d), batch, num_q_heads, max_seq_len,
                                                                ctypes.byref(out)))
    return int(out.value)


def kvq_decode_workspace_size(cache: Cache, batch: int, num_q_heads: int, max_seq_len: int,
                              num_splits: int = 0) -> int:
    out = ctypes.c_size_t(0)
    d = cache.desc()
    _check("kvq_decode_workspace_size", lib().kvq_decode_workspace_size(ctypes.byref(d), batch, num_q_heads,
                                                                        max_seq_len, num_splits, ctypes.byref(out)))
    return int(out.value)


def kvq_decode_attention(cache: Cache, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                         max_seq_len: int, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, sm_scale: float = 0.0, num_splits: int = 0,
                         out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """q: bf16 [B][Hq][D]; block_table int32 [B][max_pages]; seq_lens int32 [B].
    Returns out ([B][Hq][D], bf16 or fp32)."""
    B, Hq, D = q.shape
    assert q.dtype == torch.bfloat16 and q.is_contiguous()
    assert block_table.dtype == torch.int32 and block_table.is_contiguous() and seq_lens.dtype == torch.int32
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    odt = {torch.float32: DT_F32, torch.bfloat16: DT_BF16}[out.dtype]
    if workspace is None:
        nbytes = kvq_decode_workspace_size(cache, B, Hq, max_seq_len, num_splits)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    d = cache.desc()
    _check("kvq_decode_attention", lib().kvq_decode_attention(
        ctypes.byref(d), _ptr(q), Hq, _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B, int(max_seq_len),
        float(sm_scale), int(num_splits), _ptr(out), odt, _ptr(lse), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return out


def kvq_decode_attention_noalloc(cache: Cache, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                                 max_seq_len: int, out: torch.Tensor, lse: torch.Tensor | None = None,
                                 sm_scale: float = 0.0, num_splits: int = 0, stream=None) -> torch.Tensor:
    """kvq_decode_attention with the library's static scratch instead of a
    workspace: the caller passes every buffer (out bf16 or fp32 [B][Hq][D],
    optional lse fp32 [B][Hq]) and nothing is allocated."""
    B, Hq, D = q.shape
    assert q.dtype == torch.bfloat16 and q.is_contiguous()
    assert block_table.dtype == torch.int32 and block_table.is_contiguous() and seq_lens.dtype == torch.int32
    odt = {torch.float32: DT_F32, torch.bfloat16: DT_BF16}[out.dtype]
    d = cache.desc()
    _check("kvq_decode_attention_noalloc", lib().kvq_decode_attention_noalloc(
        ctypes.byref(d), _ptr(q), Hq, _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B, int(max_seq_len),
        float(sm_scale), int(num_splits), _ptr(out), odt, _ptr(lse), _stream(stream)))
    return out


def kvq_dequant_prefix(cache: Cache, block_table_row: torch.Tensor, prefix_len: int, k_out: torch.Tensor,
                       v_out: torch.Tensor, stream=None):
    """k_out, v_out: bf16 with rows of >= Hkv*D elements per token."""
    assert k_out.dtype == torch.bfloat16 and v_out.dtype == torch.bfloat16 and k_out.stride(0) == v_out.stride(0)
    assert block_table_row.dtype == torch.int32
    d = cache.desc()
    _check("kvq_dequant_prefix", lib().kvq_dequant_prefix(ctypes.byref(d), _ptr(block_table_row), int(prefix_len),
                                                          _ptr(k_out), _ptr(v_out), k_out.stride(0),
                                                          _stream(stream)))


def kvq_stream_read(buf: torch.Tensor, sink: torch.Tensor, num_workgroups: int = 0, stream=None):
    """Plain streaming read of a contiguous device tensor (bandwidth reference)."""
    assert buf.is_contiguous() and sink.dtype in (torch.int32, torch.uint32) and sink.numel() >= 1
    nbytes = buf.numel() * buf.element_size() // 16 * 16
    _check("kvq_stream_read", lib().kvq_stream_read(_ptr(buf), nbytes, _ptr(sink), int(num_workgroups),
                                                    _stream(stream)))


def kvq_stream_write(buf: torch.Tensor, value: int = 0, num_workgroups: int = 0, stream=None):
    """Plain streaming write over a contiguous device tensor (bandwidth reference)."""
    assert buf.is_contiguous()
    nbytes = buf.numel() * buf.element_size() // 16 * 16
    _check("kvq_stream_write", lib().kvq_stream_write(_ptr(buf), nbytes, int(value) & 0xFFFFFFFF,
                                                      int(num_workgroups), _stream(stream)))


def kvq_stream_copy(src: torch.Tensor, dst: torch.Tensor, num_workgroups: int = 0, stream=None):
    """Plain streaming copy between contiguous device tensors of equal size (bandwidth reference)."""
    assert src.is_contiguous() and dst.is_contiguous()
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == nbytes
    _check("kvq_stream_copy", lib().kvq_stream_copy(_ptr(src), _ptr(dst), nbytes // 16 * 16, int(num_workgroups),
                                                    _stream(stream)))


def kvq_mfma_rate(lds_operands: int, iterations: int, num_workgroups: int, sink: torch.Tensor, stream=None):
    """Matrix-core ceiling run: 16 v_mfma_f32_16x16x32_f16 per wavefront and iteration (16,384 flops each)
    in num_workgroups 768-thread workgroups; lds_operands = 1 reads each product's first operand from LDS in
    the QK form (16-byte reads), 2 alternates that with the PV form (two transposing 8-byte reads)."""
    assert sink.dtype in (torch.int32, torch.uint32) and sink.numel() >= 1
    _check("kvq_mfma_rate", lib().kvq_mfma_rate(int(lds_operands), int(iterations), int(num_workgroups), _ptr(sink),
                                                _stream(stream)))


def kvq_calibrate_amax(cache: Cache, k: torch.Tensor, v: torch.Tensor, running_amax: torch.Tensor, stream=None):
    """Raise running_amax (float32 [2] = {K, V}, zeroed before the first call) to max |k|, max |v|."""
    assert k.dtype == v.dtype and k.dtype in (torch.float32, torch.bfloat16) and k.stride() == v.stride()
    assert running_amax.dtype == torch.float32 and running_amax.numel() >= 2
    dt = 1 if k.dtype == torch.bfloat16 else 0
    d = cache.desc()
    _check("kvq_calibrate_amax", lib().kvq_calibrate_amax(ctypes.byref(d), _ptr(k), _ptr(v), dt, k.stride(0),
                                                          k.shape[0], _ptr(running_amax), _stream(stream)))


def kvq_calibrate_global_scale(cache: Cache, running_amax: torch.Tensor, stream=None):
    """cache.global_scale = running_amax / 2688 (1 where the amax is 0)."""
    assert running_amax.dtype == torch.float32 and running_amax.numel() >= 2
    d = cache.desc()
    _check("kvq_calibrate_global_scale", lib().kvq_calibrate_global_scale(ctypes.byref(d), _ptr(running_amax),
                                                                          _stream(stream)))


def kvq_hadamard_rotate(x: torch.Tensor, out: torch.Tensor | None = None, out_dtype: torch.dtype | None = None,
                        stream=None) -> torch.Tensor:
    """R x over the last axis (head_dim 128 or 256) of a device tensor whose
    rows are contiguous; returns out (same shape, out_dtype or x.dtype)."""
    D = x.shape[-1]
    xr = x.reshape(-1, D)
    assert xr.stride(1) == 1
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    orr = out.reshape(-1, D)
    dt = {torch.float32: DT_F32, torch.bfloat16: DT_BF16}
    _check("kvq_hadamard_rotate", lib().kvq_hadamard_rotate(_ptr(xr), dt[x.dtype], xr.stride(0), _ptr(orr),
                                                            dt[out.dtype], orr.stride(0), xr.shape[0], D,
                                                            _stream(stream)))
    return out


def kvq_extend_attention(q: torch.Tensor, k_ws: torch.Tensor, v_ws: torch.Tensor, prefix_len: int,
                         out: torch.Tensor | None = None, lse: torch.Tensor | None = None, sm_scale: float = 0.0,
                         out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """q: bf16 [n][Hq][D]; k_ws, v_ws: bf16 [>= prefix_len + n][Hkv][D] (or rows
    of >= Hkv*D elements).  Returns out [n][Hq][D]."""
    n, Hq, D = q.shape
    assert q.dtype == torch.bfloat16 and k_ws.dtype == torch.bfloat16 and v_ws.dtype == torch.bfloat16
    assert q.stride(2) == 1 and q.stride(1) == D and k_ws.stride(0) == v_ws.stride(0)
    Hkv = k_ws.shape[1] if k_ws.dim() == 3 else k_ws.shape[1] // D
    assert k_ws.shape[0] >= prefix_len + n
    if out is None:
        out = torch.empty((n, Hq, D), dtype=out_dtype, device=q.device)
    odt = {torch.float32: DT_F32, torch.bfloat16: DT_BF16}[out.dtype]
    if lse is not None:
        assert lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() >= n * Hq
    _check("kvq_extend_attention", lib().kvq_extend_attention(
        _ptr(q), q.stride(0), Hq, _ptr(k_ws), _ptr(v_ws), k_ws.stride(0), Hkv, D, int(prefix_len), n,
        float(sm_scale), _ptr(out), odt, out.stride(0), _ptr(lse) if lse is not None else None, _stream(stream)))
    return out


def kvq_extend_attention_paged(cache: Cache, block_table_row: torch.Tensor, prefix_len: int, q: torch.Tensor,
                               k_chunk: torch.Tensor, v_chunk: torch.Tensor, out: torch.Tensor | None = None,
                               lse: torch.Tensor | None = None, sm_scale: float = 0.0,
                               out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """Extend attention over [4-bit cached prefix | bf16 chunk]: q bf16 [n][Hq][D];
    k_chunk, v_chunk bf16 [n][Hkv][D] (or rows of >= Hkv*D elements)."""
    n, Hq, D = q.shape
    assert q.dtype == torch.bfloat16 and k_chunk.dtype == torch.bfloat16 and v_chunk.dtype == torch.bfloat16
    assert q.stride(2) == 1 and q.stride(1) == D and k_chunk.stride(0) == v_chunk.stride(0)
    assert k_chunk.shape[0] >= n and block_table_row.dtype == torch.int32
    if out is None:
        out = torch.empty((n, Hq, D), dtype=out_dtype, device=q.device)
    odt = {torch.float32: DT_F32, torch.bfloat16: DT_BF16}[out.dtype]
    if lse is not None:
        assert lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() >= n * Hq
    d = cache.desc()
    _check("kvq_extend_attention_paged", lib().kvq_extend_attention_paged(
        ctypes.byref(d), _ptr(block_table_row), int(prefix_len), _ptr(q), q.stride(0), Hq, _ptr(k_chunk),
        _ptr(v_chunk), k_chunk.stride(0), n, float(sm_scale), _ptr(out), odt, out.stride(0),
        _ptr(lse) if lse is not None else None, _stream(stream)))
    return out
