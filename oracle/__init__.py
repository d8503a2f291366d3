"""CPU oracle for the 4-bit paged KV cache (test infrastructure only).

This package is the slow, plainly written reference the HIP library is checked
against.  Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the product path (``bit_quantized_kv_amd``) never
does.  It shares no code with the HIP library: the arithmetic lives in
``kvq_oracle.c`` (plain C, fp32 quantization decisions, fp64 attention), built
with gcc into ``libkvq_oracle.so``, and this module only marshals numpy arrays.

Formats follow the pages "SGLang's 4-bit KV cache: the 56% is exact, the 1.78x
is untested" (Figure 2 caption; section "The 56% survives its own scale, and
names the block size") for NVFP4 and "KV cache in 4 bits: 8.8 instead of 4.7
full sessions on the same four RTX 5090s" (section "What we changed") for the
INT4 per-token-head cache; the FP8 E4M3 per-tensor-scaled cache is the
comparator the first page measures NVFP4 against (section "The 56% survives
its own scale, and names the block size").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

NVFP4 = 1
INT4 = 2
FP8 = 3  # E4M3 with one FP32 scale per tensor: the comparator format
K8V4 = 4  # FP8 (E4M3, per-tensor scale) keys with NVFP4 values

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
# KVQ_ORACLE_LIB names another build of the same source to load instead (the
# test that plants mistakes in copies of the oracle loads each copy this way)
_OTHER_LIB = os.environ.get("KVQ_ORACLE_LIB")
_LIB_PATH = _OTHER_LIB or os.path.join(_HERE, "libkvq_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE fp32/fp64: no fast-math, no FMA
    contraction) and return the path of the shared library."""
    if _OTHER_LIB:
        return _LIB_PATH  # a build made elsewhere: never overwritten from this source
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    compile_source(_SRC, _LIB_PATH + ".tmp")
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def compile_source(src: str, out: str) -> None:
    """gcc of one oracle source file into a shared library, with the flags the
    oracle is always built with."""
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32, f64, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
    sig = {
        "kvqo_e2m1_value": (f64, [i32]),
        "kvqo_e4m3_value": (f64, [i32]),
        "kvqo_e2m1_encode": (i32, [f32]),
        "kvqo_e4m3_encode": (i32, [f32]),
        "kvqo_bf16_rne": (ctypes.c_uint16, [f32]),
        "kvqo_nvfp4_quantize_row": (None, [P, i32, f32, P, P]),
        "kvqo_int4_quantize_row": (None, [P, i32, P, P]),
        "kvqo_nvfp4_dequant_row": (None, [P, P, i32, f32, P]),
        "kvqo_int4_dequant_row": (None, [P, f32, i32, P]),
        "kvqo_slab_bytes": (sz, [i32, i32, i32]),
        "kvqo_token_head_bytes": (sz, [i32, i32]),
        "kvqo_quantize_store": (None, [i32, P, i32, i32, i32, P, P, P, i32, P, i32]),
        "kvqo_hadamard_row": (None, [P, i32]),
        "kvqo_extend_attention": (None, [P, i64, i32, P, P, i64, i32, i32, i64, i64, f64, P, P]),
        "kvqo_extend_attention_paged": (None, [i32, P, i32, i32, i32, P, P, i64, P, i64, i32, P, i64, P, P, i64,
                                               f64, P, P, P]),
        "kvqo_decode_attention": (None, [i32, P, i32, i32, i32, P, P, i32, P, i32, P, i32, f64, i64, P, P]),
        "kvqo_dequant_prefix": (None, [i32, P, i32, i32, i32, P, P, i64, P, P, i64]),
        "kvqo_num_threads": (i32, []),
        "kvqo_set_num_threads": (None, [i32]),
        "kvqo_amax": (f32, [P, i64]),
        "kvqo_fp8_encode": (i32, [f32, f32]),
        "kvqo_global_scale": (f32, [f32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


# ---------------------------------------------------------------- codecs

def e2m1_value(code: int) -> float:
    return _load().kvqo_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return _load().kvqo_e4m3_value(int(code))


def e2m1_encode(r: float) -> int:
    return _load().kvqo_e2m1_encode(float(np.float32(r)))


def e4m3_encode(s: float) -> int:
    return _load().kvqo_e4m3_encode(float(np.float32(s)))


def bf16_rne(x: float) -> int:
    return _load().kvqo_bf16_rne(float(np.float32(x)))


def nvfp4_quantize_row(x, gs: float = 1.0):
    """One row of D fp32 values -> (codes uint8[D/2], scale codes uint8[D/16])."""
    x = _f32(x)
    D = x.shape[0]
    codes = np.zeros(D // 2, np.uint8)
    scales = np.zeros(D // 16, np.uint8)
    _load().kvqo_nvfp4_quantize_row(_ptr(x), D, float(np.float32(gs)), _ptr(codes), _ptr(scales))
    return codes, scales


def int4_quantize_row(x):
    """One row of D fp32 values -> (codes uint8[D/2], fp32 scale)."""
    x = _f32(x)
    D = x.shape[0]
    codes = np.zeros(D // 2, np.uint8)
    s = np.zeros(1, np.float32)
    _load().kvqo_int4_quantize_row(_ptr(x), D, _ptr(codes), _ptr(s))
    return codes, np.float32(s[0])


def nvfp4_dequant_row(codes, scales, gs: float = 1.0) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    D = codes.shape[0] * 2
    out = np.zeros(D, np.float64)
    _load().kvqo_nvfp4_dequant_row(_ptr(codes), _ptr(scales), D, float(np.float32(gs)), _ptr(out))
    return out


def int4_dequant_row(codes, scale) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    D = codes.shape[0] * 2
    out = np.zeros(D, np.float64)
    _load().kvqo_int4_dequant_row(_ptr(codes), float(np.float32(scale)), D, _ptr(out))
    return out


# ---------------------------------------------------------------- pool level

def amax(x) -> float:
    """Largest |x| (the running maximum a calibration pass keeps)."""
    a = _f32(np.ascontiguousarray(x).ravel())
    return float(_load().kvqo_amax(_ptr(a), a.size))


def hadamard(x) -> np.ndarray:
    """R x for every row of x (fp32, last axis D): R = H_D / sqrt(D), the fast
    transform's stages in order, the scale applied last (see kvqo_hadamard_row)."""
    a = _f32(x).copy()
    D = a.shape[-1]
    rows = a.reshape(-1, D)
    for r in rows:
        _load().kvqo_hadamard_row(r.ctypes.data_as(ctypes.c_void_p), D)
    return rows.reshape(a.shape)


def extend_attention(q, k_ws, v_ws, prefix_len: int, sm_scale: float | None = None):
    """Chunk queries q [n][Hq][D] over workspace rows k_ws, v_ws [>= prefix_len + n][Hkv][D]
    (bf16 values widened to fp32), query i seeing keys 0 .. prefix_len + i.
    Returns (out fp64 [n][Hq][D], lse fp64 [n][Hq])."""
    q, k, v = _f32(q), _f32(k_ws), _f32(v_ws)
    n, Hq, D = q.shape
    Hkv = k.shape[1]
    assert k.shape == v.shape and k.shape[2] == D and k.shape[0] >= prefix_len + n and Hq % Hkv == 0
    if sm_scale is None or sm_scale <= 0:
        sm_scale = 1.0 / np.sqrt(D)
    out = np.zeros((n, Hq, D), np.float64)
    lse = np.zeros((n, Hq), np.float64)
    _load().kvqo_extend_attention(_ptr(q), Hq * D, Hq, _ptr(k), _ptr(v), Hkv * D, Hkv, D, int(prefix_len), n,
                                  float(sm_scale), _ptr(out), _ptr(lse))
    return out, lse


def fp8_encode(x: float, scale: float) -> int:
    """FP8 (E4M3, per-tensor scale) code of x: E4M3 of fp32(x / scale), sign kept."""
    return int(_load().kvqo_fp8_encode(float(x), float(scale)))


def global_scale(amax_value: float) -> float:
    """NVFP4 per-layer global scale from a calibrated amax: fp32(amax / 2688)."""
    return float(_load().kvqo_global_scale(float(amax_value)))


def slab_bytes(fmt: int, page_size: int, head_dim: int) -> int:
    return int(_load().kvqo_slab_bytes(fmt, page_size, head_dim))


def token_head_bytes(fmt: int, head_dim: int) -> int:
    return int(_load().kvqo_token_head_bytes(fmt, head_dim))


class Pool:
    """One layer's paged cache on the host: uint8 [num_pages][Hkv][slab]."""

    def __init__(self, fmt: int, num_pages: int, page_size: int, num_kv_heads: int, head_dim: int,
                 global_scale=(1.0, 1.0), fill: int = 0, rotated: bool = False):
        self.fmt, self.num_pages, self.page_size = fmt, num_pages, page_size
        self.rotated = bool(rotated)  # rows Hadamard-rotated before quantization
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.slab = slab_bytes(fmt, page_size, head_dim)
        self.data = np.full((num_pages, num_kv_heads, self.slab), fill, np.uint8)
        self.gs = _f32(global_scale).reshape(2)

    def quantize_store(self, k, v, slot_mapping):
        """k, v: [n_tok][Hkv][D] (fp32, or bf16 values already widened)."""
        k, v, slots = _f32(k), _f32(v), _i32(slot_mapping)
        n = slots.shape[0]
        assert k.shape == (n, self.num_kv_heads, self.head_dim) and v.shape == k.shape
        _load().kvqo_quantize_store(self.fmt, _ptr(self.data), self.page_size, self.num_kv_heads, self.head_dim,
                                    _ptr(self.gs), _ptr(k), _ptr(v), n, _ptr(slots), int(self.rotated))

    def decode_attention(self, q, block_table, seq_lens, sm_scale: float | None = None, split_tokens: int = 0):
        """q: [B][Hq][D] (bf16 values widened to fp32).  Returns (out fp64
        [B][Hq][D], lse fp64 [B][Hq])."""
        q, bt, sl = _f32(q), _i32(block_table), _i32(seq_lens)
        B, Hq, D = q.shape
        assert D == self.head_dim and bt.shape[0] == B and sl.shape == (B,)
        if sm_scale is None or sm_scale <= 0:
            sm_scale = 1.0 / np.sqrt(D)
        out = np.zeros((B, Hq, D), np.float64)
        lse = np.zeros((B, Hq), np.float64)
        _load().kvqo_decode_attention(self.fmt, _ptr(self.data), self.page_size, self.num_kv_heads, D, _ptr(self.gs),
                                      _ptr(q), Hq, _ptr(bt), bt.shape[1], _ptr(sl), B, float(sm_scale),
                                      int(split_tokens), _ptr(out), _ptr(lse))
        return out, lse

    def extend_attention(self, q, pages, prefix_len: int, k_chunk, v_chunk, q_pos=None,
                         sm_scale: float | None = None, want_abs: bool = False):
        """Extend attention over [this pool's cached prefix | bf16 chunk rows]
        with the prefix at its exact dequantized value (kvqo_extend_attention_paged).
        q: [n_q][Hq][D]; pages: the sequence's page list; k_chunk, v_chunk:
        [chunk rows][Hkv][D] (bf16 values widened to fp32); q_pos: the sequence
        position of each query row (default prefix_len + row).  Returns (out
        fp64 [n_q][Hq][D], lse fp64 [n_q][Hq]) and, with want_abs, the
        softmax-weighted mean of |v| per output element as a third array."""
        q, pages = _f32(q), _i32(pages)
        kc, vc = _f32(k_chunk), _f32(v_chunk)
        n, Hq, D = q.shape
        Hkv = self.num_kv_heads
        assert D == self.head_dim and Hq % Hkv == 0 and kc.shape == vc.shape and kc.shape[1:] == (Hkv, D)
        pos = np.arange(prefix_len, prefix_len + n, dtype=np.int64) if q_pos is None else \
            np.ascontiguousarray(np.asarray(q_pos, dtype=np.int64))
        assert pos.shape == (n,) and np.all(pos >= prefix_len) and np.all(pos < prefix_len + kc.shape[0])
        assert pages.shape[0] * self.page_size >= prefix_len
        if sm_scale is None or sm_scale <= 0:
            sm_scale = 1.0 / np.sqrt(D)
        out = np.zeros((n, Hq, D), np.float64)
        lse = np.zeros((n, Hq), np.float64)
        oabs = np.zeros((n, Hq, D), np.float64) if want_abs else None
        _load().kvqo_extend_attention_paged(self.fmt, _ptr(self.data), self.page_size, Hkv, D, _ptr(self.gs),
                                            _ptr(pages), int(prefix_len), _ptr(q), Hq * D, Hq, _ptr(pos), n,
                                            _ptr(kc), _ptr(vc), Hkv * D, float(sm_scale), _ptr(out), _ptr(lse),
                                            _ptr(oabs) if want_abs else None)
        return (out, lse, oabs) if want_abs else (out, lse)

    def dequant_prefix(self, pages, prefix_len: int, out_token_stride: int | None = None):
        """Returns (k_out, v_out) as uint16 bf16 bit patterns [prefix_len][Hkv][D]
        (or [prefix_len][out_token_stride] when a wider stride is given)."""
        if self.fmt in (FP8, K8V4):
            raise ValueError("the FP8-keyed formats have no prefix dequantization")
        pages = _i32(pages)
        Hkv, D = self.num_kv_heads, self.head_dim
        stride = out_token_stride or Hkv * D
        k_out = np.zeros((prefix_len, stride), np.uint16)
        v_out = np.zeros((prefix_len, stride), np.uint16)
        _load().kvqo_dequant_prefix(self.fmt, _ptr(self.data), self.page_size, Hkv, D, _ptr(self.gs), _ptr(pages),
                                    int(prefix_len), _ptr(k_out), _ptr(v_out), int(stride))
        if out_token_stride is None:
            return k_out.reshape(prefix_len, Hkv, D), v_out.reshape(prefix_len, Hkv, D)
        return k_out, v_out

    def dequant_token(self, page: int, g: int, off: int, kv: int) -> np.ndarray:
        """Exact fp64 value of one stored row (kv 0 = K, 1 = V)."""
        P, D = self.page_size, self.head_dim
        slab = self.data[page, g]
        if self.fmt == FP8:
            codes = slab[off * D:(off + 1) * D] if kv == 0 else slab[P * D + off::P][:D]
            return np.array([e4m3_value(int(c)) for c in codes]) * float(self.gs[kv])
        if self.fmt == K8V4:
            if kv == 0:
                return np.array([e4m3_value(int(c)) for c in slab[off * D:(off + 1) * D]]) * float(self.gs[0])
            vsec = slab[P * D:]
            sc0 = P * (D // 2) + off * (D // 16)
            return nvfp4_dequant_row(vsec[off * (D // 2):(off + 1) * (D // 2)], vsec[sc0:sc0 + D // 16],
                                     float(self.gs[1]))
        half = slab[: self.slab // 2] if kv == 0 else slab[self.slab // 2:]
        codes = half[off * (D // 2):(off + 1) * (D // 2)]
        if self.fmt == NVFP4:
            sc0 = P * (D // 2) + off * (D // 16)
            return nvfp4_dequant_row(codes, half[sc0:sc0 + D // 16], float(self.gs[kv]))
        sc0 = P * (D // 2) + off * 4
        return int4_dequant_row(codes, half[sc0:sc0 + 4].view(np.float32)[0])


def num_threads() -> int:
    return int(_load().kvqo_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops (for timing; results do not depend on it)."""
    _load().kvqo_set_num_threads(int(n))
