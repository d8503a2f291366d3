"""The C ABI on the CPU: the library loads, exports every entry point the
header declares, sizes its buffers as the formats dictate, and rejects bad
arguments before any launch (no GPU is touched by these tests)."""
import ctypes
import os
import re

import pytest

from bit_quantized_kv_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvq.LIB_PATH):
        from bit_quantized_kv_amd import build
        build.build()
    return kvq.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"kvq_quantize_store", "kvq_decode_attention", "kvq_dequant_prefix"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_slab_bytes_match_oracle_and_pages(lib, oracle):
    for fmt in (1, 2):
        for P in (16, 48, 800, 1600):
            for D in (128, 256):
                assert kvq.kvq_slab_bytes(fmt, P, D) == oracle.slab_bytes(fmt, P, D)
    assert kvq.kvq_slab_bytes(2, 1600, 256) == 422400
    assert kvq.kvq_slab_bytes(2, 800, 256) == 211200
    assert kvq.kvq_slab_bytes(1, 16, 256) == 16 * 2 * (128 + 16)
    assert kvq.kvq_slab_bytes(7, 16, 256) == 0


FAKE = 0x10000  # a 16-byte-aligned host address that is never dereferenced


def cache(fmt=1, pages=64, P=16, H=4, D=256, pool=FAKE, gs=FAKE):
    return kvq.kvq_cache(fmt, pages, P, H, D, pool, gs)


def q_store(lib, c, k=FAKE, v=FAKE, dt=1, stride=1024, slots=FAKE, n=4):
    return lib.kvq_quantize_store(ctypes.byref(c), k, v, dt, stride, slots, n, None)


def test_quantize_store_validation(lib):
    assert lib.kvq_quantize_store(None, FAKE, FAKE, 1, 1024, FAKE, 4, None) == ERR_NULL
    assert q_store(lib, cache(pool=0)) == ERR_NULL
    assert q_store(lib, cache(gs=0)) == ERR_NULL            # NVFP4 needs global scales
    assert q_store(lib, cache(fmt=7)) == ERR_UNSUPPORTED
    assert q_store(lib, cache(D=64)) == ERR_UNSUPPORTED
    assert q_store(lib, cache(P=24)) == ERR_UNSUPPORTED
    assert q_store(lib, cache(pages=0)) == ERR_SHAPE
    assert q_store(lib, cache(pool=FAKE + 8)) == ERR_ALIGN
    assert q_store(lib, cache(), dt=7) == ERR_UNSUPPORTED
    assert q_store(lib, cache(), n=-1) == ERR_SHAPE
    assert q_store(lib, cache(), k=0) == ERR_NULL
    assert q_store(lib, cache(), slots=0) == ERR_NULL
    assert q_store(lib, cache(), stride=1000) == ERR_SHAPE     # < Hkv * D
    assert q_store(lib, cache(), stride=1028) == ERR_ALIGN     # 2056 bytes
    assert q_store(lib, cache(), k=FAKE + 2) == ERR_ALIGN
    # INT4 ignores the global scale; zero tokens is a no-op before any launch
    assert q_store(lib, cache(fmt=2, gs=0), n=0) == OK
    assert q_store(lib, cache(), n=0) == OK


def decode(lib, c, q=FAKE, hq=24, bt=FAKE, maxp=2048, sl=FAKE, B=32, L=32768, ns=0, out=FAKE, odt=1, lse=None,
           ws=FAKE, wsb=1 << 40):
    return lib.kvq_decode_attention(ctypes.byref(c), q, hq, bt, maxp, sl, B, L, 0.0, ns, out, odt, lse, ws, wsb, None)


def test_decode_validation(lib):
    c = cache()
    assert decode(lib, c, q=0) == ERR_NULL
    assert decode(lib, c, ws=0) == ERR_NULL
    assert decode(lib, c, hq=26) == ERR_SHAPE                  # not a multiple of Hkv
    assert decode(lib, c, hq=4 * 17) == ERR_UNSUPPORTED        # group of 17
    assert decode(lib, c, maxp=100) == ERR_SHAPE               # table too short for max_seq_len
    assert decode(lib, c, odt=5) == ERR_UNSUPPORTED
    assert decode(lib, c, out=FAKE + 4) == ERR_ALIGN
    assert decode(lib, c, lse=FAKE + 2) == ERR_ALIGN
    assert decode(lib, c, B=0) == ERR_SHAPE
    assert decode(lib, c, L=-1) == ERR_SHAPE
    assert decode(lib, c, wsb=16) == ERR_WORKSPACE
    assert decode(lib, cache(D=96)) == ERR_UNSUPPORTED


def decode_noalloc(lib, c, q=FAKE, hq=24, bt=FAKE, maxp=2048, sl=FAKE, B=32, L=32768, ns=0, out=FAKE, odt=1,
                   lse=None):
    return lib.kvq_decode_attention_noalloc(ctypes.byref(c), q, hq, bt, maxp, sl, B, L, 0.0, ns, out, odt, lse, None)


def test_decode_noalloc_validation(lib):
    """The no-allocation decode checks its arguments like kvq_decode_attention
    and refuses, before touching any device, a shape whose split partials need
    more than its 16 MiB static scratch."""
    c = cache()
    assert decode_noalloc(lib, c, q=0) == ERR_NULL
    assert decode_noalloc(lib, c, out=0) == ERR_NULL
    assert decode_noalloc(lib, c, hq=26) == ERR_SHAPE
    assert decode_noalloc(lib, c, hq=4 * 17) == ERR_UNSUPPORTED
    assert decode_noalloc(lib, c, maxp=100) == ERR_SHAPE
    assert decode_noalloc(lib, c, odt=5) == ERR_UNSUPPORTED
    assert decode_noalloc(lib, c, out=FAKE + 4) == ERR_ALIGN
    assert decode_noalloc(lib, cache(D=96)) == ERR_UNSUPPORTED
    size = ctypes.c_size_t(0)
    # 4096 sequences x 4 KV heads x 6 query heads x (256 + 2) floats: 101 MB of partials
    assert lib.kvq_decode_workspace_size(ctypes.byref(c), 4096, 24, 32768, 1, ctypes.byref(size)) == OK
    assert size.value > 16 << 20
    assert decode_noalloc(lib, c, B=4096, ns=1, maxp=2048) == ERR_SCRATCH
    # 256 splits of one sequence: 6.3 MB, within the scratch -- but a 70,000-split plan is not
    assert decode_noalloc(lib, c, B=1, ns=70000, L=1 << 22, maxp=1 << 18) == ERR_UNSUPPORTED
    assert decode_noalloc(lib, c, B=1, ns=4096, L=1 << 22, maxp=1 << 18) == ERR_SCRATCH


def test_workspace_and_split_plan(lib):
    c = cache()
    splits = ctypes.c_int32(0)
    size = ctypes.c_size_t(0)
    assert lib.kvq_decode_num_splits(ctypes.byref(c), 32, 24, 32768, ctypes.byref(splits)) == OK
    S = splits.value
    assert 2 <= S <= 3                                         # about one 4-wave workgroup per CU
    assert lib.kvq_decode_workspace_size(ctypes.byref(c), 32, 24, 32768, 0, ctypes.byref(size)) == OK
    assert size.value == 32 * 4 * S * 6 * (256 + 2) * 4
    assert lib.kvq_decode_workspace_size(ctypes.byref(c), 2, 8, 100, 3, ctypes.byref(size)) == OK
    assert size.value == 2 * 4 * 3 * 2 * (256 + 2) * 4
    # each of a split's 4 wavefronts gets at least 4 chunks (128 tokens)
    assert lib.kvq_decode_num_splits(ctypes.byref(c), 1, 4, 200, ctypes.byref(splits)) == OK
    assert splits.value == 1
    assert lib.kvq_decode_num_splits(ctypes.byref(c), 1, 4, 4096, ctypes.byref(splits)) == OK
    assert splits.value == 8
    assert lib.kvq_decode_num_splits(ctypes.byref(c), 1, 4, 0, ctypes.byref(splits)) == OK
    assert splits.value == 1
    assert lib.kvq_decode_num_splits(ctypes.byref(c), 1, 4, 10, None) == ERR_NULL
    # a wavefront sums at most 256 chunks (8,192 tokens) into its accumulators:
    # 1,024 sequences x 4 heads at 1M tokens need 32 splits of 4 wavefronts
    assert lib.kvq_decode_num_splits(ctypes.byref(c), 1024, 24, 1 << 20, ctypes.byref(splits)) == OK
    assert splits.value == 32
    assert lib.kvq_decode_num_splits(ctypes.byref(c), 32, 24, 1 << 20, ctypes.byref(splits)) == OK
    assert -(-(1 << 15) // splits.value) <= 4 * 256


def test_dequant_prefix_validation(lib):
    c = cache()
    f = lib.kvq_dequant_prefix
    assert f(ctypes.byref(c), FAKE, 0, FAKE, FAKE, 1024, None) == OK
    assert f(ctypes.byref(c), FAKE, -1, FAKE, FAKE, 1024, None) == ERR_SHAPE
    assert f(ctypes.byref(c), 0, 16, FAKE, FAKE, 1024, None) == ERR_NULL
    assert f(ctypes.byref(c), FAKE, 16, FAKE, 0, 1024, None) == ERR_NULL
    assert f(ctypes.byref(c), FAKE, 16, FAKE, FAKE, 512, None) == ERR_SHAPE
    assert f(ctypes.byref(c), FAKE, 16, FAKE, FAKE, 1028, None) == ERR_ALIGN
    assert f(ctypes.byref(c), FAKE, 16, FAKE + 8, FAKE, 1024, None) == ERR_ALIGN


def test_status_strings(lib):
    for s in (OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH):
        assert kvq.status_string(s) and kvq.status_string(s) != "unknown status"
    assert kvq.status_string(42) == "unknown status"
    assert lib.kvq_last_hip_error() == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kvq, "_lib", None)
    monkeypatch.setattr(kvq, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        kvq.lib()


def test_stream_read_validation(lib):
    assert lib.kvq_stream_read(None, 0, None, 0, None) == OK  # nothing to read
    assert lib.kvq_stream_read(None, 64, FAKE, 0, None) == ERR_NULL
    assert lib.kvq_stream_read(FAKE, 64, None, 0, None) == ERR_NULL
    assert lib.kvq_stream_read(FAKE + 8, 64, FAKE, 0, None) == ERR_ALIGN
    assert lib.kvq_stream_read(FAKE, 60, FAKE, 0, None) == ERR_ALIGN
    assert lib.kvq_stream_read(FAKE, 64, FAKE + 2, 0, None) == ERR_ALIGN


def test_mfma_rate_validation(lib):
    f = lib.kvq_mfma_rate
    assert f(0, 10, 4, None, None) == ERR_NULL
    assert f(3, 10, 4, FAKE, None) == ERR_UNSUPPORTED
    assert f(-1, 10, 4, FAKE, None) == ERR_UNSUPPORTED
    assert f(2, 0, 4, FAKE, None) == ERR_SHAPE
    assert f(1, 0, 4, FAKE, None) == ERR_SHAPE
    assert f(1, 10, 0, FAKE, None) == ERR_SHAPE


def test_calibration_validation(lib):
    c = cache()
    f = lib.kvq_calibrate_amax
    assert f(ctypes.byref(c), FAKE, FAKE, 1, 1024, 0, FAKE, None) == OK          # no tokens
    assert f(ctypes.byref(c), FAKE, FAKE, 1, 1024, -1, FAKE, None) == ERR_SHAPE
    assert f(ctypes.byref(c), FAKE, FAKE, 1, 1024, 4, None, None) == ERR_NULL
    assert f(ctypes.byref(c), 0, FAKE, 1, 1024, 4, FAKE, None) == ERR_NULL
    assert f(ctypes.byref(c), FAKE, FAKE, 1, 512, 4, FAKE, None) == ERR_SHAPE     # stride < Hkv * D
    assert f(ctypes.byref(c), FAKE, FAKE, 1, 1028, 4, FAKE, None) == ERR_ALIGN
    assert f(ctypes.byref(c), FAKE, FAKE, 1, 1024, 4, FAKE + 2, None) == ERR_ALIGN
    assert f(ctypes.byref(c), FAKE, FAKE, 7, 1024, 4, FAKE, None) == ERR_UNSUPPORTED
    c4 = cache(fmt=2, gs=0)
    assert f(ctypes.byref(c4), FAKE, FAKE, 1, 1024, 4, FAKE, None) == ERR_UNSUPPORTED  # INT4 has no global scale
    g = lib.kvq_calibrate_global_scale
    assert g(ctypes.byref(c), None, None) == ERR_NULL
    assert g(ctypes.byref(c4), FAKE, None) == ERR_UNSUPPORTED
    assert g(ctypes.byref(c), FAKE + 1, None) == ERR_ALIGN


def test_fp8_comparator_format(lib, oracle):
    for P in (16, 48):
        for D in (128, 256):
            assert kvq.kvq_slab_bytes(3, P, D) == oracle.slab_bytes(3, P, D) == 2 * P * D
    c = cache(fmt=3)
    assert lib.kvq_dequant_prefix(ctypes.byref(c), FAKE, 16, FAKE, FAKE, 1024, None) == ERR_UNSUPPORTED
    assert lib.kvq_calibrate_amax(ctypes.byref(c), FAKE, FAKE, 1, 1024, 4, FAKE, None) == ERR_UNSUPPORTED
    c0 = cache(fmt=3, gs=0)
    assert q_store(lib, c0) == ERR_NULL                      # the per-tensor scales are required
    assert q_store(lib, c, n=0) == OK


def test_k8v4_format(lib, oracle):
    for P in (16, 48, 1600):
        for D in (128, 256):
            assert kvq.kvq_slab_bytes(4, P, D) == oracle.slab_bytes(4, P, D) == P * (D + D // 2 + D // 16)
    c = cache(fmt=4)
    assert lib.kvq_dequant_prefix(ctypes.byref(c), FAKE, 16, FAKE, FAKE, 1024, None) == ERR_UNSUPPORTED
    assert lib.kvq_calibrate_amax(ctypes.byref(c), FAKE, FAKE, 1, 1024, 4, FAKE, None) == ERR_UNSUPPORTED
    assert lib.kvq_extend_attention_paged(ctypes.byref(c), FAKE, 100, FAKE, 24 * 256, 24, FAKE, FAKE, 4 * 256, 8,
                                          0.0, FAKE, 1, 24 * 256, None, None) == ERR_UNSUPPORTED
    c0 = cache(fmt=4, gs=0)
    assert q_store(lib, c0) == ERR_NULL                      # the key and value scales are required
    assert q_store(lib, c, n=0) == OK


def test_rotation_flag_and_rotate_validation(lib):
    c = cache()
    c.flags = 2                                                   # unknown flag bit
    assert q_store(lib, c) == ERR_UNSUPPORTED
    c.flags = kvq.FLAG_HADAMARD
    assert q_store(lib, c, n=0) == OK
    f = lib.kvq_hadamard_rotate
    assert f(FAKE, 1, 256, FAKE, 0, 256, 0, 256, None) == OK        # no rows
    assert f(FAKE, 1, 256, FAKE, 0, 256, -1, 256, None) == ERR_SHAPE
    assert f(FAKE, 1, 256, FAKE, 0, 256, 4, 64, None) == ERR_UNSUPPORTED
    assert f(FAKE, 5, 256, FAKE, 0, 256, 4, 256, None) == ERR_UNSUPPORTED
    assert f(None, 1, 256, FAKE, 0, 256, 4, 256, None) == ERR_NULL
    assert f(FAKE, 1, 128, FAKE, 0, 256, 4, 256, None) == ERR_SHAPE
    assert f(FAKE, 1, 260, FAKE, 0, 260, 4, 256, None) == ERR_ALIGN
    assert f(FAKE + 4, 1, 256, FAKE, 0, 256, 4, 256, None) == ERR_ALIGN


def test_extend_attention_validation(lib):
    f = lib.kvq_extend_attention
    ok = (FAKE, 24 * 256, 24, FAKE, FAKE, 4 * 256, 4, 256, 100, 0, 0.0, FAKE, 1, 24 * 256, None, None)
    assert f(*ok) == OK                                           # empty chunk
    a = list(ok)
    a[9] = 8
    args = list(a)
    args[0] = None
    assert f(*args) == ERR_NULL
    args = list(a)
    args[2] = 25
    assert f(*args) == ERR_SHAPE                                  # Hq not a multiple of Hkv
    args = list(a)
    args[7] = 64
    assert f(*args) == ERR_UNSUPPORTED
    args = list(a)
    args[5] = 4 * 256 - 8
    assert f(*args) == ERR_SHAPE
    args = list(a)
    args[1] = 24 * 256 + 4
    assert f(*args) == ERR_ALIGN
    args = list(a)
    args[12] = 9
    assert f(*args) == ERR_UNSUPPORTED
    args = list(a)
    args[8] = -1
    assert f(*args) == ERR_SHAPE


def test_extend_attention_paged_validation(lib):
    f = lib.kvq_extend_attention_paged
    c = cache()
    ok = [ctypes.byref(c), FAKE, 100, FAKE, 24 * 256, 24, FAKE, FAKE, 4 * 256, 0, 0.0, FAKE, 1, 24 * 256, None, None]
    assert f(*ok) == OK                                           # empty chunk
    a = list(ok)
    a[9] = 8
    for i, v, want in [(1, None, ERR_NULL),                       # a prefix needs its page list
                       (3, None, ERR_NULL), (6, None, ERR_NULL), (11, None, ERR_NULL),
                       (5, 25, ERR_SHAPE),                        # Hq not a multiple of Hkv
                       (2, -1, ERR_SHAPE), (8, 4 * 256 - 8, ERR_SHAPE), (4, 24 * 256 - 8, ERR_SHAPE),
                       (3, FAKE + 4, ERR_ALIGN), (4, 24 * 256 + 4, ERR_ALIGN),
                       (12, 9, ERR_UNSUPPORTED)]:
        args = list(a)
        args[i] = v
        assert f(*args) == want, (i, v, want)
    args = list(a)
    args[1], args[2] = None, 0                                    # no prefix: no page list needed
    args[9] = 0
    assert f(*args) == OK
    fp8 = cache(fmt=3)
    args = list(a)
    args[0] = ctypes.byref(fp8)
    assert f(*args) == ERR_UNSUPPORTED                            # the FP8 comparator has no fused extend
    bad = cache(fmt=7)
    args = list(a)
    args[0] = ctypes.byref(bad)
    assert f(*args) != OK
    huge = cache(P=16 * 1024 * 1024)                              # a slab past 2^31 bytes
    args = list(a)
    args[0] = ctypes.byref(huge)
    assert f(*args) == ERR_UNSUPPORTED
