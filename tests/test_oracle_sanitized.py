"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) runs every entry point -- quantize-store, decode with
splits, prefix dequantization, workspace and paged extend, the row codecs,
the rotation -- for all four formats, plain and rotated, with skipped slots
and an empty sequence, in a subprocess: no sanitizer report, and outputs
identical to those of the regular build of the same source."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from bit_quantized_kv_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
D, HKV, HQ, P, NTOK, B, MAXP, NPAGES, NC, LP = 64, 2, 6, 16, 65, 3, 3, 11, 9, 45


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tmp_path_factory.mktemp("oracle_asan")
    exe = str(d / "oracle_asan")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(HERE, "oracle_sanitize_main.c"), os.path.join(ROOT, "oracle", "kvq_oracle.c"),
           "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return d, exe


def test_oracle_under_address_and_undefined_behaviour_sanitizers(sanitized):
    d, exe = sanitized
    k, v = inputs.kv_outlier_channels(61, 0, NTOK, HKV, D)
    q = inputs.query(61, 1, B, HQ, D)
    bt = inputs.page_tables(61, B, MAXP, NPAGES, shuffled=True)
    lens = np.array([LP, 20, 0], np.int32)
    slots = np.concatenate([inputs.slots_for(bt, P, 0, 0, LP), inputs.slots_for(bt, P, 1, 0, 20)]).astype(np.int32)
    slots[10] = -1                                   # a skipped token keeps the fill bytes
    gs = np.array([0.5, 2.0], np.float32)
    kc, vc = inputs.kv_lognormal_channels(62, 0, NC, HKV, D)
    qe = inputs.query(62, 1, NC, HQ, D).reshape(NC, HQ, D)
    for name, a in (("k", k), ("v", v), ("q", q), ("slots", slots), ("bt", bt), ("lens", lens), ("gs", gs),
                    ("kc", kc), ("vc", vc), ("qe", qe)):
        np.ascontiguousarray(a).tofile(str(d / f"{name}.bin"))
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")
    r = subprocess.run([exe, str(d)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]

    def out(name, dtype):
        return np.fromfile(str(d / f"out_{name}.bin"), dtype=dtype)

    for fmt in (1, 2, 3, 4):
        for rot in (0, 1):
            pool = oracle.Pool(fmt, NPAGES, P, HKV, D, global_scale=gs, fill=0x11, rotated=bool(rot))
            pool.quantize_store(k, v, slots)
            assert np.array_equal(out(f"pool_{fmt}_{rot}", np.uint8), pool.data.ravel()), (fmt, rot)
            o, lse = pool.decode_attention(q, bt, lens, sm_scale=0.125, split_tokens=7)
            assert np.array_equal(out(f"dec_o_{fmt}_{rot}", np.float64), o.ravel()), (fmt, rot)
            assert np.array_equal(out(f"dec_lse_{fmt}_{rot}", np.float64), lse.ravel()), (fmt, rot)
            if fmt <= 2:
                kq, vq = pool.dequant_prefix(bt[0], LP)
                assert np.array_equal(out(f"dq_k_{fmt}_{rot}", np.uint16), kq.ravel())
                assert np.array_equal(out(f"dq_v_{fmt}_{rot}", np.uint16), vq.ravel())
                eo, _, ea = pool.extend_attention(qe, bt[0], LP, kc, vc, sm_scale=0.125, want_abs=True)
                assert np.array_equal(out(f"ext_o_{fmt}_{rot}", np.float64), eo.ravel())
                assert np.array_equal(out(f"ext_abs_{fmt}_{rot}", np.float64), ea.ravel())
    wo, wl = oracle.extend_attention(qe, k, v, LP, sm_scale=0.125)
    assert np.array_equal(out("ws_o", np.float64), wo.ravel())
    assert np.array_equal(out("ws_lse", np.float64), wl.ravel())
    codes, scales = oracle.nvfp4_quantize_row(k[0, 0], float(gs[0]))
    assert np.array_equal(out("row_nvfp4", np.float64), oracle.nvfp4_dequant_row(codes, scales, float(gs[0])))
    codes, s = oracle.int4_quantize_row(k[0, 0])
    assert np.array_equal(out("row_int4", np.float64), oracle.int4_dequant_row(codes, s))
    assert np.array_equal(out("row_hadamard", np.float32), oracle.hadamard(k[0, 0]))
    assert out("amax", np.float32)[0] == np.float32(oracle.amax(k))
