"""The C ABI's argument validation (kvq_api.cpp) built for the host alone
with AddressSanitizer and UndefinedBehaviorSanitizer, linked against stand-in
launchers (tests/abi_sanitize_stubs.cpp) and driven through every entry
point by tests/abi_sanitize_main.cpp in a subprocess: each valid call asks
for exactly one launch of the right kernel family, each invalid one returns
the documented status and asks for none, and no sanitizer reports anything.
No GPU is used."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"


def test_abi_validation_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not available")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "bit_quantized_kv_amd", "csrc")]
    objs = []
    for src in (os.path.join(ROOT, "bit_quantized_kv_amd", "csrc", "kvq_api.cpp"),
                os.path.join(HERE, "abi_sanitize_stubs.cpp"), os.path.join(HERE, "abi_sanitize_main.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        # host code only: every sanitizer flag is scoped to the host pass
        cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined", *inc, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_asan")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:exitcode=23", UBSAN_OPTIONS="halt_on_error=1:exitcode=24")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, \
        r.stdout + r.stderr[-4000:]
    assert r.stdout.startswith("0 failures"), r.stdout
