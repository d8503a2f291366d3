"""Exhaustive GPU checks of the gfx950 conversion instructions the bit-exact
paths use (tests/conv_check.hip): the E2M1 encoder behind the NVFP4 element
codes, the E4M3 encoder behind FP8 values and the bf16 rounding behind bf16
outputs and prefix dequantization, each over every fp32 input but NaN; the E2M1 and E4M3 decoders over all their
codes.  Each reference rule is written in the check kernel from the format
definitions ("SGLang's 4-bit KV cache: the 56% is exact, the 1.78x is
untested", section "The 56% survives its own scale, and names the block
size"); zero mismatches are required."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq_convcheck.so")
CHECKS = {0: "v_cvt_scalef32_pk_fp4_f32 (E2M1 encode, scale 1): every fp32 input but NaN",
          1: "v_cvt_pk_bf16_f32 (round to nearest even): every fp32 input but NaN",
          2: "v_cvt_scalef32_pk_{f16,f32}_fp4 (E2M1 decode): 256 bytes x 4 positions",
          3: "v_cvt_pk_f32_fp8, v_cvt_scalef32_pk_f16_fp8 (E4M3 decode): 256 codes x 2 positions",
          4: "v_cvt_pk_fp8_f32 after a clamp to +-448 (E4M3 encode): every fp32 input but NaN"}


@pytest.mark.parametrize("which", sorted(CHECKS))
def test_conversion_is_exact_over_its_domain(which):
    print(f"case: {CHECKS[which]}", flush=True)
    assert os.path.exists(LIB), "tests/libkvq_convcheck.so is not built (run __graft_entry__.build())"
    lib = ctypes.CDLL(LIB)
    lib.kvqc_run.restype = ctypes.c_int
    lib.kvqc_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    n = lib.kvqc_workgroups(which)
    count = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    first = torch.zeros((n,), dtype=torch.int32, device="cuda")
    rc = lib.kvqc_run(which, ctypes.c_void_p(count.data_ptr()), ctypes.c_void_p(first.data_ptr()),
                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, f"launch failed: hipError {rc}"
    torch.cuda.synchronize()
    c = count.cpu().numpy().view("uint32")
    f = first.cpu().numpy().view("uint32")
    assert (c != 0xFFFFFFFF).all(), "a workgroup wrote no result"
    bad = int(c.astype("uint64").sum())
    assert bad == 0, f"{bad} mismatches, smallest mismatching input {int(f.min()):#010x}"
