"""GPU parity of the split-precision format -- FP8 (E4M3, per-tensor scale)
keys with NVFP4 values -- through the C ABI: packed bytes bit for bit and
decode attention within the tolerance of gpu_cases, against the CPU oracle,
over several shapes, page sizes, ragged lengths, empty sequences and split
counts.  Unused cache bytes are poisoned with 0xFF (an E4M3 NaN key), so a
kernel that let a past-the-end key into a visible score would fail."""
import numpy as np
import pytest
import torch

from gpu_cases import Case, check_attention, check_pool_bitexact

pytestmark = pytest.mark.gpu

CASES = [
    # D, Hkv, G, P, lens, kind, dtype, scales {K per-tensor, V global}
    (256, 2, 6, 16, [1, 47, 0, 300], "lognormal", torch.bfloat16, (0.21, 1.0)),
    (256, 1, 16, 32, [33, 95], "outliers", torch.float32, (0.05, 0.37)),
    (128, 2, 4, 16, [17, 250, 64], "student_t", torch.bfloat16, (0.02, 1.0)),
    (128, 1, 1, 48, [5, 130], "lognormal", torch.float32, (1.0, 0.125)),
    (256, 4, 6, 1600, [2500, 1601, 33], "student_t", torch.bfloat16, (0.013, 1.0)),
]


@pytest.mark.parametrize("D,Hkv,G,P,lens,kind,dtype,scales", CASES)
def test_k8v4_store_and_decode(D, Hkv, G, P, lens, kind, dtype, scales):
    print(f"case: k8v4 D {D} Hkv {Hkv} G {G} P {P} lens {lens} {kind} {dtype} scales {scales}", flush=True)
    c = Case(4, D, Hkv, G, P, lens, kind=kind, in_dtype=dtype, gs=scales, seed=400 + D + G)
    check_pool_bitexact(c)
    ref, ref_lse = c.oracle_decode()
    out, lse = c.decode(torch.float32)
    check_attention(out, ref, c.lens, lse=lse, ref_lse=ref_lse, label="fp32 out")
    outb, _ = c.decode(torch.bfloat16, want_lse=False)
    check_attention(outb, ref, c.lens, bf16=True, label="bf16 out")
    for ns in (1, 3, 0):
        o1, l1 = c.decode(torch.float32, num_splits=ns)
        o2, l2 = c.decode(torch.float32, num_splits=ns)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        check_attention(o1, ref, c.lens, lse=l1, ref_lse=ref_lse, label=f"splits {ns}")
