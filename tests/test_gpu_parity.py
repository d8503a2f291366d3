"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element
by element, on seeded inputs spanning several pages, ragged tails, empty
sequences, skipped slots, NaN-poisoned unused cache bytes and both formats.

Packed bytes and prefix dequantization are compared bit for bit; attention
within the tolerance stated in gpu_cases (2e-3 absolute in fp32 output, plus
half a bf16 ulp in bf16 output; cosine >= 0.9995; lse within 1e-3)."""
import numpy as np
import pytest
import torch

from gpu_cases import Case, check_attention, check_dequant_prefix, check_pool_bitexact, cosine

pytestmark = pytest.mark.gpu


def test_tiny_nvfp4_reference_case():
    # 1 layer, 1 KV head, 4 query heads, head dim 256, batch 1, context 512,
    # 16-token pages; K, V fp32 N(0,1) with 4 channels x8; q bf16 N(0,1)
    print("case: tiny NVFP4 512 tokens", flush=True)
    c = Case(1, 256, 1, 4, 16, [512], kind="outliers", in_dtype=torch.float32, shuffled=False, seed=1)
    check_pool_bitexact(c)
    ref, ref_lse = c.oracle_decode()
    out, lse = c.decode(torch.float32)
    check_attention(out, ref, c.lens, lse=lse, ref_lse=ref_lse, label="fp32 out")
    outb, _ = c.decode(torch.bfloat16)
    check_attention(outb, ref, c.lens, bf16=True, label="bf16 out")
    check_dequant_prefix(c)
    # a shuffled page table over the same tokens gives bit-identical output
    s = Case(1, 256, 1, 4, 16, [512], kind="outliers", in_dtype=torch.float32, shuffled=True, seed=1)
    assert not np.array_equal(s.bt, c.bt)
    out_s, lse_s = s.decode(torch.float32)
    assert np.array_equal(out_s, out) and np.array_equal(lse_s, lse)


SWEEP = [
    # fmt, D, Hkv, G, P, lens, kind, dtype, gs
    (1, 256, 2, 6, 16, [1, 47, 0, 300], "lognormal", torch.bfloat16, (1.0, 1.0)),
    (1, 256, 1, 16, 32, [33, 95], "outliers", torch.float32, (0.37, 2.5)),
    (1, 128, 2, 4, 16, [17, 250, 64], "lognormal", torch.bfloat16, (1.0, 1.0)),
    (1, 128, 1, 1, 48, [5, 130], "student_t", torch.float32, (1.0, 0.125)),
    (2, 256, 2, 6, 16, [1, 47, 0, 300], "student_t", torch.bfloat16, (1.0, 1.0)),
    (2, 256, 1, 3, 48, [200], "lognormal", torch.float32, (1.0, 1.0)),
    (2, 128, 2, 8, 16, [31, 32, 33], "outliers", torch.bfloat16, (1.0, 1.0)),
    (2, 128, 1, 16, 32, [97], "student_t", torch.float32, (1.0, 1.0)),
]


@pytest.mark.parametrize("fmt,D,Hkv,G,P,lens,kind,dtype,gs", SWEEP)
def test_store_decode_dequant_sweep(fmt, D, Hkv, G, P, lens, kind, dtype, gs):
    print(f"case: fmt {fmt} D {D} Hkv {Hkv} G {G} P {P} lens {lens} {kind} {dtype} gs {gs}", flush=True)
    c = Case(fmt, D, Hkv, G, P, lens, kind=kind, in_dtype=dtype, gs=gs, seed=fmt * 100 + D + G)
    check_pool_bitexact(c)
    ref, ref_lse = c.oracle_decode()
    out, lse = c.decode(torch.float32)
    check_attention(out, ref, c.lens, lse=lse, ref_lse=ref_lse, label="fp32 out")
    outb, _ = c.decode(torch.bfloat16, want_lse=False)
    check_attention(outb, ref, c.lens, bf16=True, label="bf16 out")
    check_dequant_prefix(c, stride_extra=8 if P == 48 else 0)


def test_skipped_slots_keep_their_bytes():
    print("case: skipped slots", flush=True)
    for fmt in (1, 2):
        c = Case(fmt, 256, 2, 2, 16, [70, 41], kind="student_t", in_dtype=torch.bfloat16, drop_every=3, seed=5)
        check_pool_bitexact(c)


@pytest.mark.parametrize("fmt", [1, 2])
def test_split_sweep_and_determinism(fmt):
    print(f"case: split sweep fmt {fmt}", flush=True)
    c = Case(fmt, 256, 2, 6, 16, [1000, 777, 64], kind="lognormal", in_dtype=torch.bfloat16, seed=11 + fmt)
    ref, ref_lse = c.oracle_decode()
    outs = {}
    for ns in (1, 2, 3, 5, 0, 32):
        out, lse = c.decode(torch.float32, num_splits=ns)
        check_attention(out, ref, c.lens, lse=lse, ref_lse=ref_lse, label=f"splits {ns}")
        again, lse2 = c.decode(torch.float32, num_splits=ns)
        assert np.array_equal(out, again) and np.array_equal(lse, lse2), f"splits {ns} not reproducible"
        outs[ns] = out


def test_int4_page_1600_partial_pages():
    # INT4 per-token-head with 1,600-token pages; the last page of each
    # sequence is partly filled (the rest is NaN poison)
    print("case: INT4 page 1600", flush=True)
    c = Case(2, 256, 4, 6, 1600, [2500, 1601, 33], kind="student_t", in_dtype=torch.bfloat16, seed=21)
    check_pool_bitexact(c)
    ref, ref_lse = c.oracle_decode()
    out, lse = c.decode(torch.float32)
    check_attention(out, ref, c.lens, lse=lse, ref_lse=ref_lse, label="int4 p1600")
    outb, _ = c.decode(torch.bfloat16, want_lse=False)
    check_attention(outb, ref, c.lens, bf16=True, label="int4 p1600 bf16")
    check_dequant_prefix(c)


def test_quality_vs_unquantized_is_a_format_property():
    # The kernel adds nothing beyond the format: its cosine to fp32 attention
    # over the unquantized K/V matches the oracle's within 1e-5.
    print("case: quality vs unquantized", flush=True)
    for fmt in (1, 2):
        c = Case(fmt, 256, 1, 4, 16, [512], kind="outliers", in_dtype=torch.float32, shuffled=False, seed=1)
        ref, _ = c.oracle_decode()
        out, _ = c.decode(torch.float32)
        q = torch.from_numpy(c.q[0]).double()
        K = torch.from_numpy(c.k[:, 0]).double()
        V = torch.from_numpy(c.v[:, 0]).double()
        full = torch.softmax(q @ K.T / 16.0, dim=-1) @ V
        for h in range(c.Hq):
            cg = cosine(out[0, h], full[h].numpy())
            co = cosine(ref[0, h], full[h].numpy())
            assert abs(cg - co) <= 1e-5, (fmt, h, cg, co)
