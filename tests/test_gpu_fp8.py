"""GPU parity of the FP8 E4M3 per-tensor comparator format through the C ABI:
packed bytes bit for bit, decode attention within the tolerance of
gpu_cases, against the CPU oracle.  Unused cache bytes are NaN-poisoned
(0xFF is an E4M3 NaN), so a kernel that let a token past the end of a
sequence into the PV product would fail."""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_kv_amd import kvq
from gpu_cases import Case, check_attention, check_pool_bitexact

pytestmark = pytest.mark.gpu

CASES = [
    # D, Hkv, G, P, lens, kind, dtype, scales
    (256, 2, 6, 16, [1, 47, 0, 300], "lognormal", torch.bfloat16, (0.21, 0.13)),
    (256, 1, 16, 32, [33, 95], "outliers", torch.float32, (0.05, 0.03)),
    (128, 2, 4, 16, [17, 250, 64], "student_t", torch.bfloat16, (0.02, 0.5)),
    (128, 1, 1, 48, [5, 130], "lognormal", torch.float32, (1.0, 0.25)),
    (256, 4, 6, 1600, [2500, 1601, 33], "student_t", torch.bfloat16, (0.013, 0.017)),
]


@pytest.mark.parametrize("D,Hkv,G,P,lens,kind,dtype,scales", CASES)
def test_fp8_store_and_decode(D, Hkv, G, P, lens, kind, dtype, scales):
    print(f"case: fp8 D {D} Hkv {Hkv} G {G} P {P} lens {lens} {kind} {dtype} scales {scales}", flush=True)
    c = Case(3, D, Hkv, G, P, lens, kind=kind, in_dtype=dtype, gs=scales, seed=300 + D + G)
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


def test_fp8_every_code_round_trips():
    # values that are exactly s * (every finite E4M3 value, both signs) are
    # stored as their own code and decode to themselves
    D, Hkv, P = 256, 1, 16
    s = 0.375
    vals = np.array([oracle.e4m3_value(c) for c in range(0x7F)] + [-oracle.e4m3_value(c) for c in range(0x7F)])
    n = -(-vals.size // D)
    x = np.zeros(n * D, np.float32)
    x[:vals.size] = vals * s
    k = x.reshape(n, 1, D)
    v = k[::-1].copy()
    cache = kvq.Cache(3, 1, P, Hkv, D, device="cuda", global_scale=(s, s))
    cache.pool.fill_(0xFF)
    kvq.kvq_quantize_store(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                           torch.arange(n, dtype=torch.int32, device="cuda"))
    ref = oracle.Pool(3, 1, P, Hkv, D, global_scale=(s, s), fill=0xFF)
    ref.quantize_store(k, v, np.arange(n, dtype=np.int32))
    torch.cuda.synchronize()
    got = cache.pool.cpu().numpy()
    assert np.array_equal(got, ref.data)
    codes = got[0, 0, :D * n]
    expect = np.array([c for c in range(0x7F)] + [0x80 | c for c in range(0x7F)], np.uint8)
    assert np.array_equal(codes[:expect.size], expect)


@pytest.mark.parametrize("D,P,start,n,skip", [
    (256, 16, 0, 64, None),    # whole pages: every 16-token run goes through the tiled value store
    (256, 32, 0, 96, None),    # runs of 16 inside 32-token pages
    (256, 16, 8, 40, None),    # runs that start mid-way: byte-by-byte value store
    (128, 16, 0, 64, None),    # two runs per workgroup at head dim 128
    (128, 48, 24, 80, None),   # runs from an unaligned slot, some across a page boundary
    (128, 16, 0, 64, 20),      # an aligned run and one with a skipped slot in one workgroup
    (256, 16, 0, 64, 21),      # a skipped slot: that workgroup stores byte by byte
])
def test_fp8_value_rows_tiled_and_scattered(D, P, start, n, skip):
    # chunked-prefill stores whose 16-token runs fill aligned slot runs of one
    # page take the LDS-transposed value path, the others the byte scatter;
    # both must leave the same bytes as the oracle (0xFF poison elsewhere)
    print(f"case: fp8 value rows D {D} P {P} start {start} n {n} skip {skip}", flush=True)
    Hkv = 2
    g = np.random.default_rng(1000 + D + P + start)
    k = g.standard_normal((n, Hkv, D)).astype(np.float32)
    v = (g.standard_normal((n, Hkv, D)) * 2.0).astype(np.float32)
    npages = -(-(start + n) // P) + 1
    pages = g.permutation(npages).astype(np.int32)  # the sequence's pages, shuffled
    t = np.arange(start, start + n)
    slots = (pages[t // P] * P + t % P).astype(np.int32)
    if skip is not None:
        slots[skip] = -1
    cache = kvq.Cache(3, npages, P, Hkv, D, device="cuda", global_scale=(0.05, 0.07))
    cache.pool.fill_(0xFF)
    kvq.kvq_quantize_store(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                           torch.from_numpy(slots).cuda())
    ref = oracle.Pool(3, npages, P, Hkv, D, global_scale=(0.05, 0.07), fill=0xFF)
    ref.quantize_store(k, v, slots)
    torch.cuda.synchronize()
    got = cache.pool.cpu().numpy().ravel()
    want = ref.data.ravel()
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"
