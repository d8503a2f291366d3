"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element
by element, on seeded inputs spanning several pages, ragged tails, empty
sequences, skipped slots, NaN-poisoned unused cache bytes and both formats.

Packed bytes and prefix dequantization are compared bit for bit; attention
within the bar stated in gpu_cases (2e-3 absolute in fp32 output; in bf16
output one bf16 ulp of the rounded oracle value, 2e-3 where |oracle| < 0.5 and
2e-3 plus half an ulp elsewhere; cosine >= 0.9995; lse within 1e-3)."""
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
    # 16 query heads per KV head at head dim 256: the largest decode workgroup
    # LDS (four waves' [16][256] partial o), above the default 64 KiB limit
    (2, 256, 2, 16, 16, [77, 300], "student_t", torch.bfloat16, (1.0, 1.0)),
    # per-token scales over 33 binades: INT4's bound of the running max by the
    # value scale's exponent (p times the scale stays in fp16), NVFP4 block
    # scales that underflow or saturate E4M3 token by token
    (1, 256, 2, 6, 16, [300, 47], "token_scaled_o1", torch.float32, (1.0, 1.0)),
    (2, 256, 2, 6, 16, [300, 47], "token_scaled_o1", torch.float32, (1.0, 1.0)),
    (2, 128, 1, 4, 32, [1000], "token_scaled_o1", torch.bfloat16, (1.0, 1.0)),
    (2, 256, 1, 8, 1600, [2000], "token_scaled_o1", torch.bfloat16, (1.0, 1.0)),
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


def _special_rows(fmt, D, rng):
    """Rows that reach every branch of the quantizers: signed zeros, fp32
    denormals, exact rounding ties, all-zero blocks, block scales that
    underflow E4M3 or saturate at 448, and INT4 rows with denormal scales."""
    rows = []
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for _ in range(6):
        x = rng.standard_normal(D).astype(np.float32)
        x[::7] = 0.0
        x[1::7] = -0.0
        x[2::11] = np.float32(1e-40) * rng.choice([-1, 1], size=x[2::11].shape)
        rows.append(x)
    if fmt == 1:
        for S in (0.171875, 0.001953125, 1.0, 26.0):
            x = np.zeros(D, np.float32)
            for b in range(D // 16):
                blk = np.concatenate([[6.0], ties, -ties[:4], grid[1:5]])[:16] * S
                rng.shuffle(blk)
                x[16 * b:16 * b + 16] = blk
            rows.append(x.astype(np.float32))
        x = rng.standard_normal(D).astype(np.float32)
        x[:16] = 0.0                                # all-zero block
        x[16:32] *= np.float32(1e-5)                # scale below E4M3's smallest subnormal
        x[32:48] *= np.float32(1e4)                 # block scale saturated at 448
        x[48:64] = -x[48:64] * np.float32(1e-38)    # tiny but nonzero
        rows.append(x)
    else:
        x = np.array([(k % 15 - 7) + 0.5 * (k % 2) for k in range(D)], np.float32)
        x[0] = 7.0                                  # s = 1: exact ties at half-integers
        rows.append(x)
        rows.append((rng.standard_normal(D) * 1e-39).astype(np.float32))   # denormal row scale
        rows.append((rng.standard_normal(D) * 1e-30).astype(np.float32))   # scale near 2^-100
        rows.append(np.zeros(D, np.float32))
        y = rng.standard_normal(D).astype(np.float32)
        y[::5] = -0.0
        rows.append(y)
    return np.stack(rows)


@pytest.mark.parametrize("fmt,gs", [(1, (1.0, 1.0)), (1, (0.125, 4.0)), (1, (0.37, 2.5)), (2, (1.0, 1.0))])
def test_store_special_values(fmt, gs):
    import oracle
    from bit_quantized_kv_amd import kvq
    print(f"case: special values fmt {fmt} gs {gs}", flush=True)
    D, Hkv, P = 256, 2, 16
    rng = np.random.default_rng(7 + fmt)
    rows = _special_rows(fmt, D, rng)
    n = rows.shape[0] * 2
    k = np.stack([rows, rows[::-1]], axis=1)        # [n/2][2][D]
    k = np.concatenate([k, -k])                      # [n][2][D]
    v = np.ascontiguousarray(k[:, ::-1] * np.float32(0.5))
    k = np.ascontiguousarray(k)
    num_pages = -(-n // P) + 1
    slots = np.arange(n, dtype=np.int32)
    cache = kvq.Cache(fmt, num_pages, P, Hkv, D, device=torch.device("cuda"), global_scale=gs)
    cache.pool.fill_(0xFF)
    kvq.kvq_quantize_store(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                           torch.from_numpy(slots).cuda())
    ref = oracle.Pool(fmt, num_pages, P, Hkv, D, global_scale=gs, fill=0xFF)
    ref.quantize_store(k, v, slots)
    torch.cuda.synchronize()
    got = cache.pool.cpu().numpy()
    if not np.array_equal(got, ref.data):
        diff = np.argwhere(got != ref.data)
        raise AssertionError(f"{len(diff)} bytes differ, first {diff[:5].tolist()}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_int4_store_quotients_at_half_integers(dtype):
    # rows where many x / s land on or next to half-integers: x = amax (2k+1)/14
    # (exactly amax / 2 among them, common with bf16 inputs) -- rint(RN(x / s))
    # is then decided by the last bits of the quotient, ties to even; the
    # packed codes and scales must match the oracle bit for bit
    import oracle
    from bit_quantized_kv_amd import kvq
    print(f"case: int4 half-integer quotients {dtype}", flush=True)
    D, Hkv, P, n = 256, 2, 16, 96
    g = np.random.default_rng(77 if dtype == torch.bfloat16 else 78)
    x = g.standard_normal((2, n, Hkv, D)).astype(np.float32)
    amax = np.abs(x).max(axis=3, keepdims=True)
    k_odd = g.integers(0, 7, size=x.shape) * 2 + 1
    planted = (amax * k_odd / 14.0).astype(np.float32) * np.where(g.random(x.shape) < 0.5, -1.0, 1.0)
    mask = g.random(x.shape) < 0.3
    x = np.where(mask, planted, x).astype(np.float32)
    x[..., 5] = amax[..., 0] / 2.0
    xt = torch.from_numpy(x).to(dtype)
    x_in = xt.float().numpy()  # the values the kernel sees
    slots = np.arange(n, dtype=np.int32)
    cache = kvq.Cache(2, n // P, P, Hkv, D, device="cuda")
    cache.pool.fill_(0x5A)
    kvq.kvq_quantize_store(cache, xt[0].cuda(), xt[1].cuda(), torch.from_numpy(slots).cuda())
    ref = oracle.Pool(2, n // P, P, Hkv, D, fill=0x5A)
    ref.quantize_store(x_in[0], x_in[1], slots)
    torch.cuda.synchronize()
    got = cache.pool.cpu().numpy().ravel()
    want = ref.data.ravel()
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"
