"""GPU parity of extend attention over the bf16 workspace (through the C ABI)
against the oracle: random workspaces over several shapes, ragged row
blocks, both output dtypes and the lse; and the whole extend path -- a 4-bit
cached prefix expanded by kvq_dequant_prefix, the chunk's K/V appended, then
extend attention -- against the oracle on the same workspace; and the fused
extend that reads the prefix from the 4-bit pages against the oracle's paged
extend (the prefix at its exact dequantized value).

Bars (gpu_cases): the workspace path is held to the decode's absolute bar
(2e-3 in fp32 output; bf16 output as the reading in gpu_cases).  The fused
path rounds each softmax weight to fp16 on the steps wholly inside the
prefix, so its bar adds the derived 2^-11 * (softmax-weighted mean of |v|)
that the oracle reports per element."""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_kv_amd import inputs, kvq
from gpu_cases import F16_WEIGHT_REL, Case, check_attention, check_values

pytestmark = pytest.mark.gpu


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("Lp,n,G,Hkv,D", [(0, 1, 6, 4, 256), (37, 100, 6, 2, 256), (1000, 64, 4, 1, 256),
                                           (5, 33, 16, 1, 256), (64, 70, 1, 2, 128), (300, 17, 3, 3, 128)])
def test_extend_matches_oracle(Lp, n, G, Hkv, D):
    print(f"case: extend Lp {Lp} n {n} G {G} Hkv {Hkv} D {D}", flush=True)
    rng = np.random.default_rng(Lp * 7 + n)
    Hq = G * Hkv
    scale_ch = np.exp(rng.standard_normal((Hkv, D))).astype(np.float32)
    k = bf16(rng.standard_normal((Lp + n + 5, Hkv, D)) * scale_ch)
    v = bf16(rng.standard_normal((Lp + n + 5, Hkv, D)) * scale_ch)
    q = bf16(rng.standard_normal((n, Hq, D)))
    ref, ref_lse = oracle.extend_attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), Lp)
    kd, vd, qd = k.cuda(), v.cuda(), q.cuda()
    lse = torch.empty((n, Hq), dtype=torch.float32, device="cuda")
    out = kvq.kvq_extend_attention(qd, kd, vd, Lp, lse=lse, out_dtype=torch.float32)
    outb = kvq.kvq_extend_attention(qd, kd, vd, Lp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    lens = np.full(n, 1, np.int32)
    check_attention(out.cpu().numpy(), ref, lens, lse=lse.cpu().numpy(), ref_lse=ref_lse, label="fp32")
    check_values(outb.float().cpu().numpy(), ref, bf16=True, label="bf16")


@pytest.mark.parametrize("fmt", [1, 2])
def test_extend_path_over_a_4bit_prefix(fmt):
    print(f"case: extend path fmt {fmt}", flush=True)
    D, Hkv, G, P, Lp, n = 256, 2, 6, 16, 700, 96
    Hq = Hkv * G
    pps = -(-Lp // P)
    bt = inputs.page_tables(41, 1, pps, pps + 2, shuffled=True)
    cache = kvq.Cache(fmt, pps + 2, P, Hkv, D, device="cuda")
    k, v = inputs.kv_lognormal_channels(41, 0, Lp, Hkv, D)
    kvq.kvq_quantize_store(cache, bf16(k).cuda(), bf16(v).cuda(), torch.from_numpy(inputs.slots_for(bt, P, 0, 0, Lp)).cuda())
    # workspace: prefix rows from the cache, then the chunk's own K/V
    kw = torch.empty((Lp + n, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vw = torch.empty_like(kw)
    kvq.kvq_dequant_prefix(cache, torch.from_numpy(bt[0]).cuda(), Lp, kw, vw)
    kc, vc = inputs.kv_lognormal_channels(41, 1, n, Hkv, D)
    kw[Lp:] = bf16(kc).cuda()
    vw[Lp:] = bf16(vc).cuda()
    q = bf16(inputs.query(41, 3, n, Hq, D).reshape(n, Hq, D)).cuda()
    out = kvq.kvq_extend_attention(q, kw, vw, Lp, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.extend_attention(q.float().cpu().numpy(), kw.float().cpu().numpy(), vw.float().cpu().numpy(), Lp)
    check_attention(out.cpu().numpy(), ref, np.ones(n, np.int32), label="extend path")


PAGED = [
    # fmt, D, Hkv, G, P, prefix_len, chunk_len, gs
    (1, 256, 2, 6, 16, 700, 96, (0.37, 2.5)),
    (2, 256, 2, 6, 16, 700, 96, (1.0, 1.0)),
    (1, 256, 1, 4, 32, 64, 33, (1.0, 1.0)),
    (2, 256, 1, 16, 48, 5, 40, (1.0, 1.0)),
    (1, 128, 2, 4, 16, 37, 70, (1.0, 0.125)),
    (2, 128, 3, 3, 16, 300, 17, (1.0, 1.0)),
    (1, 256, 2, 6, 16, 0, 50, (0.5, 0.5)),
    (1, 256, 2, 6, 16, 2000, 40, (0.015625, 0.03125)),
    # page sizes that are not powers of two, prefixes over many pages ending mid-page
    (2, 256, 2, 6, 1600, 5000, 40, (1.0, 1.0)),
    (1, 256, 1, 6, 48, 1000, 37, (1.0, 1.0)),
    (2, 128, 1, 4, 80, 3333, 20, (1.0, 1.0)),
    # head dim 128 over many fp16 prefix steps (the two-deep loop)
    (1, 128, 2, 4, 16, 700, 50, (0.5, 2.0)),
    # group sizes 1 (one query head per KV head; 200 rows over two workgroups),
    # 8 (INT4, 32-token pages: a step's halves in one page) and 5 (385 rows: the
    # last workgroup holds one row; the prefix ends mid-page and mid-step)
    (1, 256, 4, 1, 16, 500, 200, (1.0, 1.0)),
    (2, 256, 2, 8, 32, 900, 30, (1.0, 1.0)),
    (1, 256, 1, 5, 16, 333, 77, (0.5, 1.0)),
    # around the paired prefix loop's threshold: 6 fp16 prefix steps (single
    # steps only), 7 (one paired iteration) and 8 (the pair loop's exit into
    # single steps)
    (2, 256, 1, 4, 16, 200, 33, (1.0, 1.0)),
    (1, 256, 2, 6, 16, 224, 40, (1.0, 1.0)),
    (1, 128, 1, 6, 32, 256, 24, (0.25, 0.5)),
    # one chunk token over a long prefix: 6 rows, so every wavefront but the
    # first holds padding rows -- the compute-only ones (their own paired loop,
    # no loads) and the stagers alike
    (1, 256, 1, 6, 16, 1500, 1, (1.0, 1.0)),
    (2, 256, 2, 6, 16, 1500, 1, (1.0, 1.0)),
]


def _paged_ref(c, q, Lp, kc_d, vc_d):
    """The oracle's paged extend over sequence 0's cached prefix and the chunk
    rows: (out, lse, the derived fp16-weight term of the bar)."""
    ref, ref_lse, oabs = c.ref.extend_attention(q.float().cpu().numpy(), c.bt[0], Lp, kc_d.float().cpu().numpy(),
                                                vc_d.float().cpu().numpy(), want_abs=True)
    return ref, ref_lse, F16_WEIGHT_REL * oabs


@pytest.mark.parametrize("fmt,D,Hkv,G,P,Lp,n,gs", PAGED)
def test_extend_paged_matches_oracle(fmt, D, Hkv, G, P, Lp, n, gs):
    """The fused extend reads the prefix from the 4-bit pages: same result as the
    oracle's extend over [exactly dequantized prefix | bf16 chunk]."""
    print(f"case: paged extend fmt {fmt} D {D} Hkv {Hkv} G {G} P {P} Lp {Lp} n {n} gs {gs}", flush=True)
    c = Case(fmt, D, Hkv, G, P, [max(Lp, 1)], kind="lognormal", in_dtype=torch.bfloat16, gs=gs, seed=500 + Lp + D)
    Hq = Hkv * G
    kc, vc = inputs.kv_lognormal_channels(57, Lp, n, Hkv, D)
    kc_d, vc_d = bf16(kc).cuda(), bf16(vc).cuda()
    q = bf16(inputs.query(57, 7, n, Hq, D).reshape(n, Hq, D)).cuda()
    lse = torch.empty((n, Hq), dtype=torch.float32, device="cuda")
    bt = c.bt_dev[0].contiguous()
    out = kvq.kvq_extend_attention_paged(c.cache, bt, Lp, q, kc_d, vc_d, lse=lse, out_dtype=torch.float32)
    outb = kvq.kvq_extend_attention_paged(c.cache, bt, Lp, q, kc_d, vc_d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, ref_lse, extra = _paged_ref(c, q, Lp, kc_d, vc_d)
    check_attention(out.cpu().numpy(), ref, np.ones(n, np.int32), lse=lse.cpu().numpy(), ref_lse=ref_lse,
                    label="paged fp32", extra=extra)
    check_values(outb.float().cpu().numpy(), ref, bf16=True, extra=extra, label="paged bf16")


def test_extend_paged_agrees_with_workspace_path():
    """Fused and workspace extend over the same NVFP4 prefix (global scales
    0.25 and 4, powers of two, so the bf16 workspace holds the prefix exactly):
    each against the oracle over the same keys and values, the workspace kernel
    at the absolute bar and the fused kernel at its derived bar."""
    print("case: paged vs workspace extend", flush=True)
    D, Hkv, G, P, Lp, n = 256, 2, 4, 16, 1000, 128
    c = Case(1, D, Hkv, G, P, [Lp], kind="outliers", in_dtype=torch.bfloat16, gs=(0.25, 4.0), seed=77)
    kc, vc = inputs.kv_lognormal_channels(58, 0, n, Hkv, D)
    q = bf16(inputs.query(58, 1, n, Hkv * G, D).reshape(n, Hkv * G, D)).cuda()
    kw = torch.empty((Lp + n, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vw = torch.empty_like(kw)
    kvq.kvq_dequant_prefix(c.cache, c.bt_dev[0], Lp, kw, vw)
    kw[Lp:] = bf16(kc).cuda()
    vw[Lp:] = bf16(vc).cuda()
    ws = kvq.kvq_extend_attention(q, kw, vw, Lp, out_dtype=torch.float32)
    fused = kvq.kvq_extend_attention_paged(c.cache, c.bt_dev[0].contiguous(), Lp, q, kw[Lp:], vw[Lp:],
                                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_ws, _ = oracle.extend_attention(q.float().cpu().numpy(), kw.float().cpu().numpy(), vw.float().cpu().numpy(), Lp)
    ref, _, extra = _paged_ref(c, q, Lp, kw[Lp:], vw[Lp:])
    np.testing.assert_allclose(ref_ws, ref, rtol=1e-12, atol=1e-12)  # the same keys and values
    check_attention(ws.cpu().numpy(), ref_ws, np.ones(n, np.int32), label="workspace")
    check_attention(fused.cpu().numpy(), ref, np.ones(n, np.int32), label="fused", extra=extra)


def test_extend_paged_query_rows_of_any_magnitude():
    """The fused NVFP4 extend scales each query row by a power of two into fp16's
    range on the prefix steps: rows from 2^-20 to 2^4 times N(0,1) (near-uniform
    to near-one-hot attention) still match the oracle."""
    print("case: paged extend, query rows scaled by 2^-20 .. 2^4", flush=True)
    D, Hkv, G, P, Lp, n = 256, 2, 6, 16, 700, 40
    c = Case(1, D, Hkv, G, P, [Lp], kind="lognormal", in_dtype=torch.bfloat16, gs=(1.0, 1.0), seed=901)
    Hq = Hkv * G
    kc, vc = inputs.kv_lognormal_channels(59, 0, n, Hkv, D)
    kc_d, vc_d = bf16(kc).cuda(), bf16(vc).cuda()
    rng = np.random.default_rng(59)
    row_scale = np.exp2(rng.integers(-20, 5, size=(n, Hq, 1))).astype(np.float32)
    q = bf16(inputs.query(59, 1, n, Hq, D).reshape(n, Hq, D) * row_scale).cuda()
    out = kvq.kvq_extend_attention_paged(c.cache, c.bt_dev[0].contiguous(), Lp, q, kc_d, vc_d,
                                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _, extra = _paged_ref(c, q, Lp, kc_d, vc_d)
    check_attention(out.cpu().numpy(), ref, np.ones(n, np.int32), label="paged, scaled query rows", extra=extra)


@pytest.mark.parametrize("fmt", [1, 2])
def test_extend_paged_token_scales_over_many_binades(fmt):
    """Prefix rows whose scales span 2^-30 .. 2^12 token by token: on the fp16
    prefix steps the INT4 value scale rides on p in fp16, kept in range by
    bounding the running max with the scale's exponent; NVFP4 block scales
    saturate or vanish at the ends, which the oracle reproduces byte for byte."""
    print(f"case: paged extend, token scales 2^-30 .. 2^12, fmt {fmt}", flush=True)
    D, Hkv, G, P, Lp, n = 256, 2, 6, 16, 900, 40
    c = Case(fmt, D, Hkv, G, P, [Lp], kind="token_scaled", in_dtype=torch.float32, seed=911)
    assert np.array_equal(c.gpu_pool(), c.ref.data), "cache bytes differ from the oracle's"
    kc, vc = inputs.kv_lognormal_channels(60, 0, n, Hkv, D)
    kc_d, vc_d = bf16(kc).cuda(), bf16(vc).cuda()
    q = bf16(inputs.query(60, 1, n, Hkv * G, D).reshape(n, Hkv * G, D)).cuda()
    out = kvq.kvq_extend_attention_paged(c.cache, c.bt_dev[0].contiguous(), Lp, q, kc_d, vc_d,
                                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _, extra = _paged_ref(c, q, Lp, kc_d, vc_d)
    got = out.cpu().numpy().astype(np.float64)
    check_values(got, ref, extra=extra, label="paged, token scales over 42 binades")
    # cosine where the output is not numerically zero: attention can settle on a
    # prefix token whose value row quantized to zero (a 2^-30 row under NVFP4's
    # E4M3 block scale), leaving outputs of ~1e-300 where a cosine means nothing
    from gpu_cases import MIN_COS, cosine
    norms = np.linalg.norm(ref, axis=-1)
    rows = np.argwhere(norms >= 1e-6 * np.abs(ref).max())
    assert len(rows) >= ref.shape[0] * ref.shape[1] // 2
    for i, h in rows:
        assert cosine(got[i, h], ref[i, h]) >= MIN_COS, (i, h)
