"""GPU parity of extend attention over the bf16 workspace (through the C ABI)
against the oracle: random workspaces over several shapes, ragged row
blocks, both output dtypes and the lse; and the whole extend path -- a 4-bit
cached prefix expanded by kvq_dequant_prefix, the chunk's K/V appended, then
extend attention -- against the oracle on the same workspace."""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_kv_amd import inputs, kvq
from gpu_cases import check_attention

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
    s = max(1.0, float(np.abs(ref).max()))
    check_attention(out.cpu().numpy() / s, ref / s, lens, lse=lse.cpu().numpy(), ref_lse=ref_lse, label="fp32")
    # bf16 output: within the fp32 bound plus half a bf16 ulp of the value
    from gpu_cases import ATOL, bf16_half_ulp
    err = np.abs(outb.float().cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= ATOL * s + bf16_half_ulp(ref)), err.max()


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
    s = max(1.0, float(np.abs(ref).max()))
    check_attention(out.cpu().numpy() / s, ref / s, np.ones(n, np.int32), label="extend path")
