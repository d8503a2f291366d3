"""The decode step captured in a HIP graph: quantize-store of the new token
plus decode attention (and two extend calls: over a bf16 workspace, and fused
over the first sequence's cached pages) recorded once with torch.cuda.graph, then replayed several times with eager work in between
(new queries written in place); every replay must equal the eager calls on
the same inputs bit for bit (same split plan, same kernels)."""
import numpy as np
import pytest
import torch

from bit_quantized_kv_amd import inputs, kvq
from gpu_cases import Case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", [1, 2, 4])
def test_decode_step_graph_replays_match_eager(fmt):
    print(f"case: graph replay fmt {fmt}", flush=True)
    gs = (1.0, 1.0) if fmt != 4 else (0.05, 1.0)
    c = Case(fmt, 256, 2, 6, 16, [300, 47, 129], kind="lognormal", in_dtype=torch.bfloat16, gs=gs, seed=600 + fmt,
             extra_pages=4)
    B, Hq, D = c.B, c.Hq, c.D
    # the new token of each sequence goes to a spare page's rows
    used = set(int(x) for x in c.bt.ravel())
    spare = next(pg for pg in range(c.num_pages - 1, -1, -1) if pg not in used)
    slots = torch.tensor([spare * c.P + b for b in range(B)], dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(inputs.seed_int(60, fmt, 0))
    k_new = torch.randn((B, c.Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    v_new = torch.randn((B, c.Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    q = c.q_dev.clone()
    max_len = int(c.lens.max())
    ws = torch.empty(kvq.kvq_decode_workspace_size(c.cache, B, Hq, max_len, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    # extend over a small bf16 workspace in the same graph
    n, Lp = 40, 70
    kw = torch.randn((Lp + n, c.Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    vw = torch.randn((Lp + n, c.Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    qe = torch.randn((n, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    oe = torch.empty((n, Hq, D), dtype=torch.float32, device="cuda")
    # the fused extend of the same chunk over sequence 0's 300 cached tokens
    # (the step's stores go to a spare page, outside that prefix; NVFP4 and
    # INT4 caches)
    fused = fmt in (1, 2)
    of = torch.zeros((n, Hq, D), dtype=torch.float32, device="cuda")
    lf = torch.zeros((n, Hq), dtype=torch.float32, device="cuda")

    def step():
        kvq.kvq_quantize_store(c.cache, k_new, v_new, slots)
        kvq.kvq_decode_attention(c.cache, q, c.bt_dev, c.lens_dev, max_len, out=out, lse=lse, workspace=ws)
        kvq.kvq_extend_attention(qe, kw, vw, Lp, out=oe)
        if fused:
            kvq.kvq_extend_attention_paged(c.cache, c.bt_dev[0], 300, qe, kw[Lp:], vw[Lp:], out=of, lse=lf)

    # warm up on a side stream, as torch requires before capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        # eager work between replays: new queries in place
        q.copy_(torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16))
        qe.mul_(-1.0)
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        want = (out.clone(), lse.clone(), oe.clone(), c.cache.pool.clone(), of.clone(), lf.clone())
        out.zero_()
        lse.zero_()
        oe.zero_()
        of.zero_()
        lf.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want[0]) and torch.equal(lse, want[1]), f"replay {r}: decode differs"
        assert torch.equal(oe, want[2]), f"replay {r}: extend differs"
        assert torch.equal(of, want[4]) and torch.equal(lf, want[5]), f"replay {r}: fused extend differs"
        assert torch.equal(c.cache.pool, want[3]), f"replay {r}: cache bytes differ"
        assert np.isfinite(out.cpu().numpy()).all()
