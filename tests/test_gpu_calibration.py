"""GPU parity of the NVFP4 global-scale calibration (running amax over prefill
chunks, then gs = amax / (6 * 448)) through the C ABI, and of the cache written
with the calibrated scale, against the CPU oracle, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_kv_amd import inputs, kvq
from gpu_cases import check_attention

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,dtype,magnitude", [(256, torch.bfloat16, 1e-5), (256, torch.float32, 300.0),
                                               (128, torch.bfloat16, 1.0)])
def test_calibrated_cache_matches_oracle(D, dtype, magnitude):
    print(f"case: calibration D {D} {dtype} magnitude {magnitude}", flush=True)
    Hkv, G, P = 2, 6, 16
    lens = [100, 37, 1000]            # three prefill chunks, one sequence each
    ks, vs = [], []
    for b, L in enumerate(lens):
        k, v = inputs.kv_lognormal_channels(31, b, L, Hkv, D)
        ks.append((k * np.float32(magnitude)).astype(np.float32))
        vs.append((v * np.float32(magnitude * 0.5)).astype(np.float32))
    pps = -(-max(lens) // P)
    num_pages = len(lens) * pps
    bt = inputs.page_tables(31, len(lens), pps, num_pages, shuffled=True)
    cache = kvq.Cache(1, num_pages, P, Hkv, D, device="cuda")
    cache.pool.fill_(0xFF)
    running = torch.zeros(2, dtype=torch.float32, device="cuda")
    dev = []
    for k, v in zip(ks, vs):
        kd, vd = torch.from_numpy(k).cuda().to(dtype), torch.from_numpy(v).cuda().to(dtype)
        kvq.kvq_calibrate_amax(cache, kd, vd, running)
        dev.append((kd, vd))
    kvq.kvq_calibrate_global_scale(cache, running)
    torch.cuda.synchronize()
    # the oracle sees the exact values the GPU read (bf16 inputs widened exactly)
    k_all = np.concatenate([kd.float().cpu().numpy() for kd, _ in dev])
    v_all = np.concatenate([vd.float().cpu().numpy() for _, vd in dev])
    amax = (oracle.amax(k_all), oracle.amax(v_all))
    got_amax = running.cpu().numpy()
    assert got_amax[0] == np.float32(amax[0]) and got_amax[1] == np.float32(amax[1]), (got_amax, amax)
    gs = (oracle.global_scale(amax[0]), oracle.global_scale(amax[1]))
    got_gs = cache.global_scale.cpu().numpy()
    assert got_gs[0] == np.float32(gs[0]) and got_gs[1] == np.float32(gs[1]), (got_gs, gs)
    # store every chunk with the calibrated scale, then compare bytes and attention
    ref = oracle.Pool(1, num_pages, P, Hkv, D, global_scale=gs, fill=0xFF)
    for b, (kd, vd) in enumerate(dev):
        slots = inputs.slots_for(bt, P, b, 0, lens[b])
        kvq.kvq_quantize_store(cache, kd, vd, torch.from_numpy(slots).cuda())
        ref.quantize_store(kd.float().cpu().numpy(), vd.float().cpu().numpy(), slots)
    torch.cuda.synchronize()
    assert np.array_equal(cache.pool.cpu().numpy(), ref.data)
    q = inputs.query(31, 99, len(lens), Hkv * G, D)
    lens_np = np.array(lens, np.int32)
    out = kvq.kvq_decode_attention(cache, torch.from_numpy(q).cuda().to(torch.bfloat16), torch.from_numpy(bt).cuda(),
                                   torch.from_numpy(lens_np).cuda(), max(lens), out_dtype=torch.float32)
    torch.cuda.synchronize()
    r, _ = ref.decode_attention(q, bt, lens_np)
    # the attention output scales with the V magnitude; compare relative to it
    s = float(np.abs(r).max())
    check_attention(out.cpu().numpy() / s, r / s, lens_np, label="calibrated")
