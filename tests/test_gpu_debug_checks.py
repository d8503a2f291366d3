"""Debug mode (KVQ_DEBUG=1): the calls that read device index arrays check
them on the device first and return KVQ_ERR_DEVICE_INPUT (-8), launching
nothing else, when a slot, page id or sequence length is out of range; valid
calls give the same bytes as without the checks.

Every out-of-range value used here still points inside owned memory (the
pool is a view into a tensor with one page before it and one page past the
pages the descriptor declares), so a check that failed to stop a launch
would read or write owned memory, never past it."""
import pytest
import torch

from bit_quantized_kv_amd import kvq

pytestmark = pytest.mark.gpu

FMT, N, P, H, D, G = 1, 8, 16, 2, 128, 4  # NVFP4, 8 declared pages of 16 tokens, head dim 128, 4 q heads per KV head
DEVICE_INPUT = -8


def make_cache():
    slab = kvq.kvq_slab_bytes(FMT, P, D)
    owned = torch.zeros((N + 2, H, slab), dtype=torch.uint8, device="cuda")
    return kvq.Cache(FMT, N, P, H, D, pool=owned[1:], global_scale=(0.5, 0.25))  # page -1 and page N are owned


def fill(cache, ntok, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    k = torch.randn((ntok, H, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((ntok, H, D), generator=g, device="cuda").to(torch.bfloat16)
    slots = torch.arange(ntok, dtype=torch.int32, device="cuda")  # pages 0.. in order
    kvq.kvq_quantize_store(cache, k, v, slots)
    return k, v


def expect_device_input(fn, *args, **kw):
    with pytest.raises(kvq.KvqError) as e:
        fn(*args, **kw)
    assert e.value.status == DEVICE_INPUT, e.value


@pytest.fixture
def debug(monkeypatch):
    monkeypatch.setenv("KVQ_DEBUG", "1")


def run_all(cache, table, lens, max_len, q, qc, kc, vc):
    out = kvq.kvq_decode_attention(cache, q, table, lens, max_len, out_dtype=torch.float32)
    out_na = torch.empty_like(out)
    kvq.kvq_decode_attention_noalloc(cache, q, table, lens, max_len, out_na)
    kw = torch.zeros((max_len, H * D), dtype=torch.bfloat16, device="cuda")
    vw = torch.zeros_like(kw)
    kvq.kvq_dequant_prefix(cache, table[0], int(lens[0].item()), kw, vw)
    ext = kvq.kvq_extend_attention_paged(cache, table[0], int(lens[0].item()), qc, kc, vc, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return out, out_na, kw, vw, ext


def inputs(seed=3):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn((2, H * G, D), generator=g, device="cuda").to(torch.bfloat16)
    qc = torch.randn((20, H * G, D), generator=g, device="cuda").to(torch.bfloat16)
    kc = torch.randn((20, H, D), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((20, H, D), generator=g, device="cuda").to(torch.bfloat16)
    return q, qc, kc, vc


def test_valid_calls_give_the_same_bytes_with_and_without_checks(monkeypatch):
    print("case: debug mode, valid store / decode / noalloc decode / dequant / fused extend", flush=True)
    table = torch.arange(2 * N, dtype=torch.int32, device="cuda").reshape(2, N) % N
    lens = torch.tensor([100, 37], dtype=torch.int32, device="cuda")
    q, qc, kc, vc = inputs()
    results, pools = [], []
    for debug in (False, True):
        if debug:
            monkeypatch.setenv("KVQ_DEBUG", "1")
        else:
            monkeypatch.delenv("KVQ_DEBUG", raising=False)
        cache = make_cache()
        k, v = fill(cache, 100, seed=11)
        results.append(run_all(cache, table, lens, 128, q, qc, kc, vc))
        # a skipped token (slot -1) and the pool's last row
        slots = torch.tensor([-1, 101, N * P - 1], dtype=torch.int32, device="cuda")
        kvq.kvq_quantize_store(cache, k[:3], v[:3], slots)
        torch.cuda.synchronize()
        pools.append(cache.pool.clone())
    for a, b in zip(*results):
        assert torch.equal(a, b)
    assert torch.equal(pools[0], pools[1])


def test_store_slot_past_the_pool_is_rejected(debug):
    print("case: debug mode, store slot N*P", flush=True)
    cache = make_cache()
    k, v = fill(cache, 40, seed=12)
    torch.cuda.synchronize()
    before = cache.pool.clone()
    slots = torch.tensor([5, N * P, 7], dtype=torch.int32, device="cuda")  # row 0 of the undeclared page
    expect_device_input(kvq.kvq_quantize_store, cache, k[:3], v[:3], slots)
    torch.cuda.synchronize()
    assert torch.equal(cache.pool, before)  # nothing written, the valid slots included


def test_page_ids_outside_the_pool_are_rejected(debug):
    print("case: debug mode, page id N in a used table entry", flush=True)
    cache = make_cache()
    fill(cache, 100, seed=13)
    q, qc, kc, vc = inputs()
    lens = torch.tensor([100, 37], dtype=torch.int32, device="cuda")
    good = torch.arange(2 * N, dtype=torch.int32, device="cuda").reshape(2, N) % N
    # an id past the declared pool in an entry no length reaches is never read: accepted
    unused = good.clone()
    unused[1, 5] = N
    kvq.kvq_decode_attention(cache, q, unused, lens, 128)
    for row, col, val in [(0, 6, N), (1, 2, N), (1, 0, -1)]:
        bad = good.clone()
        bad[row, col] = val
        out = torch.full((2, H * G, D), 7.0, device="cuda")
        expect_device_input(kvq.kvq_decode_attention, cache, q, bad, lens, 128, out=out)
        expect_device_input(kvq.kvq_decode_attention_noalloc, cache, q, bad, lens, 128, out)
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
    bad = good.clone()
    bad[0, 3] = N
    kw = torch.full((128, H * D), 3.0, dtype=torch.bfloat16, device="cuda")
    expect_device_input(kvq.kvq_dequant_prefix, cache, bad[0], 100, kw, kw.clone())
    ext = torch.full((20, H * G, D), 5.0, device="cuda")
    expect_device_input(kvq.kvq_extend_attention_paged, cache, bad[0], 100, qc, kc, vc, out=ext)
    torch.cuda.synchronize()
    assert bool((kw == 3.0).all()) and bool((ext == 5.0).all())


def test_sequence_lengths_outside_the_plan_are_rejected(debug):
    print("case: debug mode, seq_lens past max_seq_len and negative", flush=True)
    cache = make_cache()
    fill(cache, 100, seed=14)
    q, _, _, _ = inputs()
    table = torch.arange(2 * N, dtype=torch.int32, device="cuda").reshape(2, N) % N
    for lens in ([100, 97], [-1, 37]):
        lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
        expect_device_input(kvq.kvq_decode_attention, cache, q, table, lt, 96)
    lt = torch.tensor([96, 0], dtype=torch.int32, device="cuda")
    kvq.kvq_decode_attention(cache, q, table, lt, 96)  # the bounds themselves are valid
    torch.cuda.synchronize()
