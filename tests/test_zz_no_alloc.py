"""kvq_decode_attention_noalloc -- the decode entry point for callers that
cannot allocate -- through the C ABI against kvq_decode_attention with a
caller workspace: the same kernels and split plan over the library's static
scratch, so outputs and lse must be equal bit for bit.  Two calls in a row,
the second with a smaller batch and context (the scratch then holds the first
call's partials), in both output dtypes and both 4-bit formats; a shape whose
partials exceed the scratch is refused before any launch."""
import numpy as np
import pytest
import torch

from bit_quantized_kv_amd import kvq
from gpu_cases import Case, check_attention

pytestmark = pytest.mark.gpu


def _both(c, out_dtype, num_splits):
    """(workspace entry point, no-allocation entry point) outputs and lse."""
    lse_ws = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    ws = kvq.kvq_decode_attention(c.cache, c.q_dev, c.bt_dev, c.lens_dev, c.max_len, lse=lse_ws,
                                  num_splits=num_splits, out_dtype=out_dtype)
    out = torch.full((c.B, c.Hq, c.D), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((c.B, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attention_noalloc(c.cache, c.q_dev, c.bt_dev, c.lens_dev, c.max_len, out, lse=lse,
                                     num_splits=num_splits)
    torch.cuda.synchronize()
    return ws.float().cpu().numpy(), lse_ws.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("fmt", [1, 2])
def test_noalloc_decode_equals_workspace_decode(fmt):
    print(f"case: no-allocation decode fmt {fmt}", flush=True)
    # first call: 3 sequences up to 3,000 tokens over 2 KV heads (G 6); second:
    # one 200-token sequence, so it reads far less scratch than the first wrote
    big = Case(fmt, 256, 2, 6, 16, [3000, 1234, 0], kind="lognormal", in_dtype=torch.bfloat16, seed=70 + fmt)
    small = Case(fmt, 256, 1, 4, 16, [200], kind="student_t", in_dtype=torch.bfloat16, seed=80 + fmt)
    for c, splits in ((big, 0), (small, 3)):
        for dt in (torch.float32, torch.bfloat16):
            a, la, b, lb = _both(c, dt, splits)
            assert np.array_equal(a, b), f"outputs differ ({dt}, splits {splits}): max {np.abs(a - b).max()}"
            assert np.array_equal(la, lb), f"lse differs ({dt}, splits {splits})"
    # and the last call against the oracle, at the decode bar
    ref, ref_lse = small.oracle_decode()
    _, _, b, lb = _both(small, torch.float32, 0)
    check_attention(b, ref, small.lens, lse=lb, ref_lse=ref_lse, label="no-allocation decode vs oracle")


def test_noalloc_refuses_shapes_beyond_its_scratch():
    print("case: no-allocation decode, oversized plan", flush=True)
    c = Case(1, 256, 1, 4, 16, [64], kind="outliers", seed=90)
    out = torch.empty((c.B, c.Hq, c.D), dtype=torch.float32, device="cuda")
    bt = torch.zeros((1, 8192), dtype=torch.int32, device="cuda")  # room for a 131,072-token bound
    # 4,096 splits x 4 query heads x (256 + 2) floats = 16.9 MB of partials > 16 MiB
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attention_noalloc(c.cache, c.q_dev, bt, c.lens_dev, 4096 * 32, out, num_splits=4096)
    assert e.value.status == -7
