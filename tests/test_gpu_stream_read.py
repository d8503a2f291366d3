"""The bandwidth reference kernel reads every byte it is given: each lane
XORs the 16-byte vectors it reads and sets the sink when the result is the
mark, so one marked vector placed anywhere (including a ragged last block)
must be seen, and two marks read by the same lane must cancel."""
import pytest
import torch

from bit_quantized_kv_amd import kvq

pytestmark = pytest.mark.gpu

MARK = 0x9E3779B9


@pytest.mark.parametrize("n16,where,wgs,want", [
    (256 * 5 + 37, [256 * 5 + 36], 0, 1), (256 * 5 + 37, [3], 2, 1), (4096, [4095], 7, 1), (1, [0], 0, 1),
    (300, [17, 273], 1, 0),   # one workgroup: lane 17 reads both marks, they cancel
    (300, [17, 299], 1, 1),   # different lanes
])
def test_stream_read_sees_every_vector(n16, where, wgs, want):
    print(f"case: stream read n16 {n16} marks {where} wgs {wgs}", flush=True)
    buf = torch.zeros((n16, 4), dtype=torch.int32, device="cuda")
    for i in where:
        buf[i, 1] = MARK - (1 << 32)  # int32 view of the mark
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvq.kvq_stream_read(buf, sink, num_workgroups=wgs)
    torch.cuda.synchronize()
    assert int(sink.item()) == want


@pytest.mark.parametrize("n16,wgs", [(256 * 5 + 37, 0), (1, 0), (4096, 3)])
def test_stream_write_and_copy_touch_exactly_their_bytes(n16, wgs):
    """The write and copy ceiling kernels cover every 16-byte vector of their
    range (a ragged tail included) and nothing past it."""
    print(f"case: stream write/copy n16 {n16} wgs {wgs}", flush=True)
    buf = torch.full((n16 + 8, 4), -1, dtype=torch.int32, device="cuda")
    kvq.kvq_stream_write(buf[:n16], value=0x01020304, num_workgroups=wgs)
    torch.cuda.synchronize()
    assert bool((buf[:n16] == 0x01020304).all()) and bool((buf[n16:] == -1).all())
    src = torch.arange((n16 + 8) * 4, dtype=torch.int32, device="cuda").reshape(n16 + 8, 4)
    dst = torch.full_like(src, -7)
    kvq.kvq_stream_copy(src[:n16], dst[:n16], num_workgroups=wgs)
    torch.cuda.synchronize()
    assert bool((dst[:n16] == src[:n16]).all()) and bool((dst[n16:] == -7).all())


@pytest.mark.parametrize("lds", [0, 1, 2])
def test_mfma_rate_runs_and_leaves_the_sink(lds):
    """The matrix-core ceiling kernel runs to completion through the C-ABI in
    its three operand modes (96 KiB of LDS per workgroup) and stores nothing: its
    accumulated sum is never the 1e-30 that would write the sink."""
    print(f"case: mfma rate lds_operands {lds}", flush=True)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for wgs, iters in ((1, 1), (300, 7)):
        kvq.kvq_mfma_rate(lds, iters, wgs, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
