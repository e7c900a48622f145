"""The measurement calls (include/qift_measure.h) on the GPU: the copy mode
copies every byte (ragged sizes and the bounds-free rounds both), the
read-only mode writes nothing, and the matrix-core loop returns clock
readings that move forward."""
import pytest
import torch

import bit_quantized_fwht_amd as q
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, 256 * 1024 * 16 * 4 + 16 * 7,
                                    (64 << 20) + 16 * 1000])
def test_copy_mode_copies_every_byte(nbytes):
    g = torch.Generator(device=DEV)
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    dst = torch.zeros((nbytes + 64,), dtype=torch.uint8, device=DEV)
    say(f"measure copy {nbytes} B")
    q.qift_measure_stream(src, dst[:nbytes])
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].count_nonzero()) == 0


def test_read_mode_writes_nothing():
    src = torch.full(((8 << 20),), 7, dtype=torch.uint8, device=DEV)
    sink = torch.zeros((q.QIFT_MEASURE_SINK_WORDS,), dtype=torch.int32, device=DEV)
    say("measure read 8 MiB")
    q.qift_measure_stream(src, sink=sink)
    torch.cuda.synchronize()
    assert int(sink.count_nonzero()) == 0


def test_mfma_loop_clock_readings():
    clk = torch.zeros((4,), dtype=torch.int64, device=DEV)
    say("measure mfma 512 workgroups x 256 rounds")
    q.qift_measure_mfma_i8(256, 512, clk)
    torch.cuda.synchronize()
    c = clk.cpu().tolist()
    assert c[2] > c[0] and c[3] > c[1]
    mhz = 100.0 * (c[2] - c[0]) / (c[3] - c[1])
    assert 100.0 < mhz < 5000.0, mhz
