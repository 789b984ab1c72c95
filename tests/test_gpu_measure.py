"""The streaming-read helper used for the read ceiling: it launches, reads
every byte it is given (sizes of one partial workgroup, several, and a ragged
tail) and leaves its sink alone for data that does not hit the guard word."""

import pytest
import torch

import dequant_gemv_rht_amd as dq

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 8192, 8192 * 3 + 48, 1 << 24])
def test_stream_read_runs(nbytes):
    say(f"stream_read {nbytes} bytes")
    src = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    dq.stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


def test_stream_read_rejects_misaligned():
    src = torch.zeros(64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(dq.WqError):
        dq.stream_read(src[1:], sink, 16)
