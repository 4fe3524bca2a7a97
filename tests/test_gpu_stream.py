"""The read-only stream that weight-streaming calls are timed against: it
reaches every 16-byte vector of its buffer (a vector whose words XOR to the
kernel's fixed value makes the lane that read it store that value; placed at
the first, a middle and the last vector, past one grid-stride round), and
otherwise writes nothing."""

import pytest
import torch

import mx_scaled_fp8_amd as mx
from helpers import requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

MAGIC = 0x9E3779B9


@pytest.mark.parametrize("nvec", [1, 1000, 2048 * 2048 + 37])
def test_stream_read_reaches_every_vector(nvec):
    say("stream read", nvec)
    buf = torch.zeros((nvec, 4), dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    mx.mx_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0                                  # zeros: nothing written
    for at in sorted({0, nvec // 2, nvec - 1}):
        buf.zero_()
        sink.zero_()
        buf[at, 2] = torch.tensor(MAGIC, dtype=torch.int64).to(torch.int32)   # one lane's words XOR to the value
        mx.mx_stream_read(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) & 0xFFFFFFFF == MAGIC, f"vector {at} of {nvec} not read"


def test_stream_read_refuses_ragged_bytes():
    with pytest.raises(ValueError, match="multiple of 16"):
        mx.mx_stream_read(torch.zeros(3, dtype=torch.int32, device="cuda"), torch.zeros(1, dtype=torch.int32,
                                                                                          device="cuda"))
