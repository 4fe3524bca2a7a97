"""Wrong-shaped GPU tensors are refused by the binding with ValueError before
anything is launched (the launch counters do not move)."""

import pytest
import torch

import mx_scaled_fp8_amd as mx
from helpers import requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def _z(*shape, dtype=torch.uint8):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_wrong_shapes_raise_before_launch():
    mx.mx_reset_counters()
    before = mx.mx_get_counters()
    say("binding: wrong-shaped GPU tensors")
    T, G, N, K = 4, 2, 32, 256
    with pytest.raises(ValueError, match="w has shape"):
        mx.mx_bmm_a8w8_mxscale(_z(T, G, K), _z(T, G, 2), _z(G, N, K - 128), _z(G, N, 2))
    with pytest.raises(ValueError, match="a_scale has"):
        mx.mx_bmm_a8w8_mxscale(_z(T, G, K), _z(T, G, 1), _z(G, N, K), _z(G, N, 2))
    cs = _z(64, 32, dtype=torch.int16)
    with pytest.raises(ValueError, match="positions has"):
        mx.mx_inv_rope_group_quant(_z(T, 512, dtype=torch.int16), _z(T + 1, dtype=torch.int64), cs, cs, 4, 128, 64)
    with pytest.raises(ValueError, match="int64"):
        mx.mx_inv_rope_group_quant(_z(T, 512, dtype=torch.int16), _z(T, dtype=torch.int32), cs, cs, 4, 128, 64)
    with pytest.raises(ValueError, match="w_scale has"):
        mx.mx_linear(_z(8, 1152, dtype=torch.int16), _z(64, 1152), _z(64, 9))
    with pytest.raises(ValueError, match="out has"):
        mx.mx_dequant_mxfp8_to_bf16(_z(64, 576), _z(64, 18), out=_z(64, 288, dtype=torch.int16))
    torch.cuda.synchronize()
    assert mx.mx_get_counters() == before
