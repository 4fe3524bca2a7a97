"""The inverse-RoPE rounding cases of tests/golden/rope_rounding_cases.txt on
the GPU: inputs whose BF16 result is decided by the fp32 rounding of the
rotation's sum (derived in exact rationals).  The BF16 rotation must give the
golden bits, and the fused quantiser must give the codes and scales of the
golden rotated values, bit for bit.
"""

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from conftest import read_golden
from helpers import dev_i64, dev_u16, host_u16, host_u8, requires_gpu, say
from oracle import formats as F
from oracle.quant import group_quant
from oracle.rope import inverse_rope, pair_indices, INTERLEAVED, NEOX

pytestmark = [pytest.mark.gpu, requires_gpu]

ROWS = read_golden("rope_rounding_cases.txt")
STYLE = {INTERLEAVED: mx.MX_ROPE_INTERLEAVED, NEOX: mx.MX_ROPE_NEOX}


def _batch(style, D=128, R=64):
    """One token per case (H = 1, D = 128, the case's pair in the rotated
    half, the other dims a fixed filler) and the expected rotated BF16 rows:
    the oracle's rotation, whose bits at the case's pair are the golden ones."""
    i0, i1 = pair_indices(D, R, style)
    T = len(ROWS)
    x = np.full((T, D), 0x3F00, np.uint16)          # 0.5 in every other dim
    pos = np.zeros(T, np.int64)
    for t, row in enumerate(ROWS):
        i = int(row[1])
        pos[t] = int(row[0])
        x[t, i0[i]], x[t, i1[i]] = int(row[4], 16), int(row[5], 16)
    cos, sin = workloads.rope_tables(rows=8)
    want = inverse_rope(x, pos, cos, sin, 1, D, R, style)
    for t, row in enumerate(ROWS):
        i = int(row[1])
        assert (want[t, i0[i]], want[t, i1[i]]) == (int(row[6], 16), int(row[7], 16))
    return x, pos, want


@pytest.mark.parametrize("style", [INTERLEAVED, NEOX])
def test_bf16_rotation_golden_bits(style):
    cos, sin = workloads.rope_tables(rows=8)
    x, pos, want = _batch(style)
    say("rope rounding golden, bf16 rotation", style)
    out = mx.mx_inv_rope_bf16(dev_u16(x), dev_i64(pos), dev_u16(cos), dev_u16(sin), 1, 128, 64, STYLE[style])
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(out), want)


@pytest.mark.parametrize("fmt", [F.OCP, F.FNUZ])
@pytest.mark.parametrize("style", [INTERLEAVED, NEOX])
def test_fused_quantiser_golden(style, fmt):
    cos, sin = workloads.rope_tables(rows=8)
    x, pos, want = _batch(style)
    say("rope rounding golden, fused quantiser", style, fmt)
    q, s = mx.mx_inv_rope_group_quant(dev_u16(x), dev_i64(pos), dev_u16(cos), dev_u16(sin), 1, 128, 64,
                                      STYLE[style], 32, mx.MX_FP8_E4M3_OCP if fmt == F.OCP else mx.MX_FP8_E4M3_FNUZ)
    torch.cuda.synchronize()
    rq, rs = group_quant(want, 32, fmt)
    assert np.array_equal(host_u8(s), rs)
    assert np.array_equal(host_u8(q), rq)
