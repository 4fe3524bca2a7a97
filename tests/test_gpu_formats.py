"""GPU: the device format converters against the oracle, exhaustively.

Every BF16 pattern, scaled by powers of two across the e4m3 range (normals,
subnormals, ties, underflow, saturation), goes through the device e4m3
encoders -- the same hardware conversion the quantiser uses -- and must equal
the oracle byte for byte.  The device FP32 -> E8M0 converter is checked on
every power of two and on random patterns, with the reject count.
"""

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
from helpers import requires_gpu, say
from oracle import formats as F

pytestmark = [pytest.mark.gpu, requires_gpu]


def _grid():
    base = F.bf16_to_f32(np.arange(0x10000, dtype=np.uint16)).astype(np.float64)
    parts = []
    for k in (-140, -20, -12, -10, -9, -8, -6, -3, 0, 2, 4, 6, 8, 9, 10):
        v = np.ldexp(base, k)
        parts.append(v.astype(np.float32))
    edge = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 448, 464, 465, 480, 1e38, 224, 232, 240, 241,
                     2.0 ** -149, -2.0 ** -149], np.float32)
    return np.concatenate(parts + [edge])


@pytest.mark.parametrize("fmt,code", [(F.OCP, mx.MX_FP8_E4M3_OCP), (F.FNUZ, mx.MX_FP8_E4M3_FNUZ)])
def test_device_e4m3_encoder_exhaustive(fmt, code):
    v = _grid()
    say("device e4m3 encoder", fmt, v.size)
    out = mx.mx_f32_to_e4m3_device(torch.from_numpy(v).cuda(), code).cpu().numpy()
    ref = F.e4m3_encode(v.astype(np.float64), fmt)
    bad = np.flatnonzero(out != ref)
    assert bad.size == 0, [(float(v[i]), hex(out[i]), hex(ref[i])) for i in bad[:10]]


def test_device_e8m0_converter():
    n = np.arange(-127, 128)
    powers = np.ldexp(np.ones(n.size, np.float32), n).astype(np.float32)
    rng = np.random.default_rng(5)
    rand = rng.integers(0, 2 ** 32, 100_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    v = np.concatenate([powers, rand])
    say("device e8m0 converter", v.size)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = mx.mx_f32_pow2_to_e8m0_device(torch.from_numpy(v).cuda(), reject_count=cnt).cpu().numpy()
    ref, ok = F.f32_pow2_to_e8m0(v)
    assert np.array_equal(out[ok], ref[ok])
    assert np.all(out[~ok] == 0xFF)
    assert int(cnt.item()) == int((~ok).sum())
