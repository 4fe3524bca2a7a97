"""The MXFP8 linear at prefill-sized M (more rows than a decode batch) against
the oracle, every output: M in {65, 1000, 8192}, the pages' production
N = 5120, K in {288, 576} (weight dequantised once at load, BF16 GEMM; one
case also unprepared, dequantised per call) and K in {1152, 2304} (x
quantised to MXFP8 block 32, block-scaled FP8 GEMM on 256 x 256 tiles with
block-32 scales).  The launch counters show the branch each call took."""

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from helpers import assert_gemm_close, dev_u16, dev_u8, host_u16, requires_gpu, say
from oracle import gemm as G

pytestmark = [pytest.mark.gpu, requires_gpu, pytest.mark.timeout(600)]

N = 5120


def _case(M, K, n=N):
    rng = np.random.default_rng(7000 + M + K + n)
    x = workloads.activations(rng, M, K)
    w = workloads.weight_codes(rng, (n, K))
    ws = workloads.scale_bytes(rng, (n, K // 32), -10, -4)
    return x, w, ws


@pytest.mark.parametrize("K", [288, 576, 1152, 2304])
@pytest.mark.parametrize("M", [65, 1000, 8192])
def test_linear_large_m_every_output(M, K):
    x, w, ws = _case(M, K)
    xd, wd, wsd = dev_u16(x), dev_u8(w), dev_u8(ws)
    if mx.mx_linear_dequant_at_load(K):
        wd = mx.mx_dequant_mxfp8_to_bf16(wd, wsd)
    say("linear large M", M, N, K)
    mx.mx_reset_counters()
    out = mx.mx_linear(xd, wd, wsd)
    torch.cuda.synchronize()
    c = mx.mx_get_counters()
    assert c["linear_bf16" if K % 128 else "linear_fp8"] == 1
    assert_gemm_close(host_u16(out), G.mx_linear(x, w, ws, 32), f"M={M} N={N} K={K}")


def test_linear_large_m_unprepared_weight():
    M, K = 1000, 576
    x, w, ws = _case(M, K)
    say("linear large M, unprepared FP8 weight", M, N, K)
    mx.mx_reset_counters()
    out = mx.mx_linear(dev_u16(x), dev_u8(w), dev_u8(ws))
    torch.cuda.synchronize()
    c = mx.mx_get_counters()
    assert c["linear_percall_dequant"] == 1 and c["linear_fp8"] == 0
    assert_gemm_close(host_u16(out), G.mx_linear(x, w, ws, 32), f"unprepared M={M} K={K}")


def test_block32_tiles_match_ring_kernel_at_64_rows():
    """The same 64 rows through the decode-batch kernel (M = 64) and, as part
    of a 65-row call, through the 256 x 256 tiles: identical first 64 rows
    are not required (different accumulation order), but both lie within the
    bound of the same oracle rows."""
    K = 2304
    x, w, ws = _case(65, K)
    wd, wsd = dev_u8(w), dev_u8(ws)
    say("linear 64 rows vs 65 rows", K)
    a = mx.mx_linear(dev_u16(x[:64]), wd, wsd)
    b = mx.mx_linear(dev_u16(x), wd, wsd)
    torch.cuda.synchronize()
    ref = G.mx_linear(x, w, ws, 32)
    assert_gemm_close(host_u16(a), ref[:64], "64 rows, decode kernels")
    assert_gemm_close(host_u16(b), ref, "65 rows, tiled kernel")


@pytest.mark.parametrize("M,n,K", [(200, 1040, 288), (3000, 400, 96), (129, 16, 32), (8192, 272, 576)])
def test_bf16_tiles_ragged_m_and_n(M, n, K):
    """The BF16 branch's tiled kernel where neither M nor N fills its tiles
    (both tile widths: 128 x 128 and 128 x 256), down to one 32-element K
    step and a single 16-column weight."""
    x, w, ws = _case(M, K, n)
    wd = mx.mx_dequant_mxfp8_to_bf16(dev_u8(w), dev_u8(ws))
    say("linear BF16 tiles, ragged", M, n, K)
    out = mx.mx_linear(dev_u16(x), wd)
    torch.cuda.synchronize()
    assert_gemm_close(host_u16(out), G.mx_linear(x, w, ws, 32), f"M={M} N={n} K={K}")
