"""Empty inputs through the FP8 GEMM, the dequant pass and the MXFP8 linear.

Each entry point takes a zero row count (T = 0 tokens, M = 0 rows, N = 0
weight rows or K = 0 columns) as a valid call that returns OK, launches no
kernel (the library's launch counters stay where they were) and writes
nothing: the output passed in is the empty head of a larger buffer filled
with a sentinel, which must come back unchanged.  A non-empty call right
after checks that the empty ones left the library in a working state.
"""

import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from helpers import assert_gemm_close, dev_u8, host_u16, requires_gpu, say
from oracle import gemm as G

pytestmark = [pytest.mark.gpu, requires_gpu]

SENTINEL = -7.0


def _sentinel_out(shape):
    """Empty view at the start of a sentinel-filled BF16 buffer."""
    big = torch.full((4096,), SENTINEL, dtype=torch.bfloat16, device="cuda")
    return big, big[:0].view(shape)


def _untouched(big):
    torch.cuda.synchronize()
    assert torch.all(big.cpu() == SENTINEL).item()


def _u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8, device="cuda")


def test_bmm_zero_tokens():
    say("empty: bmm T=0")
    before = mx.mx_get_counters()
    for G_, N, K in [(1, 16, 128), (16, 1024, 4096), (3, 272, 640)]:
        big, out = _sentinel_out((0, G_, N))
        for fmt in (mx.MX_FP8_E4M3_OCP, mx.MX_FP8_E4M3_FNUZ):
            got = mx.mx_bmm_a8w8_mxscale(_u8(0, G_, K), _u8(0, G_, K // 128), _u8(G_, N, K), _u8(G_, N, K // 128),
                                         fmt, out=out)
            assert tuple(got.shape) == (0, G_, N)
        _untouched(big)
    assert mx.mx_get_counters() == before


@pytest.mark.parametrize("N,K,block", [(0, 64, 32), (0, 512, 128), (16, 0, 32), (0, 0, 128)])
def test_dequant_empty(N, K, block):
    say("empty: dequant", N, K, block)
    before = mx.mx_get_counters()
    big, out = _sentinel_out((N, K))
    got = mx.mx_dequant_mxfp8_to_bf16(_u8(N, K), _u8(N, K // block), block, out=out)
    assert tuple(got.shape) == (N, K)
    _untouched(big)
    assert mx.mx_get_counters() == before


# M = 0 on each branch (BF16 weight, FP8 weight at a K the block-scaled GEMM
# takes, FP8 weight at a K it does not), and N = 0 on the block-scaled branch.
@pytest.mark.parametrize("M,N,K,fp8", [(0, 64, 576, False), (0, 64, 2048, True), (0, 64, 576, True),
                                       (8, 0, 2048, True)])
def test_linear_empty(M, N, K, fp8):
    say("empty: linear", M, N, K, fp8)
    before = mx.mx_get_counters()
    big, out = _sentinel_out((M, N))
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    if fp8:
        got = mx.mx_linear(x, _u8(N, K), _u8(N, K // mx.MX_LINEAR_BLOCK), out=out)
    else:
        got = mx.mx_linear(x, torch.zeros((N, K), dtype=torch.bfloat16, device="cuda"), out=out)
    assert tuple(got.shape) == (M, N)
    _untouched(big)
    assert mx.mx_get_counters() == before


def test_working_after_empty_calls():
    T, Gn, N, K = 70, 2, 48, 256
    say("empty: bmm after empty calls", T, Gn, N, K)
    mx.mx_bmm_a8w8_mxscale(_u8(0, Gn, K), _u8(0, Gn, K // 128), _u8(Gn, N, K), _u8(Gn, N, K // 128))
    a, sa, w, sw = workloads.gemm_operands(4242, T, Gn, N, K)
    out = mx.mx_bmm_a8w8_mxscale(dev_u8(a), dev_u8(sa), dev_u8(w), dev_u8(sw))
    torch.cuda.synchronize()
    assert_gemm_close(host_u16(out), G.bmm_a8w8_mxscale(a, sa, w, sw), "after empty calls")
