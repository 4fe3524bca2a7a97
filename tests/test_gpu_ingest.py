"""GPU parity of mx_woa_expand_scales (checkpoint scale ingestion) against the oracle.

* E8M0 scales per (g, n, 128-K block) pass through; 128 x 128 block scales
  expand over their rows, with a ragged last block (N = 300).
* FP32 power-of-two scales give the oracle's bytes; scales that are not
  powers of two in range give 0xFF and are counted once per source scale.
* At the production shape (G = 16, N = 1024, K = 4096, FP32 scales per
  128 x 128 block) the expanded bytes equal the oracle's, and the decode-batch
  GEMM on them meets the GEMM bound against the oracle.
All byte comparisons are exact.
"""

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from helpers import assert_gemm_close, dev_u8, host_u16, host_u8, requires_gpu, say
from oracle import gemm as Gm
from oracle.ingest import E8M0, F32, expand_woa_scales

pytestmark = [pytest.mark.gpu, requires_gpu]


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("block_n", [1, 128])
def test_e8m0_layouts(block_n):
    G, N, K = 3, 300, 512
    nb = -(-N // block_n)
    s = workloads.scale_bytes(np.random.default_rng(block_n), (G, nb, K // 128), -10, 10)
    say("expand e8m0", block_n)
    out, rej = mx.mx_woa_expand_scales(dev_u8(s), G, N, K, block_n)
    torch.cuda.synchronize()
    want, ok = expand_woa_scales(s, E8M0, block_n, G, N, K)
    assert rej == 0 and ok.all()
    assert np.array_equal(host_u8(out), want)


@pytest.mark.parametrize("block_n", [1, 128])
def test_f32_scales_and_rejects(block_n):
    G, N, K = 2, 300, 1024
    nb = -(-N // block_n)
    rng = np.random.default_rng(10 + block_n)
    s = np.ldexp(np.float32(1), rng.integers(-127, 128, (G, nb, K // 128))).astype(np.float32)
    bad = [3.0, 0.0, -1.0, np.nan, np.inf, -np.inf, 2.0 ** -128, 1.5, -2.0 ** -127, 2.0 ** -149]
    flat = s.reshape(-1)
    picks = rng.choice(flat.size, len(bad), replace=False)
    flat[picks] = np.array(bad, dtype=np.float32)
    say("expand f32", block_n)
    out, rej = mx.mx_woa_expand_scales(_f32(s), G, N, K, block_n)
    torch.cuda.synchronize()
    want, ok = expand_woa_scales(s, F32, block_n, G, N, K)
    got = host_u8(out)
    assert np.array_equal(got[ok], want[ok])
    assert np.all(got[~ok] == 0xFF)
    assert rej == len(bad)


def test_production_shape_and_gemm():
    G, N, K, T = 16, 1024, 4096, 64
    rng = np.random.default_rng(40)
    w = workloads.weight_codes(rng, (G, N, K))
    s = np.ldexp(np.float32(1), rng.integers(-8, -3, (G, N // 128, K // 128))).astype(np.float32)
    a, sa, _, _ = workloads.gemm_operands(41, T, G, 16, K)
    say("expand production + decode GEMM")
    sw, rej = mx.mx_woa_expand_scales(_f32(s), G, N, K, 128)
    out = mx.mx_bmm_a8w8_mxscale(dev_u8(a), dev_u8(sa), dev_u8(w), sw)
    torch.cuda.synchronize()
    want, ok = expand_woa_scales(s, F32, 128, G, N, K)
    assert rej == 0 and ok.all()
    assert np.array_equal(host_u8(sw), want)
    assert_gemm_close(host_u16(out), Gm.bmm_a8w8_mxscale(a, sa, w, want), "decode GEMM on expanded scales")
