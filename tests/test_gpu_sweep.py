"""GPU parity over a seeded sweep of shapes, across every dispatch path.

Each case draws its shape from a fixed seed, so the sweep is the same on every
run.  Paths covered: the batched FP8 GEMM's small-T, decode-batch, one-tile
and persistent kernels (OCP and FNUZ activations), the MXFP8 linear's three
branches over M, N and K, and the BF16 arm's GEMM on both small-T kernels and
the persistent tiles.  Bound: the GEMM bound of helpers.assert_gemm_close.
"""

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from helpers import assert_gemm_close, dev_u16, dev_u8, host_u16, requires_gpu, say
from oracle import formats as F
from oracle import gemm as G

pytestmark = [pytest.mark.gpu, requires_gpu]


def _bmm_cases():
    rng = np.random.default_rng(2024)
    cases = []
    for i in range(24):
        kind = i % 4
        if kind == 0:      # small T, any K
            T, K = int(rng.integers(1, 65)), 128 * int(rng.integers(1, 6))
        elif kind == 1:    # decode-batch kernel
            T, K = int(rng.integers(1, 65)), int(rng.choice([1024, 2048, 4096, 8192]))
        elif kind == 2:    # one-tile-per-workgroup kernel
            T, K = int(rng.integers(65, 700)), 128 * int(rng.choice([1, 3, 5, 7, 10]))
        else:              # persistent kernel
            T, K = int(rng.integers(65, 1500)), int(rng.choice([2048, 4096]))
        G_ = int(rng.integers(1, 4))
        N = 16 * int(rng.integers(1, 40))
        fnuz = bool(rng.integers(0, 2))
        cases.append((i, T, G_, N, K, fnuz))
    return cases


@pytest.mark.parametrize("i,T,Gn,N,K,fnuz", _bmm_cases())
def test_bmm_sweep(i, T, Gn, N, K, fnuz):
    a, sa, w, sw = workloads.gemm_operands(7000 + i, T, Gn, N, K)
    if fnuz:                                   # the same values as FNUZ bytes: scale + 1, -0 -> 0
        a = np.where(a == 0x80, 0, a).astype(np.uint8)
        sa = (sa.astype(int) + 1).astype(np.uint8)
    fmt = mx.MX_FP8_E4M3_FNUZ if fnuz else mx.MX_FP8_E4M3_OCP
    say("sweep bmm", i, T, Gn, N, K, "fnuz" if fnuz else "ocp")
    out = mx.mx_bmm_a8w8_mxscale(dev_u8(a), dev_u8(sa), dev_u8(w), dev_u8(sw), fmt)
    torch.cuda.synchronize()
    rows = np.unique(np.random.default_rng(i).integers(0, T, 24)) if T > 256 else np.arange(T)
    ref = G.bmm_a8w8_mxscale(a[rows], sa[rows], w, sw, a_fmt=F.FNUZ if fnuz else F.OCP)
    assert_gemm_close(host_u16(out)[rows], ref, f"case {i}: T={T} G={Gn} N={N} K={K}")


def _linear_cases():
    rng = np.random.default_rng(2025)
    cases = []
    for i in range(16):
        M = int(rng.choice([1, 3, 8, 16, 17, 40, 64]))
        N = 16 * int(rng.integers(1, 80))
        # even cases: K % 128 == 0 (block-scaled FP8 branch); odd: K % 128 != 0 (BF16 branches)
        K = 128 * int(rng.integers(1, 24)) if i % 2 == 0 else 32 * (4 * int(rng.integers(0, 20)) + int(rng.integers(1, 4)))
        cases.append((i, M, N, K))
    return cases


@pytest.mark.parametrize("i,M,N,K", _linear_cases())
def test_linear_sweep(i, M, N, K):
    rng = np.random.default_rng(8000 + i)
    x = workloads.activations(rng, M, K)
    w = workloads.weight_codes(rng, (N, K))
    ws = workloads.scale_bytes(rng, (N, K // 32), -10, -4)
    dx, dw, dws = dev_u16(x), dev_u8(w), dev_u8(ws)
    say("sweep linear", i, M, N, K)
    ref = G.mx_linear(x, w, ws, 32)
    if K % 128:
        once = mx.mx_linear(dx, mx.mx_dequant_mxfp8_to_bf16(dw, dws), dws)
        percall = mx.mx_linear(dx, dw, dws)
        torch.cuda.synchronize()
        assert_gemm_close(host_u16(once), ref, f"case {i}: M={M} N={N} K={K} (bf16)")
        assert np.array_equal(host_u16(percall), host_u16(once))
    else:
        out = mx.mx_linear(dx, dw, dws)
        torch.cuda.synchronize()
        assert_gemm_close(host_u16(out), ref, f"case {i}: M={M} N={N} K={K} (fp8)")


def _bf16_cases():
    rng = np.random.default_rng(2026)
    cases = []
    for i in range(12):
        kind = i % 3
        if kind == 0:
            T, K = int(rng.integers(1, 65)), 128 * int(rng.integers(1, 5))
        elif kind == 1:
            T, K = int(rng.integers(1, 65)), int(rng.choice([512, 1024, 2048, 4096]))
        else:
            T, K = int(rng.integers(65, 900)), 128 * int(rng.integers(1, 12))
        cases.append((i, T, int(rng.integers(1, 4)), 16 * int(rng.integers(1, 40)), K))
    return cases


@pytest.mark.parametrize("i,T,Gn,N,K", _bf16_cases())
def test_bmm_bf16_sweep(i, T, Gn, N, K):
    rng = np.random.default_rng(9000 + i)
    x = workloads.activations(rng, T * Gn, K).reshape(T, Gn, K)
    w = workloads.activations(rng, Gn * N, K).reshape(Gn, N, K)
    say("sweep bf16", i, T, Gn, N, K)
    out = mx.mx_bmm_bf16(dev_u16(x), dev_u16(w))
    torch.cuda.synchronize()
    rows = np.unique(np.random.default_rng(i).integers(0, T, 24)) if T > 256 else np.arange(T)
    assert_gemm_close(host_u16(out)[rows], G.bmm_bf16(x[rows], w), f"case {i}: T={T} G={Gn} N={N} K={K}")
