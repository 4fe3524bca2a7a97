"""GPU parity of the MXFP8 dequantiser and the MXFP8 linear.

* Dequantisation is bit-exact against the oracle (the product of an e4m3
  value and a power of two is exact, only the BF16 rounding remains), for the
  linear's K = 288 / 576 and the pages' 5120 x 576 production shape.
* mx_linear on every K of the MXFP8-linear workload: the BF16 branch on a
  weight dequantised at load (K = 288, 576), the block-scaled FP8 branch
  (K = 1152, 2304), within the GEMM bound of the matching oracle branch.
* The unaligned FP8 weight that was not prepared takes the per-call
  dequantisation branch: its output equals the load-time branch bit for bit,
  and the launch counters show that the scaled GEMM was never reached (the
  review thread of the MXFP8 page asks for exactly these two checks).
* The converter turns the FP32 power-of-two scales into the same E8M0 bytes.
* The pages' production layer, the shared expert's down_proj (N = 5120) at
  each tensor-parallel share of K = 2304 (TP1/2/4/8: K = 2304, 1152, 576,
  288), decode batches of 1 and 8 rows: every branch the K allows.
* Every row/K class of the block-scaled kernels (x quantised inside the GEMM
  for up to 16 rows; the weight-resident GEMM; the ring kernels beyond), rows
  past M left untouched, NaN blocks on either operand.
* The identity as the FP8 weight makes each output one dequantised x code:
  the codes and scales made for x are checked bit for bit against the oracle.
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


@pytest.fixture(scope="module")
def data():
    return workloads.mxfp8_linear()


@pytest.mark.parametrize("K", [288, 576])
def test_dequant_bit_exact(data, K):
    _, w, ws, _ = data[K]
    say("dequant", K)
    out = host_u16(mx.mx_dequant_mxfp8_to_bf16(dev_u8(w), dev_u8(ws)))
    assert np.array_equal(out, G.dequant_mxfp8_to_bf16(w, ws, 32))


def test_dequant_production_shape():
    rng = np.random.default_rng(21)
    w = workloads.weight_codes(rng, (5120, 576))
    ws = workloads.scale_bytes(rng, (5120, 18), -10, -4)
    out = host_u16(mx.mx_dequant_mxfp8_to_bf16(dev_u8(w), dev_u8(ws)))
    assert np.array_equal(out, G.dequant_mxfp8_to_bf16(w, ws, 32))


def test_dequant_block128_and_nan():
    rng = np.random.default_rng(22)
    w = workloads.weight_codes(rng, (64, 256))
    w[0, 0] = 0x7F
    ws = workloads.scale_bytes(rng, (64, 2), -10, 10)
    ws[1, 1] = 0xFF
    out = host_u16(mx.mx_dequant_mxfp8_to_bf16(dev_u8(w), dev_u8(ws), block=128))
    ref = G.dequant_mxfp8_to_bf16(w, ws, 128)
    nan = np.isnan(F.bf16_to_f64(ref))
    assert np.array_equal(np.isnan(F.bf16_to_f64(out)), nan) and nan.sum() == 1 + 128
    assert np.array_equal(out[~nan], ref[~nan])


@pytest.mark.parametrize("K", workloads.LINEAR_KS)
def test_linear_each_k(data, K):
    x, w, ws, ws_f32 = data[K]
    # load time: FP32 power-of-two scales -> E8M0 (host converter), then
    # dequantise once iff K % 128 != 0
    sb, ok = mx.mx_f32_pow2_to_e8m0(ws_f32)
    assert ok and np.array_equal(sb, ws)
    dw = dev_u8(w)
    dws = dev_u8(sb)
    prepared = mx.mx_dequant_mxfp8_to_bf16(dw, dws) if mx.mx_linear_dequant_at_load(K) else dw
    mx.mx_reset_counters()
    say("mx_linear", K)
    out = host_u16(mx.mx_linear(dev_u16(x), prepared, dws))
    c = mx.mx_get_counters()
    ref = G.mx_linear(x, w, ws, 32)
    assert_gemm_close(out, ref, f"K={K}")
    if K % 128:
        assert c["linear_bf16"] == 1 and c["linear_fp8"] == 0
    else:
        assert c["linear_fp8"] == 1 and c["linear_bf16"] == 0


@pytest.mark.parametrize("K", [288, 576])
def test_unprepared_unaligned_weight_never_reaches_scaled_gemm(data, K):
    x, w, ws, _ = data[K]
    dx, dw, dws = dev_u16(x), dev_u8(w), dev_u8(ws)
    loaded = mx.mx_linear(dx, mx.mx_dequant_mxfp8_to_bf16(dw, dws), dws)
    mx.mx_reset_counters()
    say("mx_linear per-call dequant", K)
    percall = mx.mx_linear(dx, dw, dws)
    c = mx.mx_get_counters()
    assert c["linear_percall_dequant"] == 1 and c["linear_fp8"] == 0
    assert np.array_equal(host_u16(percall), host_u16(loaded))


def test_aligned_control_k2048():
    """K = 2048 is the aligned control that keeps reaching the scaled path."""
    rng = np.random.default_rng(23)
    x = workloads.activations(rng, 64, 2048)
    w = workloads.weight_codes(rng, (256, 2048))
    ws = workloads.scale_bytes(rng, (256, 64), -10, -4)
    mx.mx_reset_counters()
    out = host_u16(mx.mx_linear(dev_u16(x), dev_u8(w), dev_u8(ws)))
    assert mx.mx_get_counters()["linear_fp8"] == 1
    assert_gemm_close(out, G.mx_linear(x, w, ws, 32), "K=2048")


@pytest.mark.parametrize("K", [1024, 3072, 4096, 8192])
def test_linear_fp8_other_k(K):
    """Block-scaled branch at K that take the run-time stage count (and the
    deepest K the scale rows allow)."""
    rng = np.random.default_rng(K)
    x = workloads.activations(rng, 64, K)
    w = workloads.weight_codes(rng, (272, K))
    ws = workloads.scale_bytes(rng, (272, K // 32), -10, -4)
    say("mx_linear fp8", K)
    out = host_u16(mx.mx_linear(dev_u16(x), dev_u8(w), dev_u8(ws)))
    assert_gemm_close(out, G.mx_linear(x, w, ws, 32), f"K={K}")


@pytest.mark.parametrize("M", [1, 5, 16, 17, 33, 64])
def test_linear_small_m(M):
    rng = np.random.default_rng(30 + M)
    for K in (288, 1152):
        x = workloads.activations(rng, M, K)
        w = workloads.weight_codes(rng, (128, K))
        ws = workloads.scale_bytes(rng, (128, K // 32), -10, -4)
        out = host_u16(mx.mx_linear(dev_u16(x), dev_u8(w), dev_u8(ws)))
        assert_gemm_close(out, G.mx_linear(x, w, ws, 32), f"M={M} K={K}")


@pytest.fixture(scope="module")
def shards():
    return workloads.down_proj_shards()


@pytest.mark.parametrize("M", [1, 8])
@pytest.mark.parametrize("tp", workloads.DOWN_PROJ_TP)
def test_down_proj_production_shares(shards, tp, M):
    x, w, ws = shards[tp]
    x = x[:M]
    K = w.shape[1]
    dx, dw, dws = dev_u16(x), dev_u8(w), dev_u8(ws)
    ref = G.mx_linear(x, w, ws, 32)
    say("down_proj share", tp, K, M)
    if K % 128:
        once = host_u16(mx.mx_linear(dx, mx.mx_dequant_mxfp8_to_bf16(dw, dws), dws))
        assert_gemm_close(once, ref, f"TP{tp} K={K} M={M} dequant once")
        percall = host_u16(mx.mx_linear(dx, dw, dws))
        assert np.array_equal(percall, once)
    else:
        out = host_u16(mx.mx_linear(dx, dw, dws))
        assert_gemm_close(out, ref, f"TP{tp} K={K} M={M} fp8")


# Every shape class of the block-scaled branch's weight-resident GEMM: 1..16
# rows (the waves split K into quarters; some quarters empty when K / 128 < 4
# or ragged), 17..64 rows (one token tile per wave, K / 128 up to 18), and the
# ring kernel beyond that (K / 128 = 19, 32).  N = 48: three workgroups.
WRES_CASES = [(1, 1), (7, 2), (16, 3), (1, 4), (5, 5), (16, 9), (3, 13), (16, 18), (9, 29), (1, 33), (16, 48),
              (2, 61), (16, 64), (17, 1), (40, 2), (64, 5), (33, 9), (64, 17), (17, 18), (64, 18), (40, 19),
              (64, 32)]


@pytest.mark.parametrize("M,KB", WRES_CASES)
def test_linear_fp8_row_and_k_classes(M, KB):
    K, N = 128 * KB, 48
    rng = np.random.default_rng(1000 * M + KB)
    x = workloads.activations(rng, M, K)
    w = workloads.weight_codes(rng, (N, K))
    ws = workloads.scale_bytes(rng, (N, K // 32), -10, -4)
    say("mx_linear fp8 shape class", M, K)
    # rows past M of the output buffer must stay untouched
    big = torch.full((M + 3, N), -7.0, dtype=torch.bfloat16, device="cuda")
    mx.mx_linear(dev_u16(x), dev_u8(w), dev_u8(ws), out=big[:M])
    got = host_u16(big)
    assert np.all(got[M:] == host_u16(torch.full((1,), -7.0, dtype=torch.bfloat16)).item())
    assert_gemm_close(got[:M], G.mx_linear(x, w, ws, 32), f"M={M} K={K}")


@pytest.mark.parametrize("M,KB", [(5, 9), (64, 18), (16, 40)])
def test_linear_fp8_nan_blocks(M, KB):
    """A NaN in x gives its block NaN codes and the 0xFF scale, so the whole
    output row is NaN; a 0xFF weight scale makes its output column NaN; the
    rest stays within the bound."""
    K, N = 128 * KB, 48
    rng = np.random.default_rng(77 + M)
    x = workloads.activations(rng, M, K)
    x[M - 1, 37] = 0x7FC0                       # BF16 NaN in the last row
    w = workloads.weight_codes(rng, (N, K))
    ws = workloads.scale_bytes(rng, (N, K // 32), -10, -4)
    ws[21, K // 32 - 1] = 0xFF
    say("mx_linear fp8 NaN blocks", M, K)
    got = host_u16(mx.mx_linear(dev_u16(x), dev_u8(w), dev_u8(ws)))
    ref = G.mx_linear(x, w, ws, 32)
    nan = np.isnan(ref)
    assert nan[M - 1].all() and nan[:, 21].all() and nan.sum() == N + M - 1
    assert np.array_equal(np.isnan(F.bf16_to_f64(got)), nan)
    assert_gemm_close(got[~nan], ref[~nan], f"M={M} K={K} finite part")


@pytest.mark.parametrize("M,K", [(1, 128), (5, 1152), (16, 2304), (9, 4096), (40, 1152), (64, 2304)])
def test_linear_fp8_identity_weight_returns_quantised_x(M, K):
    """With the identity as the FP8 weight (code 0x38 = 1.0 on the diagonal,
    unit scales) every output is one dequantised x code, which BF16 holds
    exactly.  So the codes and scales this branch makes for x -- inside the
    GEMM for up to 16 rows, by the quantiser otherwise -- are checked bit for
    bit against the oracle's, on random BF16 bit patterns (magnitudes from
    2^-63 to 2^124, both signs) with one all-zero block per row."""
    from oracle.quant import group_quant
    rng = np.random.default_rng(M * 7919 + K)
    sign = rng.integers(0, 2, (M, K)).astype(np.uint16) << 15
    x = (sign | (rng.integers(64, 251, (M, K)).astype(np.uint16) << 7) | rng.integers(0, 128, (M, K)).astype(np.uint16))
    zero_block = rng.integers(0, K // 32, M)
    for m in range(M):
        x[m, 32 * zero_block[m]: 32 * zero_block[m] + 32] = 0
    w = np.zeros((K, K), np.uint8)
    w[np.arange(K), np.arange(K)] = 0x38
    ws = np.full((K, K // 32), 127, np.uint8)
    say("mx_linear fp8 identity weight", M, K)
    got = host_u16(mx.mx_linear(dev_u16(x.astype(np.uint16)), dev_u8(w), dev_u8(ws)))
    xq, xs = group_quant(x, 32, F.OCP)
    ref = F.f64_to_bf16_rne(G.scaled_operand(xq, xs, 32, F.OCP))
    # a zero sum is +0 on the GPU (the accumulator starts at +0)
    ref = np.where(ref == 0x8000, 0, ref).astype(np.uint16)
    got = np.where(got == 0x8000, 0, got).astype(np.uint16)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} of {ref.size} outputs differ"
