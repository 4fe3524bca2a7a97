"""GPU parity of mx_wo_a_fused (inverse RoPE + group-128 quantisation + the
MX-scale GEMM in one kernel) against the oracle's quantise-then-GEMM result:
|gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref), ref the unrounded fp64 product of
the oracle's codes and scales.  Cases: the tiny wo_a problem (both pairings),
shapes crossing every tile edge (T, N past 256; several groups; K from one
stage to 32; D of 128 to 512; rope_dim 0 to 128), the decode batch on every
row, tokens with positions outside the table, the shapes it declines, a
seeded sweep of 16 shapes, and repeated launches (bit-identical, and within
the bound of the quantiser-then-GEMM path).
The prefill chunk is checked on every output in test_gpu_full_prefill.py."""

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from helpers import assert_gemm_close, dev_i64, dev_u16, dev_u8, host_u16, requires_gpu, say
from oracle import gemm as G
from oracle.quant import inv_rope_group_quant
from oracle.rope import INTERLEAVED, NEOX

pytestmark = [pytest.mark.gpu, requires_gpu]
STYLE = {INTERLEAVED: mx.MX_ROPE_INTERLEAVED, NEOX: mx.MX_ROPE_NEOX}


def _run(x, pos, cos, sin, H, D, R, w, ws, style=INTERLEAVED):
    out = mx.mx_wo_a_fused(dev_u16(x), dev_i64(pos), dev_u16(cos), dev_u16(sin), H, D, R, dev_u8(w), dev_u8(ws),
                           STYLE[style])
    torch.cuda.synchronize()
    return host_u16(out)


def _ref(x, pos, cos, sin, H, D, R, w, ws, style=INTERLEAVED):
    T = x.shape[0]
    Gn, N, K = w.shape
    rq, rs = inv_rope_group_quant(x, pos, cos, sin, H, D, R, style, 128)
    return G.bmm_a8w8_mxscale(rq.reshape(T, Gn, K), rs.reshape(T, Gn, -1), w, ws)


@pytest.mark.parametrize("style", [INTERLEAVED, NEOX])
def test_tiny(style):
    p = workloads.tiny()
    cos, sin = workloads.rope_tables(rows=64)
    say("fused wo_a tiny", style)
    mx.mx_reset_counters()
    got = _run(p.x, p.positions, cos, sin, p.H, p.D, 64, p.w, p.w_scale, style)
    assert mx.mx_get_counters()["wo_a_fused"] == 1
    ref = _ref(p.x, p.positions, cos, sin, p.H, p.D, 64, p.w, p.w_scale, style)
    assert_gemm_close(got.reshape(ref.shape), ref, f"tiny {style}")


# T, G, N, H, D, R, style -- K = H*D/G
SHAPES = [
    (1, 1, 16, 1, 128, 64, INTERLEAVED),          # one stage, one row
    (17, 2, 272, 4, 128, 16, NEOX),                # ragged N tile, K = 256
    (255, 3, 256, 6, 256, 48, INTERLEAVED),        # K = 512, 48 rotated dims (not a power of two)
    (256, 1, 512, 3, 128, 32, NEOX),               # exactly one t-tile, K = 384 (odd stage count)
    (257, 2, 528, 8, 256, 64, NEOX),               # one row past a t-tile, N past two tiles
    (300, 1, 64, 8, 512, 0, INTERLEAVED),          # no rotation, K = 4096
    (513, 4, 128, 16, 512, 64, INTERLEAVED),       # K = 2048, three t-tiles
    (40, 16, 96, 128, 512, 64, NEOX),              # the production row width, K = 4096
]


@pytest.mark.parametrize("T,Gn,N,H,D,R,style", SHAPES)
def test_shapes(T, Gn, N, H, D, R, style):
    rng = np.random.default_rng(300 + T + N + R)
    K = H * D // Gn
    x = workloads.activations(rng, T, H * D)
    pos = rng.integers(0, 4096, T)
    w = workloads.weight_codes(rng, (Gn, N, K))
    ws = workloads.scale_bytes(rng, (Gn, N, K // 128), -8, -4)
    cos, sin = workloads.rope_tables(rows=4096, rope_dim=max(R, 16))
    say("fused wo_a", T, Gn, N, H, D, R, style)
    got = _run(x, pos, cos, sin, H, D, R, w, ws, style)
    ref = _ref(x, pos, cos, sin, H, D, R, w, ws, style)
    assert_gemm_close(got.reshape(ref.shape), ref, f"T={T} G={Gn} N={N} H={H} D={D} R={R} {style}")


def test_decode_batch_every_row():
    p = workloads.decode_batch()
    cos, sin = workloads.rope_tables(rows=32768)
    say("fused wo_a decode batch")
    got = _run(p.x, p.positions, cos, sin, p.H, p.D, 64, p.w, p.w_scale)
    ref = _ref(p.x, p.positions, cos, sin, p.H, p.D, 64, p.w, p.w_scale)
    assert_gemm_close(got.reshape(ref.shape), ref, "decode batch")


def test_positions_outside_the_table_give_nan_rows():
    rng = np.random.default_rng(41)
    T, Gn, N, H, D = 6, 2, 32, 4, 128
    K = H * D // Gn
    x = workloads.activations(rng, T, H * D)
    pos = np.array([0, 5, 4096, -1, 7, 9])               # rows 2 and 3 are outside a 4096-row table
    w = workloads.weight_codes(rng, (Gn, N, K))
    ws = workloads.scale_bytes(rng, (Gn, N, K // 128), -8, -4)
    cos, sin = workloads.rope_tables(rows=4096)
    say("fused wo_a bad positions")
    got = _run(x, pos, cos, sin, H, D, 64, w, ws).reshape(T, Gn, N)
    vals = got.astype(np.uint32) << 16
    nan = np.isnan(vals.view(np.float32))
    assert nan[2:4].all() and not nan[[0, 1, 4, 5]].any()
    good = [0, 1, 4, 5]
    ref = _ref(x[good], pos[good], cos, sin, H, D, 64, w, ws)
    assert_gemm_close(got[good], ref, "rows with valid positions")


def test_declined_shapes_and_empty():
    x = torch.zeros((4, 8192), dtype=torch.int16, device="cuda")
    pos = torch.zeros(4, dtype=torch.int64, device="cuda")
    cs = torch.zeros((16, 32), dtype=torch.int16, device="cuda")
    w = torch.zeros((1, 16, 8192), dtype=torch.uint8, device="cuda")        # K = 8192 > 4096
    s = torch.zeros((1, 16, 64), dtype=torch.uint8, device="cuda")
    mx.mx_reset_counters()
    with pytest.raises(mx.MxError, match="MX_ERR_UNSUPPORTED"):
        mx.mx_wo_a_fused(x, pos, cs, cs, 16, 512, 64, w, s)
    cs48 = torch.zeros((16, 24), dtype=torch.int16, device="cuda")
    w2 = torch.zeros((2, 16, 4096), dtype=torch.uint8, device="cuda")
    s2 = torch.zeros((2, 16, 32), dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.MxError, match="MX_ERR_UNSUPPORTED"):            # split halves of 48 dims
        mx.mx_wo_a_fused(x, pos, cs48, cs48, 16, 512, 48, w2, s2, mx.MX_ROPE_NEOX)
    cs128 = torch.zeros((16, 64), dtype=torch.int16, device="cuda")
    with pytest.raises(mx.MxError, match="MX_ERR_UNSUPPORTED"):            # more than 64 rotated dims
        mx.mx_wo_a_fused(x, pos, cs128, cs128, 16, 512, 128, w2, s2)
    e = mx.mx_wo_a_fused(x[:0], pos[:0], cs, cs, 16, 512, 64, w2, s2)
    assert e.shape == (0, 2, 16)
    assert mx.mx_get_counters()["wo_a_fused"] == 0


@pytest.mark.parametrize("style", [INTERLEAVED, NEOX])
def test_repeated_launches_match_the_two_kernel_path(style):
    """Eight rope stages per group and 64 tiles: every launch gives the same
    bits, and those agree with the quantiser followed by the GEMM (the same
    codes and scales, sums in another order) within the GEMM bound.  A
    rotation that read its tables before their DMA landed would show here as
    launch-to-launch differences or as large errors."""
    rng = np.random.default_rng(77 + (style == NEOX))
    T, Gn, N, H, D, R = 1024, 16, 512, 128, 512, 64
    K = H * D // Gn
    x = dev_u16(workloads.activations(rng, T, H * D))
    pos = dev_i64(rng.integers(0, 8192, T))
    cos, sin = workloads.rope_tables(rows=8192, rope_dim=R)
    cos, sin = dev_u16(cos), dev_u16(sin)
    w = dev_u8(workloads.weight_codes(rng, (Gn, N, K)))
    ws = dev_u8(workloads.scale_bytes(rng, (Gn, N, K // 128), -8, -4))
    say("fused wo_a repeated launches", style)
    outs = [mx.mx_wo_a_fused(x, pos, cos, sin, H, D, R, w, ws, STYLE[style]) for _ in range(3)]
    q, s = mx.mx_inv_rope_group_quant(x, pos, cos, sin, H, D, R, STYLE[style])
    two = mx.mx_bmm_a8w8_mxscale(q.view(T, Gn, K), s.view(T, Gn, K // 128), w, ws)
    torch.cuda.synchronize()
    first = outs[0].view(torch.int16)
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), first)
    a = outs[0].float().cpu().numpy()
    b = two.float().cpu().numpy().reshape(a.shape)
    assert np.isfinite(a).all()
    rms = float(np.sqrt(np.mean(b.astype(np.float64) ** 2)))
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-3 * rms)


def _sweep_cases():
    """A seeded sweep: T from 1 to 700, 1 to 4 groups, N up to 640, heads of
    128 to 512 dims, K = H*D/G from one stage to 32, rope_dim 0 to 64 in both
    pairings (NeoX only at 16, 32, 64)."""
    rng = np.random.default_rng(5150)
    cases = []
    while len(cases) < 16:
        Gn = int(rng.integers(1, 5))
        D = 128 * int(rng.integers(1, 5))
        H = int(rng.integers(1, 9))
        if (H * D) % Gn or (H * D // Gn) % 128 or H * D // Gn > 4096:
            continue
        style = NEOX if rng.integers(0, 2) else INTERLEAVED
        R = int(rng.choice([0, 16, 32, 64])) if style == NEOX else 16 * int(rng.integers(0, 5))
        T = int(rng.integers(1, 701))
        N = 16 * int(rng.integers(1, 41))
        cases.append((len(cases), T, Gn, N, H, D, R, style))
    return cases


@pytest.mark.parametrize("case,T,Gn,N,H,D,R,style", _sweep_cases())
def test_sweep(case, T, Gn, N, H, D, R, style):
    rng = np.random.default_rng(900 + case)
    K = H * D // Gn
    x = workloads.activations(rng, T, H * D)
    pos = rng.integers(0, 4096, T)
    w = workloads.weight_codes(rng, (Gn, N, K))
    ws = workloads.scale_bytes(rng, (Gn, N, K // 128), -8, -4)
    cos, sin = workloads.rope_tables(rows=4096, rope_dim=max(R, 16))
    say("fused wo_a sweep", case, T, Gn, N, H, D, R, style)
    got = _run(x, pos, cos, sin, H, D, R, w, ws, style)
    ref = _ref(x, pos, cos, sin, H, D, R, w, ws, style)
    assert_gemm_close(got.reshape(ref.shape), ref, f"sweep {case}: T={T} G={Gn} N={N} H={H} D={D} R={R} {style}")
