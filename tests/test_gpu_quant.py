"""GPU parity of mx_inv_rope_group_quant against the oracle.

* Unfused: the oracle's rotated BF16 tensor quantised with the rotation off
  must give bit-identical codes and scales.
* Fused: scales bit-exact, codes within one step on at most 1e-4 of the
  elements (the bound allows rounding ties to fall either way; the kernel
  rounds like the oracle, so the count is expected to be 0 and is reported).
* Shapes: the tiny problem, the decode batch (every row), the 8192-token
  prefill chunk (every row on the GPU, 48 rows checked), ragged row counts,
  both pairings, both byte flavours, groups of 128 and 32.
* Edge cases: empty input, all-zero / NaN / Inf groups, positions outside
  the table, determinism.
"""

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from helpers import (assert_codes_close, dev_i64, dev_u16, host_u16, host_u8, requires_gpu, say)
from oracle import formats as F
from oracle.quant import group_quant, inv_rope_group_quant
from oracle.rope import inverse_rope, INTERLEAVED, NEOX

pytestmark = [pytest.mark.gpu, requires_gpu]

FMT = {F.OCP: mx.MX_FP8_E4M3_OCP, F.FNUZ: mx.MX_FP8_E4M3_FNUZ}
STYLE = {INTERLEAVED: mx.MX_ROPE_INTERLEAVED, NEOX: mx.MX_ROPE_NEOX}


@pytest.fixture(scope="module")
def tables():
    cos, sin = workloads.rope_tables()
    return cos, sin, dev_u16(cos), dev_u16(sin)


def _gpu_quant(x, pos, tables, H, D, R, style=INTERLEAVED, group=128, fmt=F.OCP):
    _, _, dcos, dsin = tables
    q, s = mx.mx_inv_rope_group_quant(dev_u16(x), dev_i64(pos) if pos is not None else None, dcos, dsin, H, D, R,
                                      STYLE[style], group, FMT[fmt])
    torch.cuda.synchronize()
    return host_u8(q), host_u8(s)


@pytest.mark.parametrize("fmt", [F.OCP, F.FNUZ])
@pytest.mark.parametrize("style", [INTERLEAVED, NEOX])
def test_tiny_fused(tables, fmt, style):
    p = workloads.tiny()
    cos, sin = tables[0], tables[1]
    say("quant tiny fused", fmt, style)
    q, s = _gpu_quant(p.x, p.positions, tables, p.H, p.D, 64, style, 128, fmt)
    rq, rs = inv_rope_group_quant(p.x, p.positions, cos, sin, p.H, p.D, 64, style, 128, fmt)
    n = assert_codes_close(q, rq, s, rs, fmt, exact=False, what="tiny fused")
    assert n == 0, f"{n} tie flips"


@pytest.mark.parametrize("fmt", [F.OCP, F.FNUZ])
@pytest.mark.parametrize("group", [128, 32])
def test_tiny_unfused_bit_exact(tables, fmt, group):
    p = workloads.tiny()
    cos, sin = tables[0], tables[1]
    r = inverse_rope(p.x, p.positions, cos, sin, p.H, p.D, 64)
    say("quant tiny unfused", fmt, group)
    q, s = _gpu_quant(r, None, tables, p.H, p.D, 0, group=group, fmt=fmt)
    rq, rs = group_quant(r, group, fmt)
    assert_codes_close(q, rq, s, rs, fmt, exact=True, what="tiny unfused")


@pytest.mark.parametrize("T", [1, 3, 17, 129, 1000])
def test_ragged_rows(tables, T):
    rng = np.random.default_rng(T)
    H, D = 4, 128
    x = workloads.activations(rng, T, H * D)
    pos = rng.integers(0, 131072, T)
    cos, sin = tables[0], tables[1]
    say("quant ragged", T)
    q, s = _gpu_quant(x, pos, tables, H, D, 64)
    rq, rs = inv_rope_group_quant(x, pos, cos, sin, H, D, 64)
    assert_codes_close(q, rq, s, rs, F.OCP, exact=True, what=f"T={T}")


@pytest.mark.parametrize("T", [1, 7, 33])
def test_rows_not_a_multiple_of_512_and_unaligned_scales(tables, T):
    """H*D = 384: a lane row's 4 groups straddle token rows and the last one
    can be partial; the scale output starts 1 byte past an aligned address
    (the 4-byte scale store then falls back to bytes)."""
    rng = np.random.default_rng(50 + T)
    H, D = 3, 128
    x = workloads.activations(rng, T, H * D)
    pos = rng.integers(0, 8192, T)
    cos, sin, dcos, dsin = tables
    say("quant H*D=384 unaligned scales", T)
    q = torch.empty((T, H * D), dtype=torch.uint8, device="cuda")
    sbuf = torch.full((T * H * D // 128 + 8,), 0xAA, dtype=torch.uint8, device="cuda")
    s = sbuf[1:1 + T * H * D // 128].view(T, H * D // 128)
    mx.mx_inv_rope_group_quant(dev_u16(x), dev_i64(pos), dcos, dsin, H, D, 64, q=q, scale=s)
    torch.cuda.synchronize()
    rq, rs = inv_rope_group_quant(x, pos, cos, sin, H, D, 64)
    assert_codes_close(host_u8(q), rq, host_u8(s), rs, F.OCP, exact=False, what=f"T={T}")
    out = host_u8(sbuf)
    assert out[0] == 0xAA and np.all(out[1 + T * H * D // 128:] == 0xAA)    # nothing written outside


def test_empty(tables):
    _, _, dcos, dsin = tables
    x = torch.empty((0, 512), dtype=torch.int16, device="cuda")
    q, s = mx.mx_inv_rope_group_quant(x, torch.empty(0, dtype=torch.int64, device="cuda"), dcos, dsin, 4, 128, 64)
    assert q.shape == (0, 512) and s.shape == (0, 4)


def test_special_groups_and_bad_positions(tables):
    H, D = 4, 128
    rng = np.random.default_rng(9)
    x = workloads.activations(rng, 6, H * D)
    x[0, 0:128] = 0                          # all-zero group
    x[0, 128:256] = 0x8000                   # all -0
    x[1, 200] = 0x7FC0                       # NaN
    x[2, 300] = 0xFF80                       # -Inf
    x[3, 10] = 0x0001                        # smallest subnormal in an otherwise normal group
    x[3, 128:256] = 0x0003                   # a group of subnormals only
    pos = np.array([0, 5, 7, 9, 131072, -1])  # rows 4 and 5 are outside the table
    cos, sin = tables[0], tables[1]
    for fmt in (F.OCP, F.FNUZ):
        say("quant special groups", fmt)
        q, s = _gpu_quant(x, pos, tables, H, D, 64, fmt=fmt)
        rq, rs = inv_rope_group_quant(x[:4], pos[:4], cos, sin, H, D, 64, fmt=fmt)
        assert_codes_close(q[:4], rq, s[:4], rs, fmt, exact=True, what="special")
        nan = 0x7F if fmt == F.OCP else 0x80
        assert np.all(s[4:] == 0xFF) and np.all(q[4:] == nan)


def test_deterministic(tables):
    p = workloads.tiny()
    a = _gpu_quant(p.x, p.positions, tables, p.H, p.D, 64)
    b = _gpu_quant(p.x, p.positions, tables, p.H, p.D, 64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.fixture(scope="module")
def decode():
    return workloads.decode_batch()


@pytest.mark.parametrize("fmt", [F.OCP, F.FNUZ])
def test_decode_batch_every_row(tables, decode, fmt):
    p = decode
    cos, sin = tables[0], tables[1]
    say("quant decode batch", fmt)
    q, s = _gpu_quant(p.x, p.positions, tables, p.H, p.D, 64, fmt=fmt)
    rq, rs = inv_rope_group_quant(p.x, p.positions, cos, sin, p.H, p.D, 64, fmt=fmt)
    n = assert_codes_close(q, rq, s, rs, fmt, exact=False, what="decode")
    assert n == 0


@pytest.mark.slow
def test_prefill_chunk_sampled_rows(tables):
    p = workloads.prefill_chunk()
    cos, sin = tables[0], tables[1]
    say("quant prefill chunk T=8192")
    q, s = _gpu_quant(p.x, p.positions, tables, p.H, p.D, 64)
    rows = np.unique(np.concatenate([[0, 1, 4095, 8191], np.random.default_rng(11).integers(0, 8192, 44)]))
    rq, rs = inv_rope_group_quant(p.x[rows], p.positions[rows], cos, sin, p.H, p.D, 64)
    n = assert_codes_close(q[rows], rq, s[rows], rs, F.OCP, exact=False, what="prefill")
    assert n == 0


@pytest.mark.slow
def test_call_split_into_two_launches(tables):
    """H*D = 65536 and T = 262,243 tokens: 2^31 or more 8-element chunks, so the
    call runs as two launches (262,143 rows, then 100).  34 GB of seeded random
    BF16 with |x| < 2 (no Inf or NaN), drawn on the device, and random
    positions; sampled rows on both sides of the split are checked against the
    oracle."""
    H, D, T = 128, 512, 262243
    cos, sin, dcos, dsin = tables
    say("quant one call T=262243 H=128 D=512 (two launches)")
    gen = torch.Generator(device="cuda").manual_seed(616)
    x = torch.randint(-32768, 32768, (T, H * D), dtype=torch.int16, device="cuda", generator=gen)
    x.bitwise_and_(~0x4000)
    pos = torch.randint(0, cos.shape[0], (T,), dtype=torch.int64, device="cuda", generator=gen)
    q, s = mx.mx_inv_rope_group_quant(x, pos, dcos, dsin, H, D, 64)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 262142, 262143, 262144, T - 1],
                                     np.random.default_rng(616).integers(0, T, 8)]))
    idx = torch.from_numpy(rows).cuda()
    xr, pr = host_u16(x[idx].contiguous()), pos[idx].cpu().numpy()
    qr, sr = host_u8(q[idx].contiguous()), host_u8(s[idx].contiguous())
    del x, q, s
    rq, rs = inv_rope_group_quant(xr, pr, cos, sin, H, D, 64)
    n = assert_codes_close(qr, rq, sr, rs, F.OCP, exact=False, what="two launches")
    assert n == 0
