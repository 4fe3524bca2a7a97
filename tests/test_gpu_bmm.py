"""GPU parity of mx_bmm_a8w8_mxscale against the fp64 oracle.

Bound: |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref).  Cases: the tiny wo_a
problem end to end (quantiser then GEMM), stand-alone random operands over
tile-crossing and ragged shapes for both kernels (T <= 64 and larger), FNUZ
activations (and their bit-identity with the OCP run of the same values), the
decode batch and the 8192-token prefill chunk at full size with sampled rows
checked, and run-to-run determinism.
"""

import math

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from helpers import assert_gemm_close, dev_i64, dev_u16, dev_u8, host_u16, requires_gpu, say
from oracle import formats as F
from oracle import gemm as G
from oracle.quant import inv_rope_group_quant

pytestmark = [pytest.mark.gpu, requires_gpu]


def _gpu_bmm(a, sa, w, sw, fmt=mx.MX_FP8_E4M3_OCP):
    out = mx.mx_bmm_a8w8_mxscale(dev_u8(a), dev_u8(sa), dev_u8(w), dev_u8(sw), fmt)
    torch.cuda.synchronize()
    return host_u16(out)


def test_tiny_end_to_end():
    p = workloads.tiny()
    cos, sin = workloads.rope_tables(rows=64)
    say("bmm tiny end to end")
    q, s = mx.mx_inv_rope_group_quant(dev_u16(p.x), dev_i64(p.positions), dev_u16(cos), dev_u16(sin),
                                      p.H, p.D, 64)
    out = mx.mx_bmm_a8w8_mxscale(q.view(p.T, p.G, p.K), s.view(p.T, p.G, p.K // 128), dev_u8(p.w),
                                 dev_u8(p.w_scale))
    torch.cuda.synchronize()
    rq, rs = inv_rope_group_quant(p.x, p.positions, cos, sin, p.H, p.D, 64)
    ref = G.bmm_a8w8_mxscale(rq.reshape(p.T, p.G, p.K), rs.reshape(p.T, p.G, -1), p.w, p.w_scale)
    assert_gemm_close(host_u16(out), ref, "tiny")


SHAPES = [
    # T, G, N, K  -- small-T kernel (T <= 64) and the large-tile kernel
    (1, 1, 16, 128), (7, 2, 48, 256), (64, 3, 128, 512), (16, 2, 128, 256),
    (65, 1, 16, 128), (200, 2, 272, 384), (256, 1, 256, 128), (300, 3, 512, 640), (513, 2, 784, 256),
]


@pytest.mark.parametrize("T,Gn,N,K", SHAPES)
def test_random_operands(T, Gn, N, K):
    a, sa, w, sw = workloads.gemm_operands(1000 + T + N, T, Gn, N, K)
    say("bmm random", T, Gn, N, K)
    out = _gpu_bmm(a, sa, w, sw)
    ref = G.bmm_a8w8_mxscale(a, sa, w, sw)
    assert_gemm_close(out, ref, f"T={T} G={Gn} N={N} K={K}")


# T <= 64 with K in {1024, 2048, 4096, 8192} takes the decode-batch kernel
# (LDS-DMA ring of 8 K-steps): a single token, a ragged last n-block, the
# deepest and the shallowest K, and FNUZ activations
DECODE_SHAPES = [(1, 1, 16, 1024), (5, 3, 112, 2048), (64, 2, 272, 8192), (33, 16, 1024, 4096), (64, 1, 64, 1024)]


@pytest.mark.parametrize("T,Gn,N,K", DECODE_SHAPES)
def test_decode_kernel(T, Gn, N, K):
    a, sa, w, sw = workloads.gemm_operands(5000 + T + N + K, T, Gn, N, K)
    say("bmm decode kernel", T, Gn, N, K)
    out = _gpu_bmm(a, sa, w, sw)
    assert_gemm_close(out, G.bmm_a8w8_mxscale(a, sa, w, sw), f"T={T} G={Gn} N={N} K={K}")


def test_decode_kernel_fnuz():
    T, Gn, N, K = 64, 2, 192, 2048
    a, sa, w, sw = workloads.gemm_operands(77, T, Gn, N, K, a_exp=(-12, -2))
    # the same values in FNUZ: code unchanged, scale + 1, -0 -> 0
    fz = np.where(a == 0x80, 0, a).astype(np.uint8)
    sz = (sa.astype(int) + 1).astype(np.uint8)
    say("bmm decode kernel fnuz")
    out_f = _gpu_bmm(fz, sz, w, sw, mx.MX_FP8_E4M3_FNUZ)
    out_o = _gpu_bmm(a, sa, w, sw)
    assert np.array_equal(out_f, out_o)
    assert_gemm_close(out_f, G.bmm_a8w8_mxscale(fz, sz, w, sw, F.FNUZ), "decode fnuz")


# K = 2048 and 4096 (16 or 32 K-stages) take the persistent kernel: tile counts
# below one per XCD, one per workgroup, and several per workgroup (T = 4200:
# 340 tiles on 256 workgroups), with ragged T and N tiles.  Large cases are
# checked on sampled rows (first, last, tile edges and random ones).  The
# last two split the tiles into whole groups per XCD, which the kernel walks
# token tile by token tile across the XCD's groups (3 groups per XCD, one
# tile per workgroup; 2 groups per XCD, two rounds).
PERSIST_SHAPES = [(300, 1, 272, 2048), (1000, 3, 512, 4096), (4200, 5, 1024, 2048), (2600, 2, 784, 4096),
                  (512, 24, 256, 2048), (4096, 16, 512, 2048)]


def _sample_rows(T, rng, n=48):
    edges = [0, T - 1] + [t for t in range(255, T, 256)] + [t for t in range(256, T, 256)]
    return np.unique(np.concatenate([np.array(edges), rng.integers(0, T, n)]))


@pytest.mark.parametrize("T,Gn,N,K", PERSIST_SHAPES)
def test_persistent_tiles(T, Gn, N, K):
    a, sa, w, sw = workloads.gemm_operands(2000 + T + K, T, Gn, N, K)
    say("bmm persistent", T, Gn, N, K)
    out = _gpu_bmm(a, sa, w, sw)
    rows = _sample_rows(T, np.random.default_rng(T)) if T * Gn * N * K > 2 ** 31 else np.arange(T)
    ref = G.bmm_a8w8_mxscale(a[rows], sa[rows], w, sw)
    assert_gemm_close(out[rows], ref, f"T={T} G={Gn} N={N} K={K}")


# the one-tile-per-workgroup kernel: K beyond one 32-stage scale window
# (restaged in the loop), an odd number of stages, and K = 4096 with scale
# tensors that are not 16-byte aligned (which keeps the persistent kernel off)
@pytest.mark.parametrize("T,Gn,N,K", [(300, 1, 272, 8192), (280, 2, 256, 4224), (260, 1, 512, 6272)])
def test_large_kernel_scale_windows(T, Gn, N, K):
    a, sa, w, sw = workloads.gemm_operands(3000 + K, T, Gn, N, K)
    say("bmm large windows", T, Gn, N, K)
    out = _gpu_bmm(a, sa, w, sw)
    rows = _sample_rows(T, np.random.default_rng(K))
    assert_gemm_close(out[rows], G.bmm_a8w8_mxscale(a[rows], sa[rows], w, sw), f"T={T} K={K}")


def test_large_kernel_misaligned_scales():
    T, Gn, N, K = 300, 2, 256, 4096
    a, sa, w, sw = workloads.gemm_operands(41, T, Gn, N, K)
    dev = torch.device("cuda:0")
    say("bmm misaligned scales")
    # the scale tensors start 1 byte into a larger buffer
    sab = torch.zeros(sa.size + 16, dtype=torch.uint8, device=dev)
    swb = torch.zeros(sw.size + 16, dtype=torch.uint8, device=dev)
    sab[1:1 + sa.size] = torch.from_numpy(sa.reshape(-1)).to(dev)
    swb[1:1 + sw.size] = torch.from_numpy(sw.reshape(-1)).to(dev)
    sad = sab[1:1 + sa.size].view(sa.shape)
    swd = swb[1:1 + sw.size].view(sw.shape)
    out = mx.mx_bmm_a8w8_mxscale(dev_u8(a), sad, dev_u8(w), swd)
    torch.cuda.synchronize()
    assert_gemm_close(host_u16(out), G.bmm_a8w8_mxscale(a, sa, w, sw), "misaligned scales")


def test_persistent_matches_large_kernel_bit_exact():
    # Several tiles per workgroup with ragged T and N, through the persistent
    # kernel (aligned scales: LDS-staged epilogue folded into the next tile)
    # and through the one-tile-per-workgroup kernel (the same scales 1 byte
    # into a larger buffer).  Both sum each block over the same rotated K
    # order, so the outputs must agree bit for bit; sampled rows are also
    # checked against the oracle.
    T, Gn, N, K = 4200, 8, 1008, 2048
    a, sa, w, sw = workloads.gemm_operands(51, T, Gn, N, K)
    dev = torch.device("cuda:0")
    say("bmm persistent vs large", T, Gn, N, K)
    ad, wd = dev_u8(a), dev_u8(w)
    o_pers = mx.mx_bmm_a8w8_mxscale(ad, dev_u8(sa), wd, dev_u8(sw))
    sab = torch.zeros(sa.size + 16, dtype=torch.uint8, device=dev)
    swb = torch.zeros(sw.size + 16, dtype=torch.uint8, device=dev)
    sab[1:1 + sa.size] = torch.from_numpy(sa.reshape(-1)).to(dev)
    swb[1:1 + sw.size] = torch.from_numpy(sw.reshape(-1)).to(dev)
    o_large = mx.mx_bmm_a8w8_mxscale(ad, sab[1:1 + sa.size].view(sa.shape), wd, swb[1:1 + sw.size].view(sw.shape))
    torch.cuda.synchronize()
    op, ol = host_u16(o_pers), host_u16(o_large)
    assert np.array_equal(op, ol)
    rows = _sample_rows(T, np.random.default_rng(51))
    assert_gemm_close(op[rows], G.bmm_a8w8_mxscale(a[rows], sa[rows], w, sw), "persistent vs large")


def test_persistent_fnuz_bit_identical():
    T, Gn, N, K = 600, 2, 512, 4096
    a, sa, w, sw = workloads.gemm_operands(31, T, Gn, N, K, a_exp=(-12, -2))
    a_fnuz = np.where(a == 0x80, 0, a).astype(np.uint8)
    sa_fnuz = (sa.astype(int) + 1).astype(np.uint8)
    say("bmm persistent fnuz")
    o_ocp = _gpu_bmm(a, sa, w, sw)
    o_fnuz = _gpu_bmm(a_fnuz, sa_fnuz, w, sw, mx.MX_FP8_E4M3_FNUZ)
    assert np.array_equal(o_ocp, o_fnuz)
    rows = _sample_rows(T, np.random.default_rng(1))
    assert_gemm_close(o_fnuz[rows], G.bmm_a8w8_mxscale(a_fnuz[rows], sa_fnuz[rows], w, sw, a_fmt=F.FNUZ), "fnuz")


@pytest.mark.parametrize("T", [40, 300])
def test_fnuz_activations(T):
    Gn, N, K = 2, 256, 512
    a, sa, w, sw = workloads.gemm_operands(77 + T, T, Gn, N, K, a_exp=(-12, -2))
    # the same values in FNUZ: code unchanged, scale + 1, -0 -> 0
    a_fnuz = np.where(a == 0x80, 0, a).astype(np.uint8)
    sa_fnuz = (sa.astype(int) + 1).astype(np.uint8)
    say("bmm fnuz", T)
    o_ocp = _gpu_bmm(a, sa, w, sw)
    o_fnuz = _gpu_bmm(a_fnuz, sa_fnuz, w, sw, mx.MX_FP8_E4M3_FNUZ)
    ref = G.bmm_a8w8_mxscale(a_fnuz, sa_fnuz, w, sw, a_fmt=F.FNUZ)
    assert_gemm_close(o_fnuz, ref, "fnuz")
    assert np.array_equal(o_ocp, o_fnuz)


@pytest.mark.parametrize("T,Gn,N,K", [(8, 2, 64, 1024), (40, 2, 64, 384), (300, 1, 256, 512), (512, 2, 256, 2048)])
def test_fnuz_scale_byte_zero_is_computed_at_twice_its_value(T, Gn, N, K):
    """The one FNUZ block the OCP MFMA cannot express: scale byte 0 (2^-127)
    would need the OCP scale 2^-128, which E8M0 does not have, so the kernels
    keep the byte and such a block comes out twice its value (the header
    states this).  Every third token has all its blocks at byte 0; those rows
    equal twice the oracle's FNUZ result within the bound and lie outside the
    bound of the oracle's own; the other rows match the oracle.  The decode,
    small-T, large-tile and persistent kernels all take this path."""
    rng = np.random.default_rng(900 + T + K)
    a, sa, w, sw = workloads.gemm_operands(901 + T, T, Gn, N, K, a_exp=(-12, -2))
    a = np.where(a == 0x80, 0, a).astype(np.uint8)          # no FNUZ NaN in A
    sa = rng.integers(120, 126, size=sa.shape).astype(np.uint8)
    zero_rows = np.arange(0, T, 3)
    sa[zero_rows] = 0
    sw = rng.integers(200, 206, size=sw.shape).astype(np.uint8)   # lifts the 2^-127 blocks into range
    say("bmm fnuz scale byte 0", T, Gn, N, K)
    out = _gpu_bmm(a, sa, w, sw, mx.MX_FP8_E4M3_FNUZ)
    ref = G.bmm_a8w8_mxscale(a, sa, w, sw, a_fmt=F.FNUZ)
    other = np.setdiff1d(np.arange(T), zero_rows)
    assert_gemm_close(out[other], ref[other], "rows with normal scales")
    assert_gemm_close(out[zero_rows], 2.0 * ref[zero_rows], "scale-0 rows against twice the oracle")
    g = F.bf16_to_f64(out[zero_rows])
    r = ref[zero_rows]
    rms = math.sqrt(float(np.mean(r * r)))
    outside = np.abs(g - r) > 2.0 ** -7 * np.abs(r) + 1e-3 * rms
    assert outside.mean() > 0.9                           # not within the oracle's own bound


def test_deterministic():
    a, sa, w, sw = workloads.gemm_operands(5, 300, 2, 512, 512)
    assert np.array_equal(_gpu_bmm(a, sa, w, sw), _gpu_bmm(a, sa, w, sw))


@pytest.mark.parametrize("K", [256, 1024])          # the split-K small kernel and the decode kernel
def test_special_scales(K):
    """E8M0 0xFF scales make their block NaN (an activation scale: one token's
    row; a weight scale: one column); scale byte 0 (2^-127) is honoured."""
    T, Gn, N = 32, 1, 80
    a, sa, w, sw = workloads.gemm_operands(9, T, Gn, N, K)
    sa[0, 0, 1] = 0xFF
    sw[0, 5, 0] = 0xFF
    sa[3, 0, :] = 0                                    # 2^-127 on every block of token 3
    out = F.bf16_to_f64(_gpu_bmm(a, sa, w, sw))
    assert np.all(np.isnan(out[0, 0, :]))
    assert np.all(np.isnan(out[:, 0, 5]))
    keep = np.ones(out.shape, bool)
    keep[0] = False
    keep[:, :, 5] = False
    assert not np.isnan(out[keep]).any()
    ref3 = G.bmm_a8w8_mxscale(a[3:4], sa[3:4], w, sw)[0, 0]
    cols = [n for n in range(N) if n != 5]
    assert np.all(np.abs(ref3[cols]) < 2.0 ** -100)     # tiny, yet normal in fp32 and BF16
    assert_gemm_close(_gpu_bmm(a, sa, w, sw)[3:4][:, :, cols], ref3[None, None, cols], "2^-127 scales")
    ref = G.bmm_a8w8_mxscale(a[1:], sa[1:], w, sw)
    assert_gemm_close(_gpu_bmm(a, sa, w, sw)[1:][:, :, cols], ref[:, :, cols], f"special scales K={K}")


def _sampled_check(p, q_dev, s_dev, rows, what):
    out = mx.mx_bmm_a8w8_mxscale(q_dev.view(p.T, p.G, p.K), s_dev.view(p.T, p.G, p.K // 128), dev_u8(p.w),
                                 dev_u8(p.w_scale))
    torch.cuda.synchronize()
    return host_u16(out)[rows]


def test_decode_batch_full_size():
    p = workloads.decode_batch()
    cos, sin = workloads.rope_tables(rows=32768)
    say("bmm decode batch")
    q, s = mx.mx_inv_rope_group_quant(dev_u16(p.x), dev_i64(p.positions), dev_u16(cos), dev_u16(sin),
                                      p.H, p.D, 64)
    rows = np.arange(p.T)
    out = _sampled_check(p, q, s, rows, "decode")
    rq, rs = inv_rope_group_quant(p.x, p.positions, cos, sin, p.H, p.D, 64)
    ref = G.bmm_a8w8_mxscale(rq.reshape(p.T, p.G, p.K), rs.reshape(p.T, p.G, -1), p.w, p.w_scale)
    assert_gemm_close(out, ref, "decode")


@pytest.mark.slow
def test_prefill_chunk_sampled_rows():
    p = workloads.prefill_chunk()
    cos, sin = workloads.rope_tables(rows=8192)
    say("bmm prefill chunk T=8192")
    q, s = mx.mx_inv_rope_group_quant(dev_u16(p.x), dev_i64(p.positions), dev_u16(cos), dev_u16(sin),
                                      p.H, p.D, 64)
    rows = np.unique(np.concatenate([[0, 255, 256, 8191], np.random.default_rng(12).integers(0, 8192, 28)]))
    out = _sampled_check(p, q, s, rows, "prefill")
    rq, rs = inv_rope_group_quant(p.x[rows], p.positions[rows], cos, sin, p.H, p.D, 64)
    ref = G.bmm_a8w8_mxscale(rq.reshape(len(rows), p.G, p.K), rs.reshape(len(rows), p.G, -1), p.w, p.w_scale)
    assert_gemm_close(out, ref, "prefill")


@pytest.mark.slow
def test_five_chunks_in_one_call():
    """T = 40960 (five prefill chunks) in one launch: the activations span
    2.7 GB, so rows from t = 32768 on start past byte 2^31.  Seeded random
    FP8 codes (no NaN code) and scale bytes, drawn on the device; sampled rows
    on both sides of that boundary are checked against the oracle."""
    T, Gn, N, K = 40960, 16, 1024, 4096
    say("bmm one call T=40960 G=16 N=1024 K=4096")
    _, _, w, sw = workloads.gemm_operands(515, 1, Gn, N, K)
    gen = torch.Generator(device="cuda").manual_seed(515)
    a = torch.randint(0, 256, (T, Gn, K), dtype=torch.uint8, device="cuda", generator=gen)
    a[(a & 0x7F) == 0x7F] = 0x7E
    sa = torch.randint(115, 126, (T, Gn, K // 128), dtype=torch.uint8, device="cuda", generator=gen)
    out = mx.mx_bmm_a8w8_mxscale(a, sa, dev_u8(w), dev_u8(sw))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 8191, 8192, 32767, 32768, 32769, T - 256, T - 1],
                                     np.random.default_rng(515).integers(0, T, 16)]))
    idx = torch.from_numpy(rows).cuda()
    got = host_u16(out[idx].contiguous())
    ra, rsa = a[idx].cpu().numpy(), sa[idx].cpu().numpy()
    del a, sa, out
    assert_gemm_close(got, G.bmm_a8w8_mxscale(ra, rsa, w, sw), "T=40960 one call")


@pytest.mark.slow
def test_activation_rows_past_4gib():
    """T = 65793 in one launch: the activations span 4.31 GB, so for the
    token tile at t0 = 256 the distance to the last row, (T - 1 - t0) rows of
    G*K bytes, is exactly 2^32 bytes.  The persistent kernel caps its row
    offsets at the tile's last valid row; a cap computed from that distance
    in 32 bits wraps to 0 and every row of the tile would read row 256.
    Sampled rows of that tile and around the other 2^32 multiples are checked
    against the oracle."""
    T, Gn, N, K = 65793, 16, 1024, 4096
    assert ((T - 1 - 256) * Gn * K) == 2 ** 32
    say("bmm one call T=65793 G=16 N=1024 K=4096")
    _, _, w, sw = workloads.gemm_operands(657, 1, Gn, N, K)
    gen = torch.Generator(device="cuda").manual_seed(657)
    a = torch.randint(0, 256, (T, Gn, K), dtype=torch.uint8, device="cuda", generator=gen)
    a[(a & 0x7F) == 0x7F] = 0x7E
    sa = torch.randint(115, 126, (T, Gn, K // 128), dtype=torch.uint8, device="cuda", generator=gen)
    out = mx.mx_bmm_a8w8_mxscale(a, sa, dev_u8(w), dev_u8(sw))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 256, 257, 300, 400, 511, 512, 65535, 65536, 65537, 65791, T - 1],
                                     np.random.default_rng(657).integers(256, 512, 8)]))
    idx = torch.from_numpy(rows).cuda()
    got = host_u16(out[idx].contiguous())
    ra, rsa = a[idx].cpu().numpy(), sa[idx].cpu().numpy()
    del a, sa, out
    assert_gemm_close(got, G.bmm_a8w8_mxscale(ra, rsa, w, sw), "T=65793 one call")
