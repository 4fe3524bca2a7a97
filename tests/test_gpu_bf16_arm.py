"""GPU parity of the BF16 wo_a arm: mx_inv_rope_bf16 and mx_bmm_bf16.

* Inverse RoPE to BF16: bit-exact against the oracle's rotation (same fp32
  arithmetic, nearest-even BF16), both pairings, out of place and in place
  (in place touches only the rotated dims), rope_dim = 0 (a copy), positions
  outside the table (NaN in the rotated dims only), ragged and production
  head layouts.
* Batched BF16 GEMM: |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref) against the
  fp64 oracle over both small-T kernels (T <= 64: the LDS-DMA decode kernel
  for K of 512 to 4096, the split-K kernel otherwise) and the persistent tiles
  (K = 128 is a tile of only the two transition stages; ragged T and N
  tiles; several tiles per workgroup), run-to-run determinism.
* End to end: rotation, the group-128 dequantised weight, the GEMM, on the
  tiny problem and on the 8192-token prefill chunk (sampled rows).
"""

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from helpers import assert_gemm_close, dev_i64, dev_u16, dev_u8, host_u16, requires_gpu, say
from oracle import gemm as Gm
from oracle.rope import INTERLEAVED, NEOX, inverse_rope

pytestmark = [pytest.mark.gpu, requires_gpu]

STYLE = {INTERLEAVED: mx.MX_ROPE_INTERLEAVED, NEOX: mx.MX_ROPE_NEOX}


@pytest.fixture(scope="module")
def tables():
    cos, sin = workloads.rope_tables()
    return cos, sin, dev_u16(cos), dev_u16(sin)


def _gpu_rope(x, pos, tables, H, D, R, style=INTERLEAVED, in_place=False):
    _, _, dcos, dsin = tables
    dx = dev_u16(x)
    out = mx.mx_inv_rope_bf16(dx, dev_i64(pos), dcos, dsin, H, D, R, STYLE[style], out=dx if in_place else None)
    torch.cuda.synchronize()
    return host_u16(out)


ROPE_CASES = [(16, 4, 128, 64), (37, 3, 512, 64), (5, 2, 256, 128), (300, 128, 512, 64), (9, 1, 64, 16)]


@pytest.mark.parametrize("style", [INTERLEAVED, NEOX])
@pytest.mark.parametrize("T,H,D,R", ROPE_CASES)
def test_rope_bf16_bit_exact(tables, style, T, H, D, R):
    rng = np.random.default_rng(T * 7 + D)
    x = workloads.activations(rng, T, H * D)
    pos = rng.integers(0, 8192, T).astype(np.int64)
    cos, sin = workloads.rope_tables(rows=8192, rope_dim=R)          # [8192, R/2]
    tab = (cos, sin, dev_u16(cos), dev_u16(sin))
    say("rope bf16", style, T, H, D, R)
    ref = inverse_rope(x, pos, cos, sin, H, D, R, style)
    got = _gpu_rope(x, pos, tab, H, D, R, style)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} of {ref.size} differ"
    got_ip = _gpu_rope(x, pos, tab, H, D, R, style, in_place=True)
    assert np.array_equal(got_ip, ref), "in place differs"


def test_rope_bf16_in_place_touches_only_rotated_dims(tables):
    T, H, D, R = 64, 8, 512, 64
    rng = np.random.default_rng(5)
    x = workloads.activations(rng, T, H * D)
    pos = rng.integers(0, 8192, T).astype(np.int64)
    say("rope bf16 in place: pass-through dims")
    dx = dev_u16(x)
    before = host_u16(dx)
    mx.mx_inv_rope_bf16(dx, dev_i64(pos), tables[2], tables[3], H, D, R, out=dx)
    torch.cuda.synchronize()
    after = host_u16(dx).reshape(T, H, D)
    assert np.array_equal(after[:, :, : D - R], before.reshape(T, H, D)[:, :, : D - R])
    assert np.array_equal(after.reshape(T, H * D), inverse_rope(x, pos, tables[0], tables[1], H, D, R))


def test_rope_bf16_no_rotation_is_a_copy(tables):
    x = workloads.activations(np.random.default_rng(6), 33, 3 * 128)
    say("rope bf16 rope_dim = 0")
    out = mx.mx_inv_rope_bf16(dev_u16(x), None, None, None, 3, 128, 0)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(out), x)


def test_rope_bf16_positions_outside_the_table(tables):
    T, H, D, R = 6, 2, 128, 64
    x = workloads.activations(np.random.default_rng(7), T, H * D)
    cos, sin = tables[0][:100].copy(), tables[1][:100].copy()
    tab = (cos, sin, dev_u16(cos), dev_u16(sin))
    pos = np.array([0, 99, 100, -1, 5, 1 << 40], np.int64)
    say("rope bf16 bad positions")
    for in_place in (False, True):
        got = _gpu_rope(x, pos, tab, H, D, R, in_place=in_place).reshape(T, H, D)
        good = [0, 1, 4]
        ref = inverse_rope(x[good], pos[good], cos, sin, H, D, R).reshape(len(good), H, D)
        assert np.array_equal(got[good], ref)
        for t in (2, 3, 5):
            assert np.all(got[t, :, D - R:] == 0x7FC0)
            assert np.array_equal(got[t, :, : D - R], x.reshape(T, H, D)[t, :, : D - R])


def test_rope_bf16_empty(tables):
    x = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    out = mx.mx_inv_rope_bf16(x, torch.empty(0, dtype=torch.int64, device="cuda"), tables[2], tables[3], 4, 128, 64)
    assert out.shape == (0, 512)


# ---------------------------------------------------------------- GEMM

def _bf16_operands(seed, T, G, N, K):
    rng = np.random.default_rng(seed)
    x = workloads.activations(rng, T * G, K).reshape(T, G, K)
    w = workloads.activations(rng, G * N, K).reshape(G, N, K)
    return x, w


def _gpu_bmm_bf16(x, w):
    out = mx.mx_bmm_bf16(dev_u16(x), dev_u16(w))
    torch.cuda.synchronize()
    return host_u16(out)


BMM_SHAPES = [
    (1, 1, 16, 128), (7, 2, 48, 256),                                                 # small T, split-K kernel
    (64, 3, 128, 512), (16, 2, 1024, 4096), (33, 2, 272, 2048), (1, 1, 64, 1024),     # small T, decode kernel
    (65, 1, 16, 128), (300, 2, 272, 384), (256, 1, 256, 128), (513, 2, 784, 256),    # persistent
]


@pytest.mark.parametrize("T,Gn,N,K", BMM_SHAPES)
def test_bmm_bf16_random(T, Gn, N, K):
    x, w = _bf16_operands(3000 + T + N + K, T, Gn, N, K)
    say("bmm bf16", T, Gn, N, K)
    out = _gpu_bmm_bf16(x, w)
    assert_gemm_close(out, Gm.bmm_bf16(x, w), f"T={T} G={Gn} N={N} K={K}")


def _sample_rows(T, rng, n=40):
    edges = [0, T - 1] + [t for t in range(255, T, 256)] + [t for t in range(256, T, 256)]
    return np.unique(np.concatenate([np.array(edges), rng.integers(0, T, n)]))


# several tiles per workgroup (T = 4200, G = 5: 340 tiles), ragged edges
@pytest.mark.parametrize("T,Gn,N,K", [(1000, 3, 512, 4096), (4200, 5, 1024, 2048), (2600, 2, 784, 1152)])
def test_bmm_bf16_persistent_tiles(T, Gn, N, K):
    x, w = _bf16_operands(4000 + T, T, Gn, N, K)
    say("bmm bf16 persistent", T, Gn, N, K)
    out = _gpu_bmm_bf16(x, w)
    rows = _sample_rows(T, np.random.default_rng(T))
    assert_gemm_close(out[rows], Gm.bmm_bf16(x[rows], w), f"T={T} G={Gn} N={N} K={K}")


def test_bmm_bf16_deterministic():
    x, w = _bf16_operands(5, 700, 2, 512, 1024)
    dx, dw = dev_u16(x), dev_u16(w)
    say("bmm bf16 determinism")
    a = host_u16(mx.mx_bmm_bf16(dx, dw))
    b = host_u16(mx.mx_bmm_bf16(dx, dw))
    assert np.array_equal(a, b)


def test_bmm_bf16_empty():
    x = torch.empty((0, 2, 256), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((2, 64, 256), dtype=torch.bfloat16, device="cuda")
    assert mx.mx_bmm_bf16(x, w).shape == (0, 2, 64)


# ---------------------------------------------------------- end to end

def _bf16_weight_gpu(p):
    wb = mx.mx_dequant_mxfp8_to_bf16(dev_u8(p.w.reshape(p.G * p.N, p.K)),
                                     dev_u8(p.w_scale.reshape(p.G * p.N, -1)), block=128)
    return wb.view(p.G, p.N, p.K)


def test_bf16_arm_tiny_end_to_end(tables):
    p = workloads.tiny()
    cos, sin = tables[0], tables[1]
    say("bf16 arm tiny end to end")
    xr = mx.mx_inv_rope_bf16(dev_u16(p.x), dev_i64(p.positions), tables[2], tables[3], p.H, p.D, 64)
    out = mx.mx_bmm_bf16(xr.view(p.T, p.G, p.K), _bf16_weight_gpu(p))
    torch.cuda.synchronize()
    wb = Gm.dequant_mxfp8_to_bf16(p.w.reshape(p.G * p.N, p.K), p.w_scale.reshape(p.G * p.N, -1), 128)
    ref = Gm.wo_a_bf16(p.x, p.positions, cos, sin, p.H, p.D, 64, wb.reshape(p.G, p.N, p.K))
    assert_gemm_close(host_u16(out), ref, "tiny bf16 arm")


@pytest.mark.slow
def test_bf16_arm_prefill_chunk_sampled_rows(tables):
    p = workloads.prefill_chunk()
    cos, sin = tables[0], tables[1]
    say("bf16 arm prefill chunk T=8192")
    dx = dev_u16(p.x)
    mx.mx_inv_rope_bf16(dx, dev_i64(p.positions), tables[2], tables[3], p.H, p.D, 64, out=dx)   # in place
    out = mx.mx_bmm_bf16(dx.view(p.T, p.G, p.K), _bf16_weight_gpu(p))
    torch.cuda.synchronize()
    got = host_u16(out)
    rows = _sample_rows(p.T, np.random.default_rng(12), n=24)
    wb = Gm.dequant_mxfp8_to_bf16(p.w.reshape(p.G * p.N, p.K), p.w_scale.reshape(p.G * p.N, -1), 128)
    ref = Gm.wo_a_bf16(p.x[rows], p.positions[rows], cos, sin, p.H, p.D, 64, wb.reshape(p.G, p.N, p.K))
    assert_gemm_close(got[rows], ref, "prefill bf16 arm")
