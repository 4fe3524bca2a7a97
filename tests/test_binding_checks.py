"""The binding rejects tensors whose shapes do not match the sizes it passes
to the C ABI, before any pointer is taken: the library takes raw pointers and
could not tell a short tensor from a long one, so a wrong shape would become
an out-of-bounds device access.  CPU tensors suffice: the shape checks run
before the device checks.
"""

import pytest
import torch

import mx_scaled_fp8_amd as mx

u8 = torch.uint8
i16 = torch.int16


def z(*shape, dtype=u8):
    return torch.zeros(shape, dtype=dtype)


def _raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_quant_shapes():
    H, D, T = 4, 128, 8
    x, pos, cs = z(T, H * D, dtype=i16), z(T, dtype=torch.int64), z(64, 32, dtype=i16)
    _raises("x has shape", mx.mx_inv_rope_group_quant, z(T, H * D + 8, dtype=i16), pos, cs, cs, H, D, 64)
    _raises("x must be", mx.mx_inv_rope_group_quant, z(T * H * D, dtype=i16), pos, cs, cs, H, D, 64)
    _raises("positions has", mx.mx_inv_rope_group_quant, x, z(T - 1, dtype=torch.int64), cs, cs, H, D, 64)
    _raises("int64", mx.mx_inv_rope_group_quant, x, z(T, dtype=torch.int32), cs, cs, H, D, 64)
    _raises("cos has shape", mx.mx_inv_rope_group_quant, x, pos, z(64, 16, dtype=i16), cs, H, D, 64)
    _raises("sin has shape", mx.mx_inv_rope_group_quant, x, pos, cs, z(63, 32, dtype=i16), H, D, 64)
    _raises("needs positions", mx.mx_inv_rope_group_quant, x, None, cs, cs, H, D, 64)
    _raises("q has", mx.mx_inv_rope_group_quant, x, pos, cs, cs, H, D, 64, q=z(T, H * D - 1))
    _raises("scale has", mx.mx_inv_rope_group_quant, x, pos, cs, cs, H, D, 64, scale=z(T, 3))
    _raises("multiple of the group", mx.mx_inv_rope_group_quant, z(T, 96, dtype=i16), pos, cs, cs, 1, 96, 0)
    # correct shapes get as far as the device check
    _raises("GPU tensor", mx.mx_inv_rope_group_quant, x, pos, cs, cs, H, D, 64)


def test_bmm_shapes():
    T, G, N, K = 4, 2, 32, 256
    a, sa, w, sw = z(T, G, K), z(T, G, K // 128), z(G, N, K), z(G, N, K // 128)
    _raises("w has shape", mx.mx_bmm_a8w8_mxscale, a, sa, z(G, N, K + 128), sw)
    _raises("w has shape", mx.mx_bmm_a8w8_mxscale, a, sa, z(G + 1, N, K), sw)
    _raises("a_scale has", mx.mx_bmm_a8w8_mxscale, a, z(T, G, 1), w, sw)
    _raises("w_scale has", mx.mx_bmm_a8w8_mxscale, a, sa, w, z(G, N, 1))
    _raises("out has", mx.mx_bmm_a8w8_mxscale, a, sa, w, sw, out=z(T, G, N - 16, dtype=i16))
    _raises("must be", mx.mx_bmm_a8w8_mxscale, z(T, G * K), sa, w, sw)
    _raises("GPU tensor", mx.mx_bmm_a8w8_mxscale, a, sa, w, sw)


def test_bf16_arm_shapes():
    T, G, N, K = 4, 2, 32, 256
    _raises("w has shape", mx.mx_bmm_bf16, z(T, G, K, dtype=i16), z(G, N, K - 128, dtype=i16))
    _raises("out has", mx.mx_bmm_bf16, z(T, G, K, dtype=i16), z(G, N, K, dtype=i16), out=z(1, dtype=i16))
    x, pos, cs = z(T, 256, dtype=i16), z(T, dtype=torch.int64), z(16, 32, dtype=i16)
    _raises("out has", mx.mx_inv_rope_bf16, x, pos, cs, cs, 2, 128, 64, out=z(T, 128, dtype=i16))
    _raises("x has shape", mx.mx_inv_rope_bf16, x, pos, cs, cs, 2, 64, 64)


def test_linear_and_dequant_shapes():
    M, N, K = 8, 64, 1152
    x, w, ws = z(M, K, dtype=i16), z(N, K), z(N, K // 32)
    _raises("w has shape", mx.mx_linear, x, z(N, K - 32), ws)
    _raises("w_scale has", mx.mx_linear, x, w, z(N, K // 128))
    _raises("needs w_scale", mx.mx_linear, x, w, None)
    _raises("out has", mx.mx_linear, x, w, ws, out=z(M, N + 16, dtype=i16))
    _raises("w_scale has", mx.mx_dequant_mxfp8_to_bf16, w, z(N, K // 128))
    _raises("out has", mx.mx_dequant_mxfp8_to_bf16, w, ws, out=z(N, K // 2, dtype=i16))
    _raises("multiple of the block", mx.mx_dequant_mxfp8_to_bf16, z(N, 48), z(N, 1))
    _raises("w_scale has", mx.mx_dequant_mxfp8_to_bf16, w, z(N, K // 32), 128)


def test_converter_and_expand_shapes():
    _raises("out has", mx.mx_f32_pow2_to_e8m0_device, z(16, dtype=torch.float32), out=z(15))
    _raises("out has", mx.mx_f32_to_e4m3_device, z(16, dtype=torch.float32), out=z(17))
    _raises("GPU tensor", mx.mx_woa_expand_scales, z(2, 2, 2), 2, 256, 256, 128)    # [2, 2, 2] is right
    _raises("scale has", mx.mx_woa_expand_scales, z(2, 3, 2), 2, 256, 256, 128)
    _raises("out has", mx.mx_woa_expand_scales, z(2, 256, 2), 2, 256, 256, 1, out=z(2, 256, 1))
