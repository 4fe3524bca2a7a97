"""Python binding of libmxfp8, the MI355X (gfx950) FP8 ``wo_a`` library.

Argument marshalling only: every function below checks that its tensors are
contiguous and on the right device, allocates outputs with ``torch.empty``
(torch is used for device memory and streams), and calls the C entry point of
the same name on the current stream.  All arithmetic happens in the HIP
kernels of ``libmxfp8.so``; there is no fallback -- if the library is not
built, or a call fails, an exception is raised.

BF16 tensors may be passed as ``torch.bfloat16`` or as 16-bit integer bit
patterns; FP8 codes and E8M0 scales are ``torch.uint8``.
"""

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "MX_FP8_E4M3_OCP", "MX_FP8_E4M3_FNUZ", "MX_ROPE_INTERLEAVED", "MX_ROPE_NEOX",
    "MX_LINEAR_K_ALIGN", "MX_LINEAR_BLOCK", "MxError", "lib", "lib_path",
    "mx_probe", "mx_version", "mx_set_dry_run", "mx_get_counters", "mx_reset_counters",
    "mx_inv_rope_group_quant", "mx_bmm_a8w8_mxscale", "mx_wo_a_fused", "mx_dequant_mxfp8_to_bf16",
    "mx_linear_dequant_at_load", "mx_linear_workspace_bytes", "mx_linear", "mx_linear_noalloc",
    "MX_LINEAR_NOALLOC_SCRATCH_BYTES",
    "mx_inv_rope_bf16", "mx_bmm_bf16", "mx_woa_expand_scales", "MX_SCALE_E8M0", "MX_SCALE_F32",
    "mx_f32_pow2_to_e8m0", "mx_f32_pow2_to_e8m0_device", "mx_f32_to_e4m3_ocp",
    "mx_f32_to_e4m3_fnuz", "mx_f32_to_e4m3_device", "mx_e4m3_to_f32", "mx_e8m0_to_f32",
    "mx_stream_read", "COUNTER_NAMES",
]

MX_OK, MX_ERR_INVALID_ARG, MX_ERR_UNSUPPORTED, MX_ERR_NOT_LOSSLESS, MX_ERR_HIP = range(5)
MX_FP8_E4M3_OCP, MX_FP8_E4M3_FNUZ = 0, 1
MX_ROPE_INTERLEAVED, MX_ROPE_NEOX = 0, 1
MX_SCALE_E8M0, MX_SCALE_F32 = 0, 1
MX_LINEAR_K_ALIGN = 128
MX_LINEAR_BLOCK = 32
MX_LINEAR_NOALLOC_SCRATCH_BYTES = 32 << 20
COUNTER_NAMES = ("quant", "bmm_large", "bmm_small", "dequant", "linear_bf16", "linear_fp8",
                 "linear_percall_dequant", "f32_to_e8m0_device", "f32_to_e4m3_device", "rope_bf16",
                 "bmm_bf16_large", "bmm_bf16_small", "expand_scales", "wo_a_fused")

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxfp8.so")
_lib = None


class MxError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} [{status}]")
        self.status = status


def lib_path():
    return _LIB_PATH


def lib():
    """The loaded libmxfp8.so (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m mx_scaled_fp8_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "mx_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "mx_last_error": (ctypes.c_char_p, []),
            "mx_probe": (ctypes.c_int, [ctypes.c_int]),
            "mx_version": (ctypes.c_char_p, []),
            "mx_set_dry_run": (None, [ctypes.c_int]),
            "mx_get_counters": (ctypes.c_int, [P, ctypes.c_int]),
            "mx_reset_counters": (None, []),
            "mx_inv_rope_group_quant": (ctypes.c_int, [P, P, P, P, I64, I64, I32, I32, I32, I32, I32, I32, P, P, P]),
            "mx_bmm_a8w8_mxscale": (ctypes.c_int, [P, P, I32, P, P, P, I64, I32, I32, I32, P]),
            "mx_dequant_mxfp8_to_bf16": (ctypes.c_int, [P, P, P, I64, I64, I32, P]),
            "mx_inv_rope_bf16": (ctypes.c_int, [P, P, P, P, I64, I64, I32, I32, I32, I32, P, P]),
            "mx_bmm_bf16": (ctypes.c_int, [P, P, P, I64, I32, I32, I32, P]),
            "mx_woa_expand_scales": (ctypes.c_int, [P, I32, I32, I32, I32, I32, P, P, P]),
            "mx_wo_a_fused": (ctypes.c_int, [P, P, P, P, I64, I64, I32, I32, I32, I32, P, P, P, I32, I32, P]),
            "mx_linear_dequant_at_load": (ctypes.c_int, [I64]),
            "mx_linear_workspace_bytes": (SZ, [I64, I64, I64, I32]),
            "mx_linear": (ctypes.c_int, [P, I64, I64, P, P, I32, I64, P, P, SZ, P]),
            "mx_linear_noalloc": (ctypes.c_int, [P, I64, I64, P, P, I32, I64, P, P]),
            "mx_stream_read": (ctypes.c_int, [P, I64, P, P]),
            "mx_f32_pow2_to_e8m0": (ctypes.c_int, [P, P, I64]),
            "mx_f32_pow2_to_e8m0_device": (ctypes.c_int, [P, P, I64, P, P]),
            "mx_f32_to_e4m3_ocp": (ctypes.c_int, [P, P, I64]),
            "mx_f32_to_e4m3_fnuz": (ctypes.c_int, [P, P, I64]),
            "mx_f32_to_e4m3_device": (ctypes.c_int, [P, P, I64, I32, P]),
            "mx_e4m3_to_f32": (ctypes.c_int, [P, P, I64, I32]),
            "mx_e8m0_to_f32": (ctypes.c_int, [P, P, I64]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status, allow=()):
    if status != MX_OK and status not in allow:
        L = lib()
        raise MxError(L.mx_status_string(status).decode(), L.mx_last_error().decode())
    return status


def _dev(t, name, itemsize=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if itemsize is not None and t.element_size() != itemsize:
        raise ValueError(f"{name} must have {itemsize}-byte elements (got {t.dtype})")
    return t.data_ptr()


def _shape(t, shape, name):
    """Checks the exact shape of a tensor the sizes passed to the library are
    read from (before any pointer is taken: a wrong shape must not reach the
    C ABI, which takes raw pointers and cannot check it)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _numel(t, n, name):
    """Checks the element count of a tensor whose layout is fixed by the call
    (scales, outputs): any shape with exactly n elements is accepted."""
    if t is None:
        return
    if t.numel() != n:
        raise ValueError(f"{name} has {t.numel()} elements, expected {n} (shape {tuple(t.shape)})")


def _same_device(ref, *ts):
    for name, t in ts:
        if t is not None and isinstance(t, torch.Tensor) and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _rope_args(x, positions, cos, sin, T, rope_dim):
    """Shape and dtype checks of the rotation inputs; returns max_pos."""
    if rope_dim < 0 or rope_dim % 2:
        raise ValueError(f"rope_dim = {rope_dim} must be even and >= 0")
    if rope_dim == 0 or T == 0:
        return cos.shape[0] if cos is not None else 0
    if positions is None or cos is None or sin is None:
        raise ValueError("rope_dim > 0 needs positions, cos and sin")
    if positions.dtype != torch.int64:
        raise ValueError(f"positions must be int64 (got {positions.dtype})")
    _numel(positions, T, "positions")
    if cos.dim() != 2 or cos.shape[1] != rope_dim // 2:
        raise ValueError(f"cos has shape {tuple(cos.shape)}, expected [max_pos, {rope_dim // 2}]")
    _shape(sin, cos.shape, "sin")
    _same_device(x, ("positions", positions), ("cos", cos), ("sin", sin))
    return cos.shape[0]


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _host(a, dtype, name):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ status

def mx_probe(device=0):
    """True iff `device` is a gfx950 GPU the library runs on."""
    return lib().mx_probe(device) == MX_OK


def mx_version():
    return lib().mx_version().decode()


def mx_set_dry_run(on):
    lib().mx_set_dry_run(1 if on else 0)


def mx_get_counters():
    buf = (ctypes.c_uint64 * len(COUNTER_NAMES))()
    lib().mx_get_counters(ctypes.cast(buf, ctypes.c_void_p), len(COUNTER_NAMES))
    return dict(zip(COUNTER_NAMES, list(buf)))


def mx_reset_counters():
    lib().mx_reset_counters()


# ------------------------------------------------------- wo_a hot path

def mx_inv_rope_group_quant(x, positions, cos, sin, H, D, rope_dim, rope_style=MX_ROPE_INTERLEAVED,
                            group=128, fmt=MX_FP8_E4M3_OCP, q=None, scale=None):
    """x BF16 [T, H*D] -> (q uint8 [T, H*D], scale uint8 [T, H*D/group])."""
    if x.dim() != 2:
        raise ValueError(f"x must be [T, H*D] (got shape {tuple(x.shape)})")
    T = x.shape[0]
    _shape(x, (T, H * D), "x")
    if group <= 0 or (H * D) % group:
        raise ValueError(f"H*D = {H * D} is not a multiple of the group {group}")
    max_pos = _rope_args(x, positions, cos, sin, T, rope_dim)
    _numel(q, T * H * D, "q")
    _numel(scale, T * (H * D) // group, "scale")
    _same_device(x, ("q", q), ("scale", scale))
    if q is None:
        q = torch.empty((T, H * D), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((T, (H * D) // group), dtype=torch.uint8, device=x.device)
    _check(lib().mx_inv_rope_group_quant(
        _dev(x, "x", 2), _dev(positions, "positions", 8) if positions is not None else None,
        _dev(cos, "cos", 2) if cos is not None else None, _dev(sin, "sin", 2) if sin is not None else None,
        max_pos, T, H, D, rope_dim, rope_style, group, fmt,
        _dev(q, "q", 1), _dev(scale, "scale", 1), _stream(x)))
    return q, scale


def mx_bmm_a8w8_mxscale(a, a_scale, w, w_scale, a_fmt=MX_FP8_E4M3_OCP, out=None):
    """a uint8 [T,G,K], a_scale [T,G,K/128], w uint8 [G,N,K], w_scale [G,N,K/128] -> BF16 [T,G,N]."""
    if a.dim() != 3 or w.dim() != 3:
        raise ValueError(f"a must be [T,G,K] and w [G,N,K] (got {tuple(a.shape)} and {tuple(w.shape)})")
    T, G, K = a.shape
    N = w.shape[1]
    _shape(w, (G, N, K), "w")
    _numel(a_scale, T * G * (K // 128), "a_scale")
    _numel(w_scale, G * N * (K // 128), "w_scale")
    _numel(out, T * G * N, "out")
    _same_device(a, ("a_scale", a_scale), ("w", w), ("w_scale", w_scale), ("out", out))
    if out is None:
        out = torch.empty((T, G, N), dtype=torch.bfloat16, device=a.device)
    _check(lib().mx_bmm_a8w8_mxscale(_dev(a, "a", 1), _dev(a_scale, "a_scale", 1), a_fmt, _dev(w, "w", 1),
                                     _dev(w_scale, "w_scale", 1), _dev(out, "out", 2), T, G, N, K, _stream(a)))
    return out


def mx_wo_a_fused(x, positions, cos, sin, H, D, rope_dim, w, w_scale, rope_style=MX_ROPE_INTERLEAVED, out=None):
    """x BF16 [T, H*D], w uint8 [G, N, K] (K = H*D/G), w_scale [G, N, K/128] ->
    BF16 [T, G, N]: inverse RoPE, group-128 quantisation and the MX-scale GEMM
    in one kernel."""
    if x.dim() != 2 or w.dim() != 3:
        raise ValueError(f"x must be [T, H*D] and w [G,N,K] (got {tuple(x.shape)} and {tuple(w.shape)})")
    T = x.shape[0]
    _shape(x, (T, H * D), "x")
    G, N, K = w.shape
    if G * K != H * D:
        raise ValueError(f"w has shape {tuple(w.shape)}: G*K must be H*D = {H * D}")
    if K % 128:
        raise ValueError(f"K = {K} is not a multiple of 128")
    _numel(w_scale, G * N * (K // 128), "w_scale")
    max_pos = _rope_args(x, positions, cos, sin, T, rope_dim)
    _numel(out, T * G * N, "out")
    _same_device(x, ("w", w), ("w_scale", w_scale), ("out", out))
    if out is None:
        out = torch.empty((T, G, N), dtype=torch.bfloat16, device=x.device)
    _check(lib().mx_wo_a_fused(
        _dev(x, "x", 2), _dev(positions, "positions", 8) if positions is not None else None,
        _dev(cos, "cos", 2) if cos is not None else None, _dev(sin, "sin", 2) if sin is not None else None,
        max_pos, T, H, D, rope_dim, rope_style, _dev(w, "w", 1), _dev(w_scale, "w_scale", 1), _dev(out, "out", 2),
        G, N, _stream(x)))
    return out


def mx_woa_expand_scales(scale, G, N, K, block_n=1, out=None):
    """Checkpoint scales [G, ceil(N/block_n), K/128] (uint8 E8M0 or float32) ->
    (uint8 [G, N, K/128], number of rejected FP32 scales)."""
    kind = MX_SCALE_F32 if scale.dtype == torch.float32 else MX_SCALE_E8M0
    if kind == MX_SCALE_E8M0 and scale.element_size() != 1:
        raise ValueError("scale must be uint8 (E8M0) or float32")
    if block_n not in (1, 128) or G < 1 or N < 1 or K < 128 or K % 128:
        raise ValueError(f"block_n = {block_n}, G = {G}, N = {N}, K = {K} not accepted")
    _numel(scale, G * (-(-N // block_n)) * (K // 128), "scale")
    _numel(out, G * N * (K // 128), "out")
    _same_device(scale, ("out", out))
    if out is None:
        out = torch.empty((G, N, K // 128), dtype=torch.uint8, device=scale.device)
    rejects = torch.zeros(1, dtype=torch.int32, device=scale.device)
    _check(lib().mx_woa_expand_scales(_dev(scale, "scale"), kind, block_n, G, N, K, _dev(out, "out", 1),
                                      _dev(rejects, "reject_count", 4), _stream(scale)))
    return out, int(rejects.item())


# ------------------------------------------------------- BF16 arm of wo_a

def mx_inv_rope_bf16(x, positions, cos, sin, H, D, rope_dim, rope_style=MX_ROPE_INTERLEAVED, out=None):
    """x BF16 [T, H*D] -> rotated BF16 [T, H*D]; ``out=x`` rotates in place."""
    if x.dim() != 2:
        raise ValueError(f"x must be [T, H*D] (got shape {tuple(x.shape)})")
    T = x.shape[0]
    _shape(x, (T, H * D), "x")
    max_pos = _rope_args(x, positions, cos, sin, T, rope_dim)
    _numel(out, T * H * D, "out")
    _same_device(x, ("out", out))
    if out is None:
        out = torch.empty((T, H * D), dtype=x.dtype, device=x.device)
    _check(lib().mx_inv_rope_bf16(
        _dev(x, "x", 2), _dev(positions, "positions", 8) if positions is not None else None,
        _dev(cos, "cos", 2) if cos is not None else None, _dev(sin, "sin", 2) if sin is not None else None,
        max_pos, T, H, D, rope_dim, rope_style, _dev(out, "out", 2), _stream(x)))
    return out


def mx_bmm_bf16(x, w, out=None):
    """x BF16 [T,G,K], w BF16 [G,N,K] -> BF16 [T,G,N]."""
    if x.dim() != 3 or w.dim() != 3:
        raise ValueError(f"x must be [T,G,K] and w [G,N,K] (got {tuple(x.shape)} and {tuple(w.shape)})")
    T, G, K = x.shape
    N = w.shape[1]
    _shape(w, (G, N, K), "w")
    _numel(out, T * G * N, "out")
    _same_device(x, ("w", w), ("out", out))
    if out is None:
        out = torch.empty((T, G, N), dtype=torch.bfloat16, device=x.device)
    _check(lib().mx_bmm_bf16(_dev(x, "x", 2), _dev(w, "w", 2), _dev(out, "out", 2), T, G, N, K, _stream(x)))
    return out


# ------------------------------------------------------- measurement

def mx_stream_read(src, sink):
    """One read-only pass over the device tensor `src` (its bytes a multiple
    of 16): the HBM floor for weight-streaming calls.  `sink` is a device
    int32/uint32 tensor of at least one element, written only by chance."""
    nbytes = src.numel() * src.element_size()
    if nbytes % 16:
        raise ValueError(f"src has {nbytes} bytes, not a multiple of 16")
    if not isinstance(sink, torch.Tensor) or sink.numel() < 1:
        raise ValueError("sink must be a tensor of at least one element")
    _same_device(src, ("sink", sink))
    _check(lib().mx_stream_read(_dev(src, "src", src.element_size()), nbytes, _dev(sink, "sink", 4), _stream(src)))


# ------------------------------------------------------- MXFP8 linear

def mx_dequant_mxfp8_to_bf16(w, w_scale, block=MX_LINEAR_BLOCK, out=None):
    """w uint8 OCP [N,K], w_scale [N,K/block] -> BF16 [N,K]."""
    if w.dim() != 2:
        raise ValueError(f"w must be [N, K] (got shape {tuple(w.shape)})")
    N, K = w.shape
    if block not in (32, 128) or K % block:
        raise ValueError(f"K = {K} is not a multiple of the block {block} (32 or 128)")
    _numel(w_scale, N * (K // block), "w_scale")
    _numel(out, N * K, "out")
    _same_device(w, ("w_scale", w_scale), ("out", out))
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=w.device)
    _check(lib().mx_dequant_mxfp8_to_bf16(_dev(w, "w", 1), _dev(w_scale, "w_scale", 1), _dev(out, "out", 2),
                                          N, K, block, _stream(w)))
    return out


def mx_linear_dequant_at_load(K):
    return bool(lib().mx_linear_dequant_at_load(K))


def mx_linear_workspace_bytes(M, N, K, w_elem_bytes):
    return int(lib().mx_linear_workspace_bytes(M, N, K, w_elem_bytes))


def mx_linear(x, w, w_scale=None, out=None, workspace=None):
    """x BF16 [M,K] @ W^T; W is FP8 uint8 [N,K] (+ w_scale [N,K/32]) or BF16 [N,K]."""
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError(f"x must be [M,K] and w [N,K] (got {tuple(x.shape)} and {tuple(w.shape)})")
    M, K = x.shape
    N = w.shape[0]
    eb = w.element_size()
    _shape(w, (N, K), "w")
    if eb == 1:
        if w_scale is None:
            raise ValueError("an FP8 weight needs w_scale [N, K/32]")
        if K % MX_LINEAR_BLOCK:
            raise ValueError(f"K = {K} is not a multiple of {MX_LINEAR_BLOCK}")
        _numel(w_scale, N * (K // MX_LINEAR_BLOCK), "w_scale")
    _numel(out, M * N, "out")
    _same_device(x, ("w", w), ("w_scale", w_scale), ("out", out), ("workspace", workspace))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    need = mx_linear_workspace_bytes(M, N, K, eb)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().mx_linear(_dev(x, "x", 2), M, K, _dev(w, "w"),
                           _dev(w_scale, "w_scale", 1) if w_scale is not None else None, eb, N,
                           _dev(out, "out", 2), ws_ptr, ws_bytes, _stream(x)))
    return out


def mx_linear_noalloc(x, w, w_scale=None, out=None):
    """As mx_linear, with the library's own scratch instead of a workspace:
    the library allocates nothing (``out`` may be given to allocate nothing
    here either).  Overlapping calls on one GPU race on that scratch."""
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError(f"x must be [M,K] and w [N,K] (got {tuple(x.shape)} and {tuple(w.shape)})")
    M, K = x.shape
    N = w.shape[0]
    eb = w.element_size()
    _shape(w, (N, K), "w")
    if eb == 1:
        if w_scale is None:
            raise ValueError("an FP8 weight needs w_scale [N, K/32]")
        if K % MX_LINEAR_BLOCK:
            raise ValueError(f"K = {K} is not a multiple of {MX_LINEAR_BLOCK}")
        _numel(w_scale, N * (K // MX_LINEAR_BLOCK), "w_scale")
    _numel(out, M * N, "out")
    _same_device(x, ("w", w), ("w_scale", w_scale), ("out", out))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(lib().mx_linear_noalloc(_dev(x, "x", 2), M, K, _dev(w, "w"),
                                   _dev(w_scale, "w_scale", 1) if w_scale is not None else None, eb, N,
                                   _dev(out, "out", 2), _stream(x)))
    return out


# ---------------------------------------------------- format converters

def mx_f32_pow2_to_e8m0(x):
    """Host: float32 array -> (E8M0 uint8 array, ok); ok is False if any value did not convert."""
    src, p = _host(x, np.float32, "x")
    out = np.empty(src.shape, dtype=np.uint8)
    st = _check(lib().mx_f32_pow2_to_e8m0(p, out.ctypes.data_as(ctypes.c_void_p), src.size),
                allow=(MX_ERR_NOT_LOSSLESS,))
    return out, st == MX_OK


def mx_f32_pow2_to_e8m0_device(x, out=None, reject_count=None):
    """Device: float32 tensor -> E8M0 uint8 tensor; rejected values become 0xFF
    and are counted into `reject_count` (int32 GPU tensor of one element) if given."""
    _numel(out, x.numel(), "out")
    if reject_count is not None and reject_count.numel() < 1:
        raise ValueError("reject_count must hold one int32")
    _same_device(x, ("out", out), ("reject_count", reject_count))
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().mx_f32_pow2_to_e8m0_device(_dev(x, "x", 4), _dev(out, "out", 1), x.numel(),
                                            _dev(reject_count, "reject_count", 4) if reject_count is not None
                                            else None, _stream(x)))
    return out


def mx_f32_to_e4m3_ocp(x):
    src, p = _host(x, np.float32, "x")
    out = np.empty(src.shape, dtype=np.uint8)
    _check(lib().mx_f32_to_e4m3_ocp(p, out.ctypes.data_as(ctypes.c_void_p), src.size))
    return out


def mx_f32_to_e4m3_fnuz(x):
    src, p = _host(x, np.float32, "x")
    out = np.empty(src.shape, dtype=np.uint8)
    _check(lib().mx_f32_to_e4m3_fnuz(p, out.ctypes.data_as(ctypes.c_void_p), src.size))
    return out


def mx_f32_to_e4m3_device(x, fmt=MX_FP8_E4M3_OCP, out=None):
    _numel(out, x.numel(), "out")
    _same_device(x, ("out", out))
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().mx_f32_to_e4m3_device(_dev(x, "x", 4), _dev(out, "out", 1), x.numel(), fmt, _stream(x)))
    return out


def mx_e4m3_to_f32(codes, fmt=MX_FP8_E4M3_OCP):
    src, p = _host(codes, np.uint8, "codes")
    out = np.empty(src.shape, dtype=np.float32)
    _check(lib().mx_e4m3_to_f32(p, out.ctypes.data_as(ctypes.c_void_p), src.size, fmt))
    return out


def mx_e8m0_to_f32(b):
    src, p = _host(b, np.uint8, "b")
    out = np.empty(src.shape, dtype=np.float32)
    _check(lib().mx_e8m0_to_f32(p, out.ctypes.data_as(ctypes.c_void_p), src.size))
    return out
