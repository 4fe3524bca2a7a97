"""Shared helpers of the GPU parity tests: moving arrays to and from the GPU
and the parity bounds.

Bounds (the acceptance rules of this library):
* FP8 codes and E8M0 scale bytes: bit-exact when the quantiser sees the same
  rotated BF16 tensor as the oracle; the fused rotation may differ by at most
  one FP8 code on at most 1e-4 of the elements (rounding ties).
* GEMM, linear: |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref), ref the unrounded
  fp64 oracle, rms over the checked outputs of one call.
* Dequantisation: bit-exact.
"""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import formats as F


def gpu_available():
    return torch.cuda.is_available()


requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def say(*a):
    """Progress line that names the case before a GPU step (flushed)."""
    print("[case]", *a, file=sys.stderr, flush=True)


def dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_i64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).cuda()


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t):
    return t.contiguous().cpu().numpy()


def assert_gemm_close(gpu_bits, ref64, what=""):
    g = F.bf16_to_f64(gpu_bits).astype(np.float64)
    ref = np.asarray(ref64, dtype=np.float64)
    assert g.shape == ref.shape
    rms = math.sqrt(float(np.mean(ref * ref))) if ref.size else 0.0
    bound = 2.0 ** -7 * np.abs(ref) + 1e-3 * rms
    err = np.abs(g - ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(bound, 1e-300), 0)), ref.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {ref.size} outside the bound; worst at {i}: "
                             f"gpu {g[i]!r} ref {ref[i]!r} bound {bound[i]!r}")
    return float((err / np.maximum(bound, 1e-300)).max()) if ref.size else 0.0


def assert_codes_close(gpu_q, ref_q, gpu_s, ref_s, fmt, exact, what=""):
    """Scales must match exactly; codes exactly, or (fused rotation) within
    one code on at most 1e-4 of the elements."""
    assert np.array_equal(gpu_s, ref_s), f"{what}: {int((gpu_s != ref_s).sum())} scale bytes differ"
    diff = gpu_q != ref_q
    if exact:
        assert not diff.any(), f"{what}: {int(diff.sum())} of {diff.size} codes differ"
        return 0
    n = int(diff.sum())
    assert n <= 1e-4 * diff.size, f"{what}: {n} of {diff.size} codes differ"
    if n:
        a = F.e4m3_decode(gpu_q[diff], fmt)
        b = F.e4m3_decode(ref_q[diff], fmt)
        # neighbouring codes: same sign, adjacent magnitudes
        step = np.abs(gpu_q[diff].astype(int) - ref_q[diff].astype(int))
        assert np.all((step == 1) | (np.abs(a - b) == 0)), f"{what}: a code differs by more than one step"
    return n
