"""mx_linear_noalloc -- the MXFP8 linear without a workspace argument (the
library's own scratch) -- against mx_linear, through the C ABI, on every
branch: two calls in a row, the second with a smaller input, each compared
bit for bit with mx_linear on the same inputs and with the oracle within the
GEMM bound.  The branches are told apart by the launch counters."""

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from helpers import assert_gemm_close, dev_u16, dev_u8, host_u16, requires_gpu, say
from oracle import gemm as G

pytestmark = [pytest.mark.gpu, requires_gpu]


def _case(seed, M, N, K):
    rng = np.random.default_rng(seed)
    x = workloads.activations(rng, M, K)
    w = workloads.weight_codes(rng, (N, K))
    ws = workloads.scale_bytes(rng, (N, K // 32), -10, -4)
    return x, w, ws


# (branch counter, prepared BF16 weight?, [(M, N, K) first call, second call smaller])
BRANCHES = [
    ("linear_fp8", False, [(64, 4096, 1152), (8, 1024, 1152)]),
    ("linear_fp8", False, [(40, 2048, 2304), (3, 512, 2304)]),
    ("linear_percall_dequant", False, [(16, 4096, 576), (5, 1024, 288)]),
    ("linear_bf16", True, [(64, 4096, 288), (1, 512, 288)]),
]


@pytest.mark.parametrize("branch,prepared,calls", BRANCHES, ids=lambda v: str(v))
def test_noalloc_matches_mx_linear(branch, prepared, calls):
    for i, (M, N, K) in enumerate(calls):
        x, w, ws = _case(100 * M + K + i, M, N, K)
        xd, wd, wsd = dev_u16(x), dev_u8(w), dev_u8(ws)
        if prepared:
            wd = mx.mx_dequant_mxfp8_to_bf16(wd, wsd)
        say("noalloc", branch, "call", i, "M N K", M, N, K)
        ref_gpu = mx.mx_linear(xd, wd, wsd)
        mx.mx_reset_counters()
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        got = mx.mx_linear_noalloc(xd, wd, wsd, out=out)
        torch.cuda.synchronize()
        c = mx.mx_get_counters()
        assert c[branch] == 1 and sum(c[k] for k in ("linear_bf16", "linear_fp8", "linear_percall_dequant")) == 1
        assert got.data_ptr() == out.data_ptr()
        assert np.array_equal(host_u16(got), host_u16(ref_gpu)), f"call {i}: differs from mx_linear"
        assert_gemm_close(host_u16(got), G.mx_linear(x, w, ws, 32), f"{branch} call {i}")


def test_noalloc_rejects_more_than_its_scratch():
    # per-call dequant of a 16384 x 1056 FP8 weight needs 34.6 MB of scratch
    M, N, K = 1, 16384, 1056
    assert mx.mx_linear_workspace_bytes(M, N, K, 1) > mx.MX_LINEAR_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    w = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    s = torch.zeros((N, K // 32), dtype=torch.uint8, device="cuda")
    mx.mx_reset_counters()
    with pytest.raises(mx.MxError, match="scratch"):
        mx.mx_linear_noalloc(x, w, s)
    assert sum(mx.mx_get_counters().values()) == 0
