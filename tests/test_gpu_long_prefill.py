"""GPU: the 100,000-token prefill streamed in 8192-token chunks (last 1,696),
once with OCP and once with FNUZ activation bytes.

Per chunk, on every element (properties that hold at any size): FNUZ scale
bytes are the OCP ones plus one, FNUZ codes are the OCP codes with 0x80 -> 0,
and the GEMM output of the FNUZ run is bit-identical to the OCP run.  Against
the oracle: 8 rows per chunk (first, last, six random), quantiser exact and
GEMM within the bound.  Also the literal 1,704-token chunk at positions
98,304 .. 100,007.
"""

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from helpers import assert_codes_close, assert_gemm_close, host_u16, host_u8, requires_gpu, say
from oracle import formats as F
from oracle import gemm as G
from oracle.quant import inv_rope_group_quant

pytestmark = [pytest.mark.gpu, requires_gpu, pytest.mark.slow]

H, D, GR, N, K = 128, 512, 16, 1024, 4096


def test_long_prefill_ocp_and_fnuz():
    dev = torch.device("cuda:0")
    cols, w, ws = workloads.long_prefill_weights()
    wd, wsd = torch.from_numpy(w).to(dev), torch.from_numpy(ws).to(dev)
    cos, sin = workloads.rope_tables()
    cosd = torch.from_numpy(cos.view(np.int16)).to(dev)
    sind = torch.from_numpy(sin.view(np.int16)).to(dev)
    chunks = workloads.long_prefill_chunks()
    assert len(chunks) == 13 and chunks[-1] == (98304, 1696)
    extra = (98304, 1704)                         # the literal last-chunk size, positions to 100,007
    rng = np.random.default_rng(44)
    xs_rows, pos_rows, q_rows, s_rows, o_rows = [], [], [], [], []
    for c, (s0, n) in enumerate(chunks + [extra]):
        say("long prefill chunk", c, s0, n)
        x = workloads.device_activations(c, n, H * D, cols, dev)
        pos = torch.arange(s0, s0 + n, dtype=torch.int64, device=dev)
        res = {}
        for fmt in (mx.MX_FP8_E4M3_OCP, mx.MX_FP8_E4M3_FNUZ):
            q, s = mx.mx_inv_rope_group_quant(x, pos, cosd, sind, H, D, 64, fmt=fmt)
            o = mx.mx_bmm_a8w8_mxscale(q.view(n, GR, K), s.view(n, GR, K // 128), wd, wsd, fmt)
            res[fmt] = (q, s, o)
        (qo, so, oo), (qf, sf, of) = res[0], res[1]
        assert torch.equal(sf.to(torch.int32), so.to(torch.int32) + 1)
        assert torch.equal(qf, torch.where(qo == 0x80, torch.zeros_like(qo), qo))
        assert torch.equal(of.view(torch.int16), oo.view(torch.int16))
        rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 6)]))
        ri = torch.from_numpy(rows).to(dev)
        xs_rows.append(host_u16(x[ri]))
        pos_rows.append(s0 + rows)
        q_rows.append(host_u8(qo[ri]))
        s_rows.append(host_u8(so[ri]))
        o_rows.append(host_u16(oo[ri]))
        del x, res, qo, so, oo, qf, sf, of
    xh = np.concatenate(xs_rows)
    ph = np.concatenate(pos_rows)
    rq, rs = inv_rope_group_quant(xh, ph, cos, sin, H, D, 64)
    n = assert_codes_close(np.concatenate(q_rows), rq, np.concatenate(s_rows), rs, F.OCP, exact=False,
                           what="long prefill quant")
    assert n == 0
    R = xh.shape[0]
    ref = G.bmm_a8w8_mxscale(rq.reshape(R, GR, K), rs.reshape(R, GR, -1), w, ws)
    assert_gemm_close(np.concatenate(o_rows), ref, "long prefill bmm")
