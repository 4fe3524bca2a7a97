"""Pins of the oracle's checkpoint scale ingestion (oracle/ingest.py).

* The per-(g, n, 128-K block) E8M0 layout passes through unchanged.
* A ragged 128 x 128 layout (N = 300: blocks of 128, 128 and 44 rows) against
  a brute-force loop over every (g, n, kb).
* FP32 scales: every power of two 2^-127 .. 2^127 in a block converts to the
  pinned converter's byte; a block holding a value that is not a power of two
  in range (3.0, 0, -1, NaN, Inf, 2^-128) rejects exactly its own rows.
* Dequantising a weight with the expanded scales equals dequantising each
  128 x 128 block with its one scale (the meaning of the layout).
"""

import numpy as np

import workloads
from oracle import formats as F
from oracle import gemm as Gm
from oracle.ingest import E8M0, F32, expand_woa_scales


def test_per_row_e8m0_is_identity():
    s = workloads.scale_bytes(np.random.default_rng(1), (3, 40, 4), -8, -4)
    b, ok = expand_woa_scales(s, E8M0, 1, 3, 40, 512)
    assert np.array_equal(b, s) and ok.all()


def test_block128_brute_force_ragged():
    G, N, K = 2, 300, 384
    s = workloads.scale_bytes(np.random.default_rng(2), (G, 3, 3), -10, 10)
    b, ok = expand_woa_scales(s, E8M0, 128, G, N, K)
    assert b.shape == (G, N, 3) and ok.all()
    for g in range(G):
        for n in range(N):
            for kb in range(3):
                assert b[g, n, kb] == s[g, n // 128, kb]


def test_f32_powers_and_rejects():
    G, N, K = 1, 300, 256
    e = np.arange(-127, 128)
    vals = np.ldexp(np.float32(1), e).astype(np.float32)       # 2^-127 is an FP32 subnormal
    s = np.empty((G, 3, 2), np.float32)
    s[0, 0, 0], s[0, 0, 1] = vals[0], vals[-1]                  # 2^-127, 2^127
    s[0, 1, 0], s[0, 1, 1] = 1.0, 3.0                           # block (1, 1) is rejected
    s[0, 2, 0], s[0, 2, 1] = 0.5, np.float32(2.0 ** -20)
    b, ok = expand_woa_scales(s, F32, 128, G, N, K)
    want, wok = F.f32_pow2_to_e8m0(s)
    rows = np.arange(N) // 128
    assert np.array_equal(b, want[:, rows, :]) and np.array_equal(ok, wok[:, rows, :])
    assert b[0, 0, 0] == 0 and b[0, 0, 1] == 254 and b[0, 299, 0] == 126
    assert not ok[0, 128:256, 1].any() and ok[0, :128].all() and ok[0, 256:].all() and ok[0, 128:256, 0].all()
    for bad in (0.0, -1.0, np.nan, np.inf, np.float32(2.0 ** -128), np.float32(1.5)):
        s2 = np.ones((1, 1, 1), np.float32)
        s2[0, 0, 0] = bad
        _, ok2 = expand_woa_scales(s2, F32, 128, 1, 100, 128)
        assert not ok2.any(), bad
    # every in-range power of two, one per row
    s3 = vals.reshape(1, 255, 1)
    b3, ok3 = expand_woa_scales(s3, F32, 1, 1, 255, 128)
    assert ok3.all() and np.array_equal(b3[0, :, 0], np.arange(255))


def test_dequant_with_expanded_scales_is_blockwise():
    G, N, K = 2, 200, 256
    rng = np.random.default_rng(3)
    w = workloads.weight_codes(rng, (G, N, K))
    s = workloads.scale_bytes(rng, (G, 2, 2), -8, -4)
    b, _ = expand_woa_scales(s, E8M0, 128, G, N, K)
    got = Gm.dequant_mxfp8_to_bf16(w.reshape(G * N, K), b.reshape(G * N, 2), 128).reshape(G, N, K)
    for g in range(G):
        for nb in range(2):
            for kb in range(2):
                blk = w[g, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
                want = F.f64_to_bf16_rne(F.e4m3_decode(blk, F.OCP) * F.e8m0_decode(s[g, nb, kb]))
                assert np.array_equal(got[g, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128], want)
