"""Checkpoint scale ingestion for the wo_a weight -- oracle, test infrastructure.

"[ROCm][DSV4][Perf] Use FP8 WO_A output projection", Implementation: the
weight and scale layouts are validated as group-128 layouts before the fast
path is used, and power-of-two FP32 scales become E8M0 bytes without loss.
The pages name the checks, not the layouts, so the readings taken here are:

* a checkpoint holds either one scale per (g, n, 128-K block) -- the layout
  the GEMM reads, [G, N, K/128] -- or one per 128 x 128 (n, k) block of each
  group's weight, [G, ceil(N/128), K/128];
* a 128 x 128 block's scale applies to each of its 128 rows of n (the last
  block of a ragged N covers the rows that exist);
* a scale is E8M0 bytes already, or FP32 that must be 2**n with
  -127 <= n <= 127 (the lossless rule of formats.f32_pow2_to_e8m0); any other
  FP32 value is rejected.

Pins (tests/test_oracle_ingest.py): the per-row E8M0 layout is the identity;
a brute-force loop over a ragged 128 x 128 layout; FP32 scales agree with the
pinned converter and a rejected block rejects exactly its rows; dequantising
with the expanded scales equals dequantising each 128 x 128 block with its
own scale.
"""

import numpy as np

from .formats import f32_pow2_to_e8m0

E8M0 = "e8m0"
F32 = "f32"


def expand_woa_scales(scale, kind, block_n, G, N, K):
    """Checkpoint scales -> (E8M0 bytes uint8 [G, N, K/128], ok bool [G, N, K/128]).

    ``block_n`` is 1 (scale [G, N, K/128]) or 128 (scale [G, ceil(N/128), K/128]).
    Bytes are 0 where ok is False (an FP32 scale that is not a power of two in range).
    """
    assert K % 128 == 0 and block_n in (1, 128)
    kb = K // 128
    nb = -(-N // block_n)
    s = np.asarray(scale)
    assert s.shape == (G, nb, kb), (s.shape, (G, nb, kb))
    rows = np.arange(N) // block_n                     # source row of every n
    s = s[:, rows, :]
    if kind == E8M0:
        b = s.astype(np.uint8)
        return b, np.ones(b.shape, dtype=bool)
    assert kind == F32
    return f32_pow2_to_e8m0(s.astype(np.float32))
