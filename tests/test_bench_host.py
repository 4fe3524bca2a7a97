"""Host-side checks of bench.py's measurement arithmetic (no GPU).

The algorithmic byte and FLOP counts are pinned to the per-unit figures of
the workloads: the quantiser moves 3 + 1/128 bytes per element plus a
position and a 64-wide BF16 cos/sin row per token; the GEMM moves A, W, their
E8M0 scales (one per 128 K) and the BF16 output, and does 2*K FLOP per output
element.
"""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_quantiser_bytes():
    # 8192 tokens x 65536 channels: 197,120 B per token of data, 136 B of position and cos/sin
    assert bench.quant_bytes(8192, 65536) == 8192 * (65536 * 3 + 512 + 136) == 1_615_921_152
    assert bench.quant_bytes(64, 65536) == 12_624_384


def test_gemm_bytes_and_flops():
    assert bench.bmm_bytes(8192, 16, 1024, 4096) == 877_133_824
    assert bench.bmm_bytes(64, 16, 1024, 4096) == 73_957_376
    assert 2 * 8192 * 16 * 1024 * 4096 == 1_099_511_627_776


def test_traffic_lookup():
    t = bench.measured_traffic("bmm_persistent_kernel")
    # present while the kernel source matches the counters; never below the algorithmic bytes
    assert t is None or t >= bench.bmm_bytes(8192, 16, 1024, 4096)
    q = bench.measured_traffic("quant_kernel")
    assert q is None or q >= bench.quant_bytes(8192, 65536)
    assert bench.measured_traffic("no_such_kernel") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr


def test_parity_record_flags_each_kind_of_mismatch():
    """The bench's parity record on planted differences: identical results
    pass; a scale byte, a code two steps away, too many one-step codes, or a
    GEMM output outside 2^-7 |ref| + 1e-3 rms(ref) each fail it."""
    import numpy as np
    rng = np.random.default_rng(0)
    rq = rng.integers(0, 0x7E, (64, 256), dtype=np.uint8)
    rs = rng.integers(110, 130, (64, 2), dtype=np.uint8)
    ref = rng.standard_normal((64, 32))
    bits = (ref.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)     # truncation: within 2^-7
    ok = bench.parity_record(rq.copy(), rs.copy(), bits, rq, rs, ref, "same")
    assert ok["pass"] and ok["outputs_outside_bound"] == 0 and ok["worst_err_over_bound"] <= 1

    s2 = rs.copy(); s2[3, 1] ^= 1
    assert not bench.parity_record(rq, s2, bits, rq, rs, ref, "scale")["pass"]
    q2 = rq.copy(); q2[5, 7] = rq[5, 7] + 2
    assert not bench.parity_record(q2, rs, bits, rq, rs, ref, "code two steps")["pass"]
    q3 = rq.copy(); q3[0, :3] = rq[0, :3] + 1                                     # 3 > 1e-4 * 16384
    assert not bench.parity_record(q3, rs, bits, rq, rs, ref, "too many one-step codes")["pass"]
    b2 = bits.copy(); b2[2, 2] ^= 0x0040                                           # a mantissa bit high up
    r = bench.parity_record(None, None, b2, None, None, ref, "gemm")
    assert not r["pass"] and r["outputs_outside_bound"] >= 1
