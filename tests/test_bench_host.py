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
