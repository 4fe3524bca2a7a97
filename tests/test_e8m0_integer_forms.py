"""The integer forms of the E8M0 scale exponent that the HIP kernels use,
checked against the oracle's definition (e = ceil(log2(amax / M)), exact
rational arithmetic) for every finite BF16 amax, on the host.

* the quantiser's form (e8m0_exponent<EM> in the library's common header):
  e = max((bits >> 7) - 127 - EM + (mantissa field > 0x60), -127), with
  M = 1.75 * 2^EM (448: EM = 8 for OCP, 224: EM = 7 for FNUZ);
* the single-kernel wo_a's biased byte for OCP: max((bits - 0x3E1) >> 7, 0)
  with an arithmetic shift, which must equal e + 127.

These restate the kernels' arithmetic on purpose: the test pins that those
few integer operations are the definition, for all 32,640 inputs, including
zero and every subnormal (which reach -127 through the clamp)."""

import numpy as np

from oracle import formats as F


def _bf16_value(bits):
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def _quantiser_form(bits, em):
    return max((bits >> 7) - 127 - em + (1 if (bits & 0x7F) > 0x60 else 0), -127)


def _fused_byte_form(bits):
    v = (bits - 0x3E1) & 0xFFFFFFFF
    v = v - (1 << 32) if v >= (1 << 31) else v        # as a signed 32-bit value
    return max(v >> 7, 0)                              # Python's >> on a negative int is arithmetic


def test_every_finite_bf16_amax():
    for bits in range(0x7F80):
        amax = _bf16_value(bits)
        e_ocp = F.e8m0_exponent_for_amax(amax, F.OCP)
        e_fnuz = F.e8m0_exponent_for_amax(amax, F.FNUZ)
        assert _quantiser_form(bits, 8) == e_ocp, hex(bits)
        assert _quantiser_form(bits, 7) == e_fnuz, hex(bits)
        assert _fused_byte_form(bits) == e_ocp + 127, hex(bits)
