"""CPU oracle for the FP8 ``wo_a`` path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, deliberately unoptimised numpy reference of
everything the HIP library computes.  It exists so that the GPU results can be
checked against something that a reader can verify by eye against the source
pages.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it; the product package never does, and this
package imports nothing from the product package (they share no code, tables or
constants).

Conventions: BF16 tensors are carried as ``uint16`` bit patterns, FP8 codes and
E8M0 scale bytes as ``uint8``.  Floating point is fp64 unless the method fixes
the precision (the rotation is defined in fp32).

Sources (cited by page title and section):

* vLLM pull request 54894, "[ROCm][DSV4][Perf] Use FP8 WO_A output projection"
  (Summary; Implementation) -- the fused inverse-RoPE + per-token group-128
  E8M0 quantiser and the batched a8w8 MX-scale GEMM, E8M0 scale ingestion.
* vLLM pull request 45681, "[ROCm][DSv4] Functional fixes for DeepSeek V4 on
  MI300X/MI325X" (Purpose) -- OCP vs FNUZ e4m3 bytes, FNUZ max 224.
* vLLM pull request 56560, "[ROCm][DSv4.1][Perf] Dequantize the MXFP8 weight
  once when dot_scaled cannot be used" (Purpose; Why it is worth a patch;
  review thread) -- MXFP8 dequant, the K % 128 dispatch.
* The first page again (Implementation) -- checkpoint scale ingestion:
  group-128 and 128 x 128 scale layouts, FP32 power-of-two scales.

Parity status of each function is listed in its docstring.  Functions with no
pin independent of themselves say "parity unpinned".
"""

from . import formats, rope, quant, gemm, ingest  # noqa: F401
