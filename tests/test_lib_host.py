"""Host-side checks of libmxfp8 (no GPU needed).

* The built library exports every function declared in include/mxfp8.h.
* The host encoders/converters agree with the oracle on every BF16 pattern
  scaled across the e4m3 range, on edge values, and on every E8M0 power.
* Argument validation: every device entry point rejects bad shapes, pointers
  and layouts with MX_ERR_INVALID_ARG before touching HIP; valid calls pass in
  dry-run mode.
* The MXFP8 linear's load/apply predicate follows the pages' branch table.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import mx_scaled_fp8_amd as mx
from conftest import ROOT, read_golden
from oracle import formats as F

pytestmark = pytest.mark.skipif(not os.path.exists(mx.lib_path()), reason="libmxfp8.so not built")


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "mxfp8.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = ctypes.CDLL(mx.lib_path())
    names = _declared_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def _bf16_grid():
    base = F.bf16_to_f32(np.arange(0x10000, dtype=np.uint16)).astype(np.float64)
    out = []
    for k in (-140, -20, -12, -9, -6, -3, 0, 3, 6, 9):
        v = np.ldexp(base, k)
        v = v[np.isfinite(v) | np.isnan(v)]
        out.append(v.astype(np.float32))
    edge = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 448, 464, 465, 480, 1e38, -1e38, 224, 232, 240, 241,
                     2.0 ** -9, 2.0 ** -10, 2.0 ** -11, 2.0 ** -149, -2.0 ** -149, 3.4e38], np.float32)
    return np.concatenate(out + [edge])


@pytest.mark.parametrize("fmt", [F.OCP, F.FNUZ])
def test_host_e4m3_encoder_matches_oracle(fmt):
    v = _bf16_grid()
    ours = mx.mx_f32_to_e4m3_ocp(v) if fmt == F.OCP else mx.mx_f32_to_e4m3_fnuz(v)
    ref = F.e4m3_encode(v.astype(np.float64), fmt)
    bad = np.flatnonzero(ours != ref)
    assert bad.size == 0, [(float(v[i]), hex(ours[i]), hex(ref[i])) for i in bad[:8]]


def test_host_e4m3_encoder_random_f32():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    for fmt, fn in ((F.OCP, mx.mx_f32_to_e4m3_ocp), (F.FNUZ, mx.mx_f32_to_e4m3_fnuz)):
        assert np.array_equal(fn(v), F.e4m3_encode(v.astype(np.float64), fmt))


@pytest.mark.parametrize("fmt,code", [(F.OCP, mx.MX_FP8_E4M3_OCP), (F.FNUZ, mx.MX_FP8_E4M3_FNUZ)])
def test_host_e4m3_decoder(fmt, code):
    c = np.arange(256, dtype=np.uint8)
    ours = mx.mx_e4m3_to_f32(c, code).astype(np.float64)
    ref = F.e4m3_decode(c, fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_host_e8m0_decoder():
    b = np.arange(256, dtype=np.uint8)
    ours = mx.mx_e8m0_to_f32(b).astype(np.float64)
    ref = F.e8m0_decode(b)
    assert np.isnan(ours[255]) and np.array_equal(ours[:255], ref[:255])


def test_host_f32_pow2_to_e8m0_matches_oracle():
    n = np.arange(-127, 128)
    powers = np.ldexp(np.ones(n.size, np.float32), n).astype(np.float32)
    b, ok = mx.mx_f32_pow2_to_e8m0(powers)
    assert ok and np.array_equal(b.astype(int), n + 127)
    rows = read_golden("e8m0_convert_cases.txt")
    x = np.array([int(r[0], 16) for r in rows], np.uint32).view(np.float32)
    b, ok = mx.mx_f32_pow2_to_e8m0(x)
    assert not ok
    ref_b, ref_ok = F.f32_pow2_to_e8m0(x)
    assert np.array_equal(b[ref_ok], ref_b[ref_ok])
    assert np.all(b[~ref_ok] == 0xFF)
    rng = np.random.default_rng(1)
    v = rng.integers(0, 2 ** 32, 100_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    b, _ = mx.mx_f32_pow2_to_e8m0(v)
    ref_b, ref_ok = F.f32_pow2_to_e8m0(v)
    assert np.array_equal(b[ref_ok], ref_b[ref_ok]) and np.all(b[~ref_ok] == 0xFF)


@pytest.mark.parametrize("row", read_golden("mxfp8_linear_dispatch.txt"), ids=lambda r: r[0])
def test_linear_predicate_table(row):
    K, branch = int(row[0]), row[2]
    assert mx.mx_linear_dequant_at_load(K) == (branch == "bf16")


def test_linear_workspace_sizes():
    assert mx.mx_linear_workspace_bytes(64, 4096, 576, 2) == 0
    assert mx.mx_linear_workspace_bytes(64, 4096, 576, 1) == 4096 * 576 * 2
    assert mx.mx_linear_workspace_bytes(64, 4096, 1152, 1) == 64 * 1152 + 64 * 1152 // 32


# ------------------------------------------------------------ validation

FAKE = 1 << 20   # a 16-byte aligned non-null address; never dereferenced in dry-run


def _call(name, *args):
    return getattr(mx.lib(), name)(*args)


@pytest.fixture
def dry():
    mx.mx_set_dry_run(True)
    yield
    mx.mx_set_dry_run(False)


def _quant(**kw):
    a = dict(x=FAKE, pos=FAKE, cos=FAKE, sin=FAKE, max_pos=100, T=16, H=4, D=128, R=64, style=0, group=128,
             fmt=0, q=FAKE, s=FAKE)
    a.update(kw)
    return _call("mx_inv_rope_group_quant", a["x"], a["pos"], a["cos"], a["sin"], a["max_pos"], a["T"], a["H"],
                 a["D"], a["R"], a["style"], a["group"], a["fmt"], a["q"], a["s"], None)


def test_quant_validation(dry):
    assert _quant() == mx.MX_OK
    assert _quant(T=0, x=None, q=None, s=None) == mx.MX_OK            # empty is a no-op
    for bad in (dict(T=-1), dict(H=0), dict(D=12), dict(group=64), dict(R=72), dict(R=8), dict(R=256),
                dict(style=2), dict(fmt=3), dict(x=None), dict(q=None), dict(pos=None), dict(x=FAKE + 8),
                dict(max_pos=0), dict(cos=FAKE + 4), dict(H=3, D=8)):
        assert _quant(**bad) == mx.MX_ERR_INVALID_ARG, bad
        assert mx.lib().mx_last_error().decode()
    assert _quant(R=0, pos=None, cos=None, sin=None) == mx.MX_OK        # no rotation needs no tables
    assert _quant(style=1, cos=FAKE + 8) == mx.MX_ERR_INVALID_ARG       # split halves read 16 bytes


def _fused(**kw):
    a = dict(x=FAKE, pos=FAKE, cos=FAKE, sin=FAKE, max_pos=100, T=16, H=128, D=512, R=64, style=0, w=FAKE,
             sw=FAKE, out=FAKE, G=16, N=1024)
    a.update(kw)
    return _call("mx_wo_a_fused", a["x"], a["pos"], a["cos"], a["sin"], a["max_pos"], a["T"], a["H"], a["D"],
                 a["R"], a["style"], a["w"], a["sw"], a["out"], a["G"], a["N"], None)


def test_wo_a_fused_validation(dry):
    assert _fused() == mx.MX_OK
    assert _fused(T=0, x=None, out=None) == mx.MX_OK                     # empty is a no-op
    assert _fused(R=0, pos=None, cos=None, sin=None) == mx.MX_OK
    for bad in (dict(T=-1), dict(H=0), dict(G=3), dict(N=100), dict(R=8), dict(style=2), dict(x=None),
                dict(out=FAKE + 2), dict(pos=None), dict(max_pos=0), dict(cos=FAKE + 4)):
        assert _fused(**bad) == mx.MX_ERR_INVALID_ARG, bad
    # shapes the one kernel does not take; the two calls serve them
    for unsupported in (dict(G=8),                                      # K = 8192
                        dict(R=128), dict(R=48, style=1),
                        dict(max_pos=(1 << 31) // 64),                  # 2 GiB cos table
                        dict(R=16, max_pos=1 << 27)):
        assert _fused(**unsupported) == mx.MX_ERR_UNSUPPORTED, unsupported
    assert _fused(max_pos=(1 << 31) // 64 - 1) == mx.MX_OK             # just under 2 GiB


def _bmm(**kw):
    a = dict(a=FAKE, sa=FAKE, fmt=0, w=FAKE, sw=FAKE, out=FAKE, T=64, G=16, N=1024, K=4096)
    a.update(kw)
    return _call("mx_bmm_a8w8_mxscale", a["a"], a["sa"], a["fmt"], a["w"], a["sw"], a["out"], a["T"], a["G"],
                 a["N"], a["K"], None)


def test_bmm_validation(dry):
    assert _bmm() == mx.MX_OK
    assert _bmm(T=0, a=None) == mx.MX_OK
    for bad in (dict(K=4000), dict(K=64), dict(N=100), dict(G=0), dict(T=-3), dict(fmt=7), dict(a=None),
                dict(w=FAKE + 4), dict(out=FAKE + 2), dict(sw=None)):
        assert _bmm(**bad) == mx.MX_ERR_INVALID_ARG, bad


def test_dequant_validation(dry):
    f = lambda **kw: _call("mx_dequant_mxfp8_to_bf16", kw.get("w", FAKE), kw.get("s", FAKE), kw.get("o", FAKE),
                           kw.get("N", 4096), kw.get("K", 576), kw.get("block", 32), None)
    assert f() == mx.MX_OK
    assert f(N=0, w=None) == mx.MX_OK
    for bad in (dict(K=100), dict(block=16), dict(K=576, block=128), dict(w=None), dict(o=FAKE + 8), dict(N=-1)):
        assert f(**bad) == mx.MX_ERR_INVALID_ARG, bad


def test_linear_validation(dry):
    def f(M=64, K=576, eb=1, N=4096, ws=FAKE, wsb=1 << 30, **kw):
        return _call("mx_linear", kw.get("x", FAKE), M, K, kw.get("w", FAKE), kw.get("s", FAKE), eb, N,
                     kw.get("o", FAKE), ws, wsb, None)
    assert f() == mx.MX_OK
    assert f(eb=2, ws=None, wsb=0) == mx.MX_OK                       # BF16 weight needs no workspace
    assert f(K=1152, wsb=64 * 1152 + 64 * 36) == mx.MX_OK
    assert f(ws=None, wsb=0) == mx.MX_ERR_INVALID_ARG               # unprepared FP8 unaligned: workspace needed
    assert f(wsb=4096 * 576 * 2 - 1) == mx.MX_ERR_INVALID_ARG
    assert f(K=100) == mx.MX_ERR_INVALID_ARG
    assert f(N=100) == mx.MX_ERR_INVALID_ARG
    assert f(eb=4) == mx.MX_ERR_INVALID_ARG
    assert f(s=None) == mx.MX_ERR_INVALID_ARG
    assert f(K=1152, M=65, wsb=65 * 1152 * 2) == mx.MX_OK             # prefill-sized M: the tiled kernel
    # K on its own past 2^31 (N small enough for N*K): rejected before any
    # kernel narrows it to 32 bits
    assert f(K=1 << 31, N=16, M=1, eb=2, ws=None, wsb=0) == mx.MX_ERR_INVALID_ARG
    assert f(K=32, N=1 << 31, M=1, eb=2, ws=None, wsb=0) == mx.MX_ERR_INVALID_ARG     # N past 32 bits
    assert f(K=32, N=1 << 20, M=1 << 20, eb=2, ws=None, wsb=0) == mx.MX_ERR_INVALID_ARG   # M*N = 2^40


def _rope_bf16(**kw):
    a = dict(x=FAKE, pos=FAKE, cos=FAKE, sin=FAKE, max_pos=100, T=16, H=4, D=128, R=64, style=0, out=FAKE * 4)
    a.update(kw)
    return _call("mx_inv_rope_bf16", a["x"], a["pos"], a["cos"], a["sin"], a["max_pos"], a["T"], a["H"], a["D"],
                 a["R"], a["style"], a["out"], None)


def test_rope_bf16_validation(dry):
    assert _rope_bf16() == mx.MX_OK
    assert _rope_bf16(out=FAKE) == mx.MX_OK                              # in place
    assert _rope_bf16(T=0, x=None, out=None) == mx.MX_OK
    assert _rope_bf16(R=0, pos=None, cos=None, sin=None) == mx.MX_OK     # a plain copy
    # x spans 16 * 512 * 2 = 16 KiB: an out that starts inside it overlaps
    for bad in (dict(T=-1), dict(H=0), dict(D=12), dict(R=72), dict(R=8), dict(R=256), dict(style=2),
                dict(x=None), dict(out=None), dict(pos=None), dict(x=FAKE + 8), dict(out=FAKE * 4 + 8),
                dict(max_pos=0), dict(cos=FAKE + 8), dict(out=FAKE + 4096), dict(x=FAKE * 4 + 1024)):
        assert _rope_bf16(**bad) == mx.MX_ERR_INVALID_ARG, bad
        assert mx.lib().mx_last_error().decode()
    assert _rope_bf16(out=FAKE + 16 * 512 * 2) == mx.MX_OK              # adjacent, not overlapping


def _bmm_bf16(**kw):
    a = dict(x=FAKE, w=FAKE, out=FAKE, T=8192, G=16, N=1024, K=4096)
    a.update(kw)
    return _call("mx_bmm_bf16", a["x"], a["w"], a["out"], a["T"], a["G"], a["N"], a["K"], None)


def test_bmm_bf16_validation(dry):
    assert _bmm_bf16() == mx.MX_OK
    assert _bmm_bf16(T=0, x=None) == mx.MX_OK
    for bad in (dict(K=4000), dict(K=64), dict(N=100), dict(G=0), dict(T=-3), dict(x=None), dict(w=FAKE + 4),
                dict(out=FAKE + 2), dict(G=2048, K=4096)):
        assert _bmm_bf16(**bad) == mx.MX_ERR_INVALID_ARG, bad


def test_expand_scales_validation(dry):
    f = lambda **kw: _call("mx_woa_expand_scales", kw.get("s", FAKE), kw.get("kind", 1), kw.get("bn", 128),
                           kw.get("G", 16), kw.get("N", 1024), kw.get("K", 4096), kw.get("o", FAKE),
                           kw.get("rc", FAKE), None)
    assert f() == mx.MX_OK
    assert f(kind=0, bn=1, rc=None) == mx.MX_OK
    for bad in (dict(kind=2), dict(bn=64), dict(G=0), dict(N=0), dict(K=4000), dict(K=64), dict(s=None),
                dict(o=None), dict(s=FAKE + 2), dict(rc=FAKE + 1), dict(G=65536, N=65536)):
        assert f(**bad) == mx.MX_ERR_INVALID_ARG, bad
    assert f(kind=0, s=FAKE + 1) == mx.MX_OK                           # E8M0 bytes need no alignment


def test_converter_validation(dry):
    assert _call("mx_f32_to_e4m3_device", FAKE, FAKE, 10, 0, None) == mx.MX_OK
    assert _call("mx_f32_to_e4m3_device", FAKE, FAKE, 10, 5, None) == mx.MX_ERR_INVALID_ARG
    assert _call("mx_f32_to_e4m3_device", None, FAKE, 10, 0, None) == mx.MX_ERR_INVALID_ARG
    assert _call("mx_f32_pow2_to_e8m0_device", FAKE, FAKE, -1, None, None) == mx.MX_ERR_INVALID_ARG
    assert _call("mx_f32_pow2_to_e8m0_device", FAKE + 2, FAKE, 4, None, None) == mx.MX_ERR_INVALID_ARG


def test_no_device_means_unsupported():
    """Without dry-run and without a GPU, a valid call reports MX_ERR_UNSUPPORTED
    (the caller's cue to fall back) and launches nothing."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _quant() == mx.MX_ERR_UNSUPPORTED
    assert mx.lib().mx_probe(0) == mx.MX_ERR_UNSUPPORTED


def test_linear_noalloc_validation(dry):
    def f(M=64, K=576, eb=1, N=4096, **kw):
        return _call("mx_linear_noalloc", kw.get("x", FAKE), M, K, kw.get("w", FAKE), kw.get("s", FAKE), eb, N,
                     kw.get("o", FAKE), None)
    assert f() == mx.MX_OK                                           # 4.7 MB of per-call dequant: fits
    assert f(K=1152) == mx.MX_OK
    assert f(eb=2) == mx.MX_OK
    assert f(N=16384, K=1056) == mx.MX_ERR_INVALID_ARG               # 34.6 MB > the 32 MiB scratch
    assert f(N=16384, K=1056, eb=2) == mx.MX_OK                      # a BF16 weight needs no scratch
    assert f(K=1152, M=8192) == mx.MX_OK                             # no scratch needed beyond 32 MiB
    assert f(K=100) == mx.MX_ERR_INVALID_ARG
    assert f(s=None) == mx.MX_ERR_INVALID_ARG
    assert f(M=0, x=None) == mx.MX_OK


def test_stream_read_validation(dry):
    def f(src=FAKE, nbytes=1 << 20, sink=FAKE):
        return _call("mx_stream_read", src, nbytes, sink, None)
    assert f() == mx.MX_OK
    assert f(nbytes=0, src=None, sink=None) == mx.MX_OK
    assert f(nbytes=24) == mx.MX_ERR_INVALID_ARG                     # not a multiple of 16
    assert f(nbytes=-16) == mx.MX_ERR_INVALID_ARG
    assert f(src=FAKE + 8) == mx.MX_ERR_INVALID_ARG                  # src not 16-byte aligned
    assert f(sink=FAKE + 2) == mx.MX_ERR_INVALID_ARG                 # sink not 4-byte aligned
    assert f(sink=None) == mx.MX_ERR_INVALID_ARG
