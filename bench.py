"""Benchmark of the FP8 wo_a hot path on one MI355X.

One step = one pass of the wo_a path over an 8192-token prefill chunk
(T = 8192, G = 16 groups, K = 4096 = 8 heads x 512, N = 1024): the fused
inverse-RoPE + group-128 E8M0 FP8 quantiser, then the batched MX-scale FP8
GEMM.  Inputs are seeded synthetic tensors resident in HBM before the timed
region.  The headline value is the GEMM's FLOPs per step (2*T*G*N*K) divided
by the step time, in TFLOP/s.

Printed: one JSON line -- the headline, with `roofline` for the GEMM
(measured with HIP events on the stream the kernels run on), `cpu_baseline`
(the CPU oracle timed on a bounded sample of the same workload) and `parity`
(the timed run's codes, scales and outputs on that sample against the
oracle's), then `secondary`: the decode batch, the MXFP8 linear at its four
K (64 rows, and 8192 rows at N = 5120) and the 100,000-token chunked
prefill (OCP and FNUZ), each with its
roofline fraction, the oracle's time and a parity record, then the
production down_proj, the load-time dequant and the BF16 arm (the path the
FP8 one replaces).  The decode GEMM and the decode-M linear are also set
against a read-only stream of the same weights.  Progress goes to stderr.  The exit status is 3 if any parity record fails.

Timing: whole steps run back to back for --settle-ms of wall time (the
clocks and power settle under this load), then W untimed warm-up steps, then
K timed steps; no timed step is dropped.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
                       [--no-cpu-baseline] [--cpu-tokens N] [--no-secondary]
                       [--copy-calibration]
"""

import argparse
import ctypes
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "wo_a fused quant+MX-FP8 bmm TFLOP/s at T=8192 (%FP8 peak); quant HBM GB/s"
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def quant_bytes(T, L, group=128):
    """Algorithmic HBM bytes of the quantiser: BF16 in, FP8 out, one scale byte
    per group, plus the per-token position and cos/sin row (R = 64)."""
    return T * (L * 2 + L + L // group) + T * (8 + 2 * 64)


def bmm_bytes(T, G, N, K):
    """Algorithmic HBM bytes of one GEMM: A and its scales, W and its scales, BF16 out."""
    return T * G * K + T * G * K // 128 + G * N * K + G * N * K // 128 + T * G * N * 2


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain-copy calibration), or None
    when the summary is missing or the kernel's source changed since."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "wo_a_T8192_hbm_bytes.md")
    try:
        text = open(path).read()
        rec = json.loads(re.search(r"^traffic-json: (.*)$", text, re.M).group(1))[kernel]
        src = open(os.path.join(ROOT, rec["src"]), "rb").read()
    except (OSError, AttributeError, KeyError, ValueError):
        return None
    return rec["bytes"] if hashlib.sha256(src).hexdigest() == rec["src_sha256"] else None


class Timer:
    """HIP events recorded on the given torch stream (the stream the library launches on)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e


def run_env(torch):
    """Device, clocks and software versions the numbers were taken with."""
    prop = torch.cuda.get_device_properties(0)
    env = {"device": torch.cuda.get_device_name(0), "arch": getattr(prop, "gcnArchName", None),
           "compute_units": prop.multi_processor_count, "hbm_GiB": round(prop.total_memory / 2**30, 1),
           "max_sclk_MHz": None, "torch": torch.__version__, "hip": torch.version.hip, "git": None}
    try:
        env["git"] = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=os.path.dirname(os.path.abspath(__file__)),
                                    capture_output=True, text=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        # the runtime's peak shader clock (hipDeviceAttributeClockRate, in kHz)
        hip = ctypes.CDLL("libamdhip64.so")
        khz = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, torch.cuda.current_device()) == 0:
            env["max_sclk_MHz"] = khz.value // 1000
    except OSError:
        pass
    return env


def bench_prefill(mx, torch, workloads, steps, warmup, settle_ms, fmt=0):
    p = workloads.prefill_chunk()
    cos, sin = workloads.rope_tables(rows=8192)
    dev = torch.device("cuda:0")
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    x, cosd, sind = u16(p.x), u16(cos), u16(sin)
    pos = torch.from_numpy(p.positions).to(dev)
    w = torch.from_numpy(p.w).to(dev)
    ws = torch.from_numpy(p.w_scale).to(dev)
    L = p.H * p.D
    q = torch.empty((p.T, L), dtype=torch.uint8, device=dev)
    s = torch.empty((p.T, L // 128), dtype=torch.uint8, device=dev)
    out = torch.empty((p.T, p.G, p.N), dtype=torch.bfloat16, device=dev)
    qv, sv = q.view(p.T, p.G, p.K), s.view(p.T, p.G, p.K // 128)
    stream = torch.cuda.current_stream(dev)
    tm = Timer(torch, stream)

    def step():
        mx.mx_inv_rope_group_quant(x, pos, cosd, sind, p.H, p.D, 64, 0, 128, fmt, q=q, scale=s)
        mx.mx_bmm_a8w8_mxscale(qv, sv, w, ws, fmt, out=out)

    # settle: whole steps, back to back, until settle_ms of wall time have
    # passed (the chip's clocks and power settle under this load); then the
    # warm-up steps, then the timed ones.  No timed step is dropped.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for _ in range(8):
            step()
        settle_steps += 8
        torch.cuda.synchronize()
    settle_wall_ms = (time.perf_counter() - t_settle) * 1e3
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    marks = []
    t_wall = time.perf_counter()
    e0 = tm.event()
    for _ in range(steps):
        a = tm.event()
        mx.mx_inv_rope_group_quant(x, pos, cosd, sind, p.H, p.D, 64, 0, 128, fmt, q=q, scale=s)
        b = tm.event()
        mx.mx_bmm_a8w8_mxscale(qv, sv, w, ws, fmt, out=out)
        c = tm.event()
        marks.append((a, b, c))
    e1 = tm.event()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = e0.elapsed_time(e1)
    q_ms = np.array([a.elapsed_time(b) for a, b, _ in marks])
    b_ms = np.array([b.elapsed_time(c) for _, b, c in marks])
    # the same step in one kernel (mx_wo_a_fused), right after, on the same
    # resident chunk: `steps` launches, each timed
    fout = torch.empty_like(out)
    for _ in range(3):
        mx.mx_wo_a_fused(x, pos, cosd, sind, p.H, p.D, 64, w, ws, out=fout)
    fmarks = []
    for _ in range(steps):
        a = tm.event()
        mx.mx_wo_a_fused(x, pos, cosd, sind, p.H, p.D, 64, w, ws, out=fout)
        fmarks.append((a, tm.event()))
    torch.cuda.synchronize()
    f_ms = np.array([a.elapsed_time(b) for a, b in fmarks])
    return dict(p=p, total_ms=total_ms, wall_s=wall, q_ms=q_ms, b_ms=b_ms, L=L, q=q, s=s, out=out, f_ms=f_ms,
                fout=fout, settle={"ms": round(settle_wall_ms, 1), "steps": settle_steps, "requested_ms": settle_ms})


def fused_bytes(T, G, N, K):
    """Algorithmic HBM bytes of the one-kernel step: BF16 activations, W and
    its scales, the positions and one cos/sin row per token, BF16 out."""
    return T * G * K * 2 + G * N * K + G * N * K // 128 + T * (8 + 2 * 64) + T * G * N * 2


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return None


def cpu_baseline(workloads, tokens):
    """The oracle (as it stands) on the first `tokens` tokens of the same
    chunk; returns the baseline record and the oracle's codes, scales and
    fp64 GEMM output for those tokens."""
    from oracle.gemm import bmm_a8w8_mxscale
    from oracle.quant import inv_rope_group_quant
    p = workloads._big(1, 8192, False, "sample", x_rows=tokens)
    cos, sin = workloads.rope_tables(rows=8192)
    with np.errstate(invalid="ignore"):           # NaN BF16 patterns cast to fp64 on purpose
        t0 = time.perf_counter()
        rq, rs = inv_rope_group_quant(p.x, p.positions[:tokens], cos, sin, p.H, p.D, 64)
        t1 = time.perf_counter()
        ref = bmm_a8w8_mxscale(rq.reshape(tokens, p.G, p.K), rs.reshape(tokens, p.G, -1), p.w, p.w_scale)
        t2 = time.perf_counter()
    flops = 2 * tokens * p.G * p.N * p.K
    threads = blas_threads()
    cores = threads or len(os.sched_getaffinity(0))
    rec = {"value": flops / (t2 - t0) / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": f"first {tokens} of the 8192 tokens of the prefill chunk, all G/N/K; quant "
                     f"{t1 - t0:.2f} s single-threaded numpy, fp64 GEMM {t2 - t1:.2f} s on BLAS "
                     f"({threads} threads); host has {os.cpu_count()} CPUs, affinity "
                     f"{len(os.sched_getaffinity(0))}"}
    return rec, rq, rs, ref


def parity_record(gq, gs, gout_bits, rq, rs, ref, what):
    """Parity of GPU results against the oracle's, by the library's bars:
    scale bytes exact; codes within one step on at most 1e-4 of the elements;
    GEMM outputs within 2^-7 |ref| + 1e-3 rms(ref), rms over the checked
    outputs.  gq/gs may be None (GEMM only) and gout_bits None (quantiser only)."""
    rec = {"what": what}
    ok = True
    if gq is not None:
        from oracle.formats import e4m3_decode, OCP
        d = gq != rq
        n = int(d.sum())
        step_ok = True
        if n:
            step = np.abs(gq[d].astype(np.int64) - rq[d].astype(np.int64))
            step_ok = bool(np.all((step == 1) | (e4m3_decode(gq[d], OCP) == e4m3_decode(rq[d], OCP))))
        sm = int((gs != rs).sum())
        rec.update(codes_checked=int(gq.size), code_mismatches=n, code_mismatch_frac=n / max(1, gq.size),
                   scales_checked=int(gs.size), scale_mismatches=sm)
        ok &= sm == 0 and n <= 1e-4 * gq.size and step_ok
    if gout_bits is not None:
        from oracle.formats import bf16_to_f64
        g = bf16_to_f64(gout_bits).reshape(ref.shape)
        rms = math.sqrt(float(np.mean(ref * ref))) if ref.size else 0.0
        bound = 2.0 ** -7 * np.abs(ref) + 1e-3 * rms
        err = np.abs(g - ref)
        outside = int(np.sum(~(err <= bound)))
        nz = np.abs(ref) > 1e-3 * rms
        rec.update(outputs_checked=int(ref.size), outputs_outside_bound=outside,
                   worst_err_over_bound=float(np.max(err / np.maximum(bound, 1e-300))) if ref.size else 0.0,
                   max_abs_err=float(err.max()) if ref.size else 0.0,
                   max_rel_err=float(np.max(err[nz] / np.abs(ref[nz]))) if nz.any() else 0.0,
                   rms_ref=rms)
        ok &= outside == 0
    rec["pass"] = bool(ok)
    return rec


def time_graph(torch, record, calls, replays=20):
    """Device-side cost per call of `calls` calls recorded by `record`,
    captured in one HIP graph and replayed: replay time / replays / calls."""
    dev = torch.device("cuda:0")
    st = torch.cuda.Stream(device=dev)
    st.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(st):                 # warm-up outside the graph
        record()
    torch.cuda.current_stream(dev).wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        record()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / replays / calls


def event_median_us(torch, fn, n=50, warm=3):
    """Median and min of per-call HIP-event times on the current stream."""
    tm = Timer(torch, torch.cuda.current_stream(torch.device("cuda:0")))
    for i in range(warm):
        fn(i)
    ts = []
    for i in range(n):
        a = tm.event()
        fn(i)
        b = tm.event()
        ts.append((a, b))
    torch.cuda.synchronize()
    v = np.array([a.elapsed_time(b) for a, b in ts]) * 1e3
    return float(np.median(v)), float(v.min())


def bench_decode(mx, torch, workloads, cpu, calls=40):
    """The decode batch (T = 64 at random positions, G = 16, K = 4096, N = 1024):
    quantiser and GEMM with cold weights (copies rotating through more than
    the 256 MB last-level cache), a 40-call graph of the two (one weight per
    layer of a 40-layer stack), parity of every row against the oracle and
    the oracle's time."""
    dev = torch.device("cuda:0")
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    p = workloads.decode_batch()
    cos, sin = workloads.rope_tables(rows=32768)
    x, cosd, sind = u16(p.x), u16(cos), u16(sin)
    pos = torch.from_numpy(p.positions).to(dev)
    w0, ws0 = torch.from_numpy(p.w).to(dev), torch.from_numpy(p.w_scale).to(dev)
    wts = [(w0.clone(), ws0.clone()) for _ in range(calls)]          # 40 x 64.5 MiB
    L = p.H * p.D
    q = torch.empty((p.T, L), dtype=torch.uint8, device=dev)
    s = torch.empty((p.T, L // 128), dtype=torch.uint8, device=dev)
    out = torch.empty((p.T, p.G, p.N), dtype=torch.bfloat16, device=dev)
    qv, sv = q.view(p.T, p.G, p.K), s.view(p.T, p.G, p.K // 128)
    us_q, _ = event_median_us(torch, lambda i: mx.mx_inv_rope_group_quant(x, pos, cosd, sind, p.H, p.D, 64,
                                                                        q=q, scale=s))
    us_b, us_b_min = event_median_us(torch, lambda i: mx.mx_bmm_a8w8_mxscale(qv, sv, *wts[i % calls], out=out))

    def rec():
        for w, sw in wts:
            mx.mx_inv_rope_group_quant(x, pos, cosd, sind, p.H, p.D, 64, q=q, scale=s)
            mx.mx_bmm_a8w8_mxscale(qv, sv, w, sw, out=out)
    us_graph = time_graph(torch, rec, calls)
    # the GEMM alone in the same graph shape, and the read-only stream floor
    # of its cold weights (one pass over each copy, nothing computed)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def rec_bmm():
        for w, sw in wts:
            mx.mx_bmm_a8w8_mxscale(qv, sv, w, sw, out=out)

    def rec_floor():
        for w, _ in wts:
            mx.mx_stream_read(w, sink)
    us_bmm_graph = time_graph(torch, rec_bmm, calls)
    us_floor = time_graph(torch, rec_floor, calls)
    mx.mx_inv_rope_group_quant(x, pos, cosd, sind, p.H, p.D, 64, q=q, scale=s)
    mx.mx_bmm_a8w8_mxscale(qv, sv, w0, ws0, out=out)
    torch.cuda.synchronize()
    gq, gs = q.cpu().numpy(), s.cpu().numpy()
    gout = out.view(torch.int16).cpu().numpy().view(np.uint16)
    del wts, x, q, s, out, w0, ws0
    bb = bmm_bytes(p.T, p.G, p.N, p.K)
    qb = quant_bytes(p.T, L)
    r = {"workload": p.name,
         "quant": {"us": us_q, "GBps": qb / us_q / 1e3, "frac": qb / us_q / 1e3 / PEAK_HBM_GBS,
                   "algorithmic_bytes": qb},
         "bmm": {"us": us_b, "us_min": us_b_min, "GBps": bb / us_b / 1e3,
                 "roofline": {"bound": "hbm", "frac": bb / us_b / 1e3 / PEAK_HBM_GBS, "algorithmic_bytes": bb},
                 "TFLOPs": p.flops / us_b / 1e6, "weights": f"cold ({calls} rotating copies)"},
         "graph_40_calls": {"us_per_call": us_graph, "GBps": (bb + qb) / us_graph / 1e3,
                            "hbm_frac": (bb + qb) / us_graph / 1e3 / PEAK_HBM_GBS,
                            "note": "quantiser + GEMM per call, one weight per call"},
         "bmm_graph_40_calls": {"us_per_call": us_bmm_graph, "GBps": bb / us_bmm_graph / 1e3,
                                "vs_stream_floor": us_bmm_graph / us_floor},
         "stream_floor": {"us_per_call": us_floor, "GBps": p.G * p.N * p.K / us_floor / 1e3,
                          "bytes": p.G * p.N * p.K,
                          "note": "mx_stream_read over the same 40 cold weight copies, 40-call graph"}}
    if cpu:
        from oracle.gemm import bmm_a8w8_mxscale
        from oracle.quant import inv_rope_group_quant
        with np.errstate(invalid="ignore"):
            t0 = time.perf_counter()
            rq, rs = inv_rope_group_quant(p.x, p.positions, cos, sin, p.H, p.D, 64)
            t1 = time.perf_counter()
            ref = bmm_a8w8_mxscale(rq.reshape(p.T, p.G, p.K), rs.reshape(p.T, p.G, -1), p.w, p.w_scale)
            t2 = time.perf_counter()
        r["cpu_oracle"] = {"quant_s": t1 - t0, "bmm_s": t2 - t1, "cores": blas_threads(),
                           "note": "the whole decode batch; quantiser single-threaded numpy, fp64 GEMM on BLAS"}
        r["parity"] = parity_record(gq, gs, gout, rq, rs, ref, "every row of the decode batch")
    return r


def bench_linear(mx, torch, workloads, cpu, calls=40):
    """The MXFP8 linear, M = 64, N = 4096, K in {288, 576, 1152, 2304}: per-call
    device time in a 40-call graph (one weight per call), the load-time
    dequantisation for the unaligned K, parity of every output against the
    oracle (and of the FP32 power-of-two scales' lossless conversion), and
    the oracle's time."""
    dev = torch.device("cuda:0")
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    res = {}
    for K, (xh, wh, wsh, wsf) in workloads.mxfp8_linear().items():
        xd, wd = u16(xh), torch.from_numpy(wh).to(dev)
        M, N = xh.shape[0], wh.shape[0]
        # the scales arrive as FP32 powers of two and are converted on the device
        rej = torch.zeros(1, dtype=torch.int32, device=dev)
        wsd = mx.mx_f32_pow2_to_e8m0_device(torch.from_numpy(wsf).to(dev), reject_count=rej)
        conv_ok = bool(np.array_equal(wsd.cpu().numpy(), wsh)) and int(rej.item()) == 0
        rec = {"branch": "bf16 (dequantised at load)" if K % 128 else "block-scaled fp8"}
        if K % 128:
            dq_bytes = N * K * 3 + N * K // 32
            ob = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in range(calls)]
            copies = [(wd.clone(), wsd.clone()) for _ in range(calls)]

            def rec_dq():
                for (w, sw), o in zip(copies, ob):
                    mx.mx_dequant_mxfp8_to_bf16(w, sw, out=o)
            us_dq = time_graph(torch, rec_dq, calls)
            rec["dequant"] = {"us_per_call": us_dq, "GBps": dq_bytes / us_dq / 1e3,
                              "hbm_frac": dq_bytes / us_dq / 1e3 / PEAK_HBM_GBS, "algorithmic_bytes": dq_bytes}
            del copies
            wprep, wbytes, wl = ob, N * K * 2, [(o, wsd) for o in ob]
        else:
            wprep, wbytes = None, N * K + N * K // 32
            wl = [(wd.clone(), wsd.clone()) for _ in range(calls)]
        o = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        eb = wl[0][0].element_size()
        wsp = torch.empty(max(1, mx.mx_linear_workspace_bytes(M, N, K, eb)), dtype=torch.uint8, device=dev)

        def rec_lin():
            for w, sw in wl:
                mx.mx_linear(xd, w, sw, out=o, workspace=wsp)
        us = time_graph(torch, rec_lin, calls)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)

        def rec_floor():
            for w, _ in wl:
                mx.mx_stream_read(w, sink)
        us_floor = time_graph(torch, rec_floor, calls)
        lb = wbytes + M * K * 2 + M * N * 2
        rec["linear"] = {"us_per_call": us, "GBps": lb / us / 1e3,
                         "roofline": {"bound": "hbm", "frac": lb / us / 1e3 / PEAK_HBM_GBS, "algorithmic_bytes": lb},
                         "vs_stream_floor": us / us_floor,
                         "note": "40-call graph, one weight per call"}
        rec["stream_floor"] = {"us_per_call": us_floor, "bytes": wl[0][0].numel() * eb,
                               "note": "mx_stream_read over the same weights, 40-call graph"}
        mx.mx_linear(xd, wl[0][0], wl[0][1], out=o, workspace=wsp)
        torch.cuda.synchronize()
        gout = o.view(torch.int16).cpu().numpy().view(np.uint16)
        del wl, wprep
        if cpu:
            from oracle.gemm import mx_linear as oracle_linear
            t0 = time.perf_counter()
            ref = oracle_linear(xh, wh, wsh, 32)
            rec["cpu_oracle_us"] = (time.perf_counter() - t0) * 1e6
            rec["parity"] = parity_record(None, None, gout, None, None, ref, f"every output, K = {K}")
            rec["parity"]["f32_scales_to_e8m0_lossless"] = conv_ok
            rec["parity"]["pass"] = rec["parity"]["pass"] and conv_ok
        res[f"K{K}"] = rec
    return res


def bench_linear_prefill(mx, torch, workloads, cpu, M=8192, N=5120):
    """The MXFP8 linear at a prefill chunk's rows (M = 8192) and the pages'
    production N = 5120, K in {288, 576, 1152, 2304}: per-call time (event
    median), TFLOP/s against the branch's peak (BF16 for the dequantised
    weight, FP8 for the block-scaled one), every output checked against the
    oracle, and the oracle's time."""
    dev = torch.device("cuda:0")
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    res = {}
    for K in workloads.LINEAR_KS:
        rng = np.random.default_rng(9000 + K)
        xh = workloads.activations(rng, M, K)
        wh = workloads.weight_codes(rng, (N, K))
        wsh = workloads.scale_bytes(rng, (N, K // 32), -10, -4)
        xd, wd, wsd = u16(xh), torch.from_numpy(wh).to(dev), torch.from_numpy(wsh).to(dev)
        wprep = mx.mx_dequant_mxfp8_to_bf16(wd, wsd) if K % 128 else wd
        o = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsp = torch.empty(max(1, mx.mx_linear_workspace_bytes(M, N, K, wprep.element_size())), dtype=torch.uint8,
                          device=dev)
        us, us_min = event_median_us(torch, lambda i: mx.mx_linear(xd, wprep, wsd, out=o, workspace=wsp), n=20)
        flops = 2 * M * N * K
        peak = PEAK_BF16_TFLOPS if K % 128 else PEAK_FP8_TFLOPS
        rec = {"branch": "bf16 (dequantised at load)" if K % 128 else "block-scaled fp8 (x quantised per call)",
               "us": us, "us_min": us_min, "TFLOPs": flops / us / 1e6,
               "roofline": {"bound": "mfma", "peak": peak, "frac": flops / us / 1e6 / peak}}
        torch.cuda.synchronize()
        gout = o.view(torch.int16).cpu().numpy().view(np.uint16)
        del xd, wd, wsd, wprep, o, wsp
        if cpu:
            from oracle.gemm import mx_linear as oracle_linear
            with np.errstate(invalid="ignore"):
                t0 = time.perf_counter()
                ref = oracle_linear(xh, wh, wsh, 32)
                rec["cpu_oracle_s"] = time.perf_counter() - t0
            rec["parity"] = parity_record(None, None, gout, None, None, ref, f"every output, M = {M}, K = {K}")
        res[f"K{K}"] = rec
    return res


def bench_long(mx, torch, workloads, cpu):
    """The 100,000-token prefill streamed in 8192-token chunks (last 1,696),
    quantiser + GEMM per chunk, OCP then FNUZ activations; activations are
    generated on the GPU (seeded) and resident before timing.  Per-chunk
    events split the time between the two kernels.  The last chunk of each
    run is checked against the oracle (the oracle's time is reported), and
    the FNUZ run against the OCP run (scale bytes one higher, codes equal but
    0x80 -> 0x00, GEMM output bit-identical)."""
    dev = torch.device("cuda:0")
    tm = Timer(torch, torch.cuda.current_stream(dev))
    cols, w, ws = workloads.long_prefill_weights()
    wd, wsd = torch.from_numpy(w).to(dev), torch.from_numpy(ws).to(dev)
    cos, sin = workloads.rope_tables()
    cosd = torch.from_numpy(cos.view(np.int16)).to(dev)
    sind = torch.from_numpy(sin.view(np.int16)).to(dev)
    chunks = workloads.long_prefill_chunks()
    xs = [workloads.device_activations(c, n, 65536, cols, dev) for c, (_, n) in enumerate(chunks)]
    poss = [torch.arange(s0, s0 + n, dtype=torch.int64, device=dev) for s0, n in chunks]
    H, D, G, N, K = 128, 512, 16, 1024, 4096
    q = torch.empty((8192, H * D), dtype=torch.uint8, device=dev)
    s = torch.empty((8192, H * D // 128), dtype=torch.uint8, device=dev)
    out = torch.empty((8192, G, N), dtype=torch.bfloat16, device=dev)
    res, last = {}, {}
    total_tokens = sum(n for _, n in chunks)
    flops = 2 * total_tokens * G * N * K
    qbytes = sum(quant_bytes(n, H * D) for _, n in chunks)
    for fmt, name in ((0, "ocp"), (1, "fnuz")):
        def run(marks=None):
            for (s0, n), x, pos in zip(chunks, xs, poss):
                a = tm.event() if marks is not None else None
                mx.mx_inv_rope_group_quant(x, pos, cosd, sind, H, D, 64, 0, 128, fmt, q=q[:n], scale=s[:n])
                b = tm.event() if marks is not None else None
                mx.mx_bmm_a8w8_mxscale(q[:n].view(n, G, K), s[:n].view(n, G, K // 128), wd, wsd, fmt,
                                       out=out[:n])
                if marks is not None:
                    marks.append((a, b, tm.event()))
        run()
        torch.cuda.synchronize()
        a = tm.event()
        run()
        b = tm.event()
        marks = []
        run(marks)                               # a third pass with per-chunk events
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        q_us = sum(x.elapsed_time(y) for x, y, _ in marks) * 1e3
        b_us = sum(y.elapsed_time(z) for _, y, z in marks) * 1e3
        res[name] = {"ms": ms, "tokens_per_s": total_tokens / (ms / 1e3), "TFLOPs": flops / (ms / 1e3) / 1e12,
                     "quant_us_total": q_us, "quant_frac_hbm": qbytes / q_us / 1e3 / PEAK_HBM_GBS,
                     "bmm_us_total": b_us, "bmm_frac_fp8": flops / b_us / 1e6 / PEAK_FP8_TFLOPS}
        n = chunks[-1][1]
        last[name] = (q[:n].cpu().numpy(), s[:n].cpu().numpy(),
                      out[:n].view(torch.int16).cpu().numpy().view(np.uint16))
    res["chunks"] = [n for _, n in chunks]
    res["tokens"] = total_tokens
    c = len(chunks) - 1
    s0, n = chunks[c]
    xb = xs[c].cpu().numpy().view(np.uint16)
    del xs, q, s, out
    oq, os_, oo = last["ocp"]
    fq, fs, fo = last["fnuz"]
    ocp_scale_plus1 = np.where(os_ == 0xFF, 0xFF, os_.astype(np.int64) + 1)
    res["fnuz_vs_ocp_last_chunk"] = {
        "scales_are_ocp_plus_1": bool(np.array_equal(fs.astype(np.int64), ocp_scale_plus1)),
        "codes_are_ocp_with_negzero_cleared": bool(np.array_equal(fq, np.where(oq == 0x80, 0, oq))),
        "gemm_bit_identical": bool(np.array_equal(fo, oo))}
    if cpu:
        from oracle.formats import FNUZ, OCP
        from oracle.gemm import bmm_a8w8_mxscale
        from oracle.quant import inv_rope_group_quant
        pos = np.arange(s0, s0 + n, dtype=np.int64)
        for name, ofmt in (("ocp", OCP), ("fnuz", FNUZ)):
            with np.errstate(invalid="ignore"):
                t0 = time.perf_counter()
                rq, rs = inv_rope_group_quant(xb, pos, cos, sin, H, D, 64, fmt=ofmt)
                t1 = time.perf_counter()
                ref = bmm_a8w8_mxscale(rq.reshape(n, G, K), rs.reshape(n, G, -1), w, ws, a_fmt=ofmt)
                t2 = time.perf_counter()
            gq, gs, go = last[name]
            res[name]["cpu_oracle_last_chunk"] = {"tokens": n, "quant_s": t1 - t0, "bmm_s": t2 - t1,
                                                  "tokens_per_s": n / (t2 - t0), "cores": blas_threads()}
            res[name]["parity"] = parity_record(gq, gs, go.reshape(n, G, N), rq, rs, ref,
                                                f"last chunk ({n} tokens, every row)")
    return res


def bench_extra(mx, torch, workloads, fp8_step_us, fp8_bmm_us, decode_bmm_us):
    """The BF16 arm, the pages' production down_proj in 40-call graphs and
    the load-time dequantisation of its 5120 x 576 weight."""
    res = {"graph_40_calls": bench_graphs(mx, torch, workloads),
           "bf16_arm": bench_bf16_arm(mx, torch, workloads, fp8_step_us, fp8_bmm_us, decode_bmm_us)}
    return res


def bench_bf16_arm(mx, torch, workloads, fp8_step_us, fp8_bmm_us, fp8_decode_bmm_us, reps=30):
    """The BF16 wo_a arm (the path the FP8 one replaces): inverse RoPE to BF16,
    then the batched BF16 GEMM on the weight dequantised once at load (block
    128), on the same prefill chunk and decode batch; the FP8 arm's speedups
    are ratios of per-launch times measured in this process."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    tm = Timer(torch, stream)
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    def timeit(fn, n=reps):
        for _ in range(3):
            fn(0)
        ts = []
        for i in range(n):
            a = tm.event()
            fn(i)
            b = tm.event()
            ts.append((a, b))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ts])) * 1e3

    res = {}
    for name, prob, rows, copies in (("prefill_T8192", workloads.prefill_chunk, 8192, 1),
                                     ("decode_T64", workloads.decode_batch, 32768, 6)):
        p = prob()
        cos, sin = workloads.rope_tables(rows=rows)
        x, cosd, sind = u16(p.x), u16(cos), u16(sin)
        pos = torch.from_numpy(p.positions).to(dev)
        w8 = torch.from_numpy(p.w.reshape(p.G * p.N, p.K)).to(dev)
        ws8 = torch.from_numpy(p.w_scale.reshape(p.G * p.N, -1)).to(dev)
        wb = [mx.mx_dequant_mxfp8_to_bf16(w8, ws8, block=128).view(p.G, p.N, p.K) for _ in range(copies)]
        del w8, ws8
        L = p.H * p.D
        xr = torch.empty_like(x)
        out = torch.empty((p.T, p.G, p.N), dtype=torch.bfloat16, device=dev)
        us_copy = timeit(lambda i: mx.mx_inv_rope_bf16(x, pos, cosd, sind, p.H, p.D, 64, out=xr))
        xi = x.clone()       # rotated in place again and again: same cost every time
        us_inpl = timeit(lambda i: mx.mx_inv_rope_bf16(xi, pos, cosd, sind, p.H, p.D, 64, out=xi))
        us_bmm = timeit(lambda i: mx.mx_bmm_bf16(xr.view(p.T, p.G, p.K), wb[i % copies], out=out))
        rope_bytes_inpl = p.T * (p.H * 64 * 4 + 8 + 2 * 64)
        rope_bytes_copy = p.T * (L * 4 + 8 + 2 * 64)
        gemm_bytes = p.T * p.G * p.K * 2 + p.G * p.N * p.K * 2 + p.T * p.G * p.N * 2
        res[name] = {
            "rope_in_place_us": us_inpl, "rope_in_place_GBps": rope_bytes_inpl / us_inpl / 1e3,
            "rope_copy_us": us_copy, "rope_copy_GBps": rope_bytes_copy / us_copy / 1e3,
            "bmm_bf16_us": us_bmm, "bmm_bf16_TFLOPs": p.flops / us_bmm / 1e6,
            "bmm_bf16_frac_bf16_peak": p.flops / us_bmm / 1e6 / PEAK_BF16_TFLOPS,
            "bmm_bf16_GBps": gemm_bytes / us_bmm / 1e3,
            "step_us": us_inpl + us_bmm,
            "weights": "cold (6 rotating copies)" if copies > 1 else "resident",
        }
        if name == "prefill_T8192":
            res[name]["fp8_speedup_bmm"] = us_bmm / fp8_bmm_us
            res[name]["fp8_speedup_step"] = (us_inpl + us_bmm) / fp8_step_us
        else:
            res[name]["fp8_speedup_bmm"] = us_bmm / fp8_decode_bmm_us
        del x, xr, xi, out, wb
    return res


def bench_graphs(mx, torch, workloads, calls=40):
    """Device-side cost per call of the pages' production layer in 40-call
    graphs: the shared expert's down_proj (N = 5120) at each tensor-parallel
    share of K = 2304, decode batches of 1 and 8 rows, every branch the
    share allows, one weight per layer; and the load-time dequantisation of
    the 5120 x 576 weight."""
    dev = torch.device("cuda:0")
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    out = {}
    dp = {}
    for tp, (xh, wh, wsh) in workloads.down_proj_shards().items():
        N, K = wh.shape
        wd, wsd = torch.from_numpy(wh).to(dev), torch.from_numpy(wsh).to(dev)
        arms = {"fp8 block-scaled": wd} if K % 128 == 0 else {
            "per-call dequant": wd, "dequant once": mx.mx_dequant_mxfp8_to_bf16(wd, wsd)}
        for M in (1, 8):
            xd = u16(xh[:M])
            o = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            for arm, wprep in arms.items():
                copies = [(wprep.clone(), wsd.clone()) for _ in range(calls)]
                wsp = torch.empty(max(1, mx.mx_linear_workspace_bytes(M, N, K, wprep.element_size())),
                                  dtype=torch.uint8, device=dev)

                def rec_dp():
                    for w, sw in copies:
                        mx.mx_linear(xd, w, sw, out=o, workspace=wsp)
                us = time_graph(torch, rec_dp, calls)
                io = M * K * 2 + M * N * 2
                if arm == "per-call dequant":
                    b = N * K + N * K // 32 + N * K * 2 + N * K * 2 + io      # dequant pass + BF16 GEMM
                elif arm == "dequant once":
                    b = N * K * 2 + io
                else:
                    b = N * K + N * K // 32 + io
                dp[f"TP{tp}_K{K}_M{M}_{arm.replace(' ', '_')}"] = {
                    "us_per_call": us, "us_per_token_40_layers": 40 * us, "bytes_per_call": b,
                    "bytes_per_token_40_layers": 40 * b, "GBps": b / us / 1e3}
                del copies
        del arms, wd, wsd
    out["down_proj_decode_N5120"] = dp

    rng = np.random.default_rng(21)
    wd = torch.from_numpy(workloads.weight_codes(rng, (5120, 576))).to(dev)
    wsd = torch.from_numpy(workloads.scale_bytes(rng, (5120, 18), -10, -4)).to(dev)
    copies = [(wd.clone(), wsd.clone(), torch.empty((5120, 576), dtype=torch.bfloat16, device=dev))
              for _ in range(calls)]

    def rec_dq():
        for w, sw, ob in copies:
            mx.mx_dequant_mxfp8_to_bf16(w, sw, out=ob)
    us = time_graph(torch, rec_dq, calls)
    db = 5120 * 576 * 3 + 5120 * 18
    out["dequant_5120x576"] = {"us_per_call": us, "GBps": db / us / 1e3, "hbm_frac": db / us / 1e3 / PEAK_HBM_GBS}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    # under this load the chip's clocks and power take about 40 steps (30 ms)
    # to settle, GEMM launches in that ramp running up to 40% slower; whole
    # steps run back to back for this long before the warm-up steps
    ap.add_argument("--settle-ms", type=float, default=1000.0)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip every oracle leg (the CPU baseline and all parity records)")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the records beside the prefill chunk: decode batch, MXFP8 linear, 100,000-token "
                         "stream, production down_proj, load-time dequant and the BF16 arm")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with three plain 1 GiB device-to-device copies (the reference kernel for "
                         "scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the wo_a path runs and is measured on one MI355X only; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import mx_scaled_fp8_amd as mx
    import workloads

    mx.lib()
    if not torch.cuda.is_available() or not mx.mx_probe(0):
        print("bench.py: needs a gfx950 GPU and the built libmxfp8.so", file=sys.stderr)
        sys.exit(1)
    cpu = not args.no_cpu_baseline
    log(f"[bench] device {torch.cuda.get_device_name(0)}; generating the prefill chunk")
    r = bench_prefill(mx, torch, workloads, args.steps, args.warmup, args.settle_ms)
    p = r["p"]
    ms_step = r["total_ms"] / args.steps
    tflops = p.flops / (ms_step / 1e3) / 1e12
    b_avg_ms = float(r["b_ms"].mean())
    q_avg_ms = float(r["q_ms"].mean())
    b_ach = p.flops / (b_avg_ms / 1e3) / 1e12
    qb = quant_bytes(p.T, r["L"])
    q_gbs = qb / (q_avg_ms / 1e3) / 1e9
    log(f"[bench] settle {r['settle']['ms']:.0f} ms ({r['settle']['steps']} steps); step {ms_step * 1e3:.1f} us: "
        f"quant {q_avg_ms * 1e3:.1f} us ({q_gbs:.0f} GB/s), bmm {b_avg_ms * 1e3:.1f} us ({b_ach:.0f} TFLOP/s)")
    bq = np.percentile(r["b_ms"] * 1e3, [0, 50, 100])
    qq = np.percentile(r["q_ms"] * 1e3, [0, 50, 100])
    log(f"[bench] per-launch min/median/max: bmm {bq[0]:.1f}/{bq[1]:.1f}/{bq[2]:.1f} us, "
        f"quant {qq[0]:.1f}/{qq[1]:.1f}/{qq[2]:.1f} us")
    # the library runs the persistent large-tile kernel for K = 2048 and 4096
    # (16-byte aligned scales, as here), the one-tile-per-workgroup kernel otherwise
    bmm_kernel = "bmm_persistent_kernel" if p.K in (2048, 4096) else "bmm_large_kernel"
    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": p.name, "T": p.T, "G": p.G, "K": p.K, "N": p.N, "heads": p.H, "head_dim": p.D,
                   "rope_dim": 64, "quant_group": 128, "fp8": "OCP e4m3 + E8M0", "parallelism": "single GPU"},
        "settle": r["settle"],
        "pct_fp8_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
        "quant_hbm_GBps": round(q_gbs, 1),
        "quant": {"us": round(q_avg_ms * 1e3, 2), "GBps": round(q_gbs, 1), "frac": round(q_gbs / PEAK_HBM_GBS, 4),
                  "algorithmic_bytes": qb, "traffic": measured_traffic("quant_kernel")},
        "roofline": {"bound": "mfma", "kernel": bmm_kernel, "achieved": round(b_ach, 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(b_ach / PEAK_FP8_TFLOPS, 4),
                     "traffic": measured_traffic(bmm_kernel),
                     "launch_us": round(b_avg_ms * 1e3, 2),
                     "launch_us_min_median_max": [round(v, 1) for v in bq],
                     "algorithmic_flops": p.flops, "algorithmic_bytes": bmm_bytes(p.T, p.G, p.N, p.K)},
        "wall_s_timed_region": round(r["wall_s"], 4),
        "env": run_env(torch),
    }
    f_avg_ms = float(r["f_ms"].mean())
    fb = fused_bytes(p.T, p.G, p.N, p.K)
    rec["single_kernel_wo_a"] = {
        "kernel": "woa_fused_kernel", "launches": int(r["f_ms"].size), "us": round(f_avg_ms * 1e3, 2),
        "us_min_median_max": [round(v, 1) for v in np.percentile(r["f_ms"] * 1e3, [0, 50, 100])],
        "TFLOPs": round(p.flops / (f_avg_ms / 1e3) / 1e12, 1),
        "frac_fp8_peak": round(p.flops / (f_avg_ms / 1e3) / 1e12 / PEAK_FP8_TFLOPS, 4),
        "algorithmic_bytes": fb, "two_kernel_algorithmic_bytes": qb + bmm_bytes(p.T, p.G, p.N, p.K),
        "two_kernel_step_us": round(ms_step * 1e3, 2),
        "step_speedup_vs_two_kernels": round(ms_step / f_avg_ms, 4),
        "traffic": measured_traffic("woa_fused_kernel")}
    log(f"[bench] single-kernel wo_a: {f_avg_ms * 1e3:.1f} us per launch against the {ms_step * 1e3:.1f} us "
        f"two-kernel step")
    parity_ok = True
    if cpu:
        # the timed run's last results (every step computes the same values)
        T = args.cpu_tokens
        gq, gs = r["q"][:T].cpu().numpy(), r["s"][:T].cpu().numpy()
        gout = r["out"][:T].view(torch.int16).cpu().numpy().view(np.uint16)
        log(f"[bench] CPU oracle on {T} tokens")
        rec["cpu_baseline"], rq, rs, ref = cpu_baseline(workloads, T)
        rec["parity"] = parity_record(gq, gs, gout, rq, rs, ref,
                                      f"timed run vs oracle, first {T} tokens (rms over those outputs)")
        gf = r["fout"][:T].view(torch.int16).cpu().numpy().view(np.uint16)
        rec["single_kernel_wo_a"]["parity"] = parity_record(
            None, None, gf, None, None, ref, f"single-kernel wo_a vs oracle, first {T} tokens")
        parity_ok &= rec["parity"]["pass"] and rec["single_kernel_wo_a"]["parity"]["pass"]
        del gq, gs, gout, gf, rq, rs, ref
    del r
    torch.cuda.empty_cache()
    if not args.no_secondary:
        log("[bench] decode batch")
        dec = bench_decode(mx, torch, workloads, cpu)
        log("[bench] MXFP8 linear")
        lin = bench_linear(mx, torch, workloads, cpu)
        torch.cuda.empty_cache()
        log("[bench] MXFP8 linear, prefill rows")
        linp = bench_linear_prefill(mx, torch, workloads, cpu)
        torch.cuda.empty_cache()
        log("[bench] 100,000-token chunked prefill")
        lng = bench_long(mx, torch, workloads, cpu)
        rec["secondary"] = {"decode_T64": dec, "mxfp8_linear_M64_N4096": lin, "mxfp8_linear_M8192_N5120": linp,
                            "long_prefill_100k": lng}
        parities = [dec.get("parity"), *[v.get("parity") for v in lin.values()],
                    *[v.get("parity") for v in linp.values()], lng["ocp"].get("parity"), lng["fnuz"].get("parity")]
        parity_ok &= all(x["pass"] for x in parities if x is not None)
        parity_ok &= all(lng["fnuz_vs_ocp_last_chunk"].values())
        torch.cuda.empty_cache()
    if not args.no_secondary:
        log("[bench] production down_proj, load-time dequant, BF16 arm")
        dec_us = rec.get("secondary", {}).get("decode_T64", {}).get("bmm", {}).get("us", float("nan"))
        rec["extra"] = bench_extra(mx, torch, workloads, ms_step * 1e3, b_avg_ms * 1e3, dec_us)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    rec["parity_pass"] = bool(parity_ok) if cpu else None
    print(json.dumps(rec), flush=True)
    if not parity_ok:
        log("[bench] PARITY FAILURE: a GPU result is outside its bound against the oracle (see the JSON line)")
        sys.exit(3)


if __name__ == "__main__":
    main()
