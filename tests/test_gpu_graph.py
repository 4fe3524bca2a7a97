"""GPU: the library's launches captured in a HIP graph.

The wo_a step (quantiser, then batched GEMM) and the MXFP8 linear on both
branches are captured in one graph.  The graph is replayed several times, with
eager work and synchronisations between the replays, and every replay must
equal the eager result bit for bit.  The library records no memset nodes.
"""

import numpy as np
import pytest
import torch

import mx_scaled_fp8_amd as mx
import workloads
from helpers import dev_i64, dev_u16, dev_u8, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def test_graph_replays_match_eager():
    dev = torch.device("cuda:0")
    T, H, D, G, N, K = 300, 16, 512, 2, 512, 4096     # persistent GEMM path (K = 4096), ragged T
    rng = np.random.default_rng(9)
    x = dev_u16(workloads.activations(rng, T, H * D))
    pos = dev_i64(rng.integers(0, 8192, T))
    cos, sin = workloads.rope_tables(rows=8192)
    cosd, sind = dev_u16(cos), dev_u16(sin)
    w = dev_u8(workloads.weight_codes(rng, (G, N, K)))
    ws = dev_u8(workloads.scale_bytes(rng, (G, N, K // 128), -8, -4))
    lx = dev_u16(workloads.activations(rng, 64, 1152))
    lw = dev_u8(workloads.weight_codes(rng, (256, 1152)))
    lws = dev_u8(workloads.scale_bytes(rng, (256, 1152 // 32), -10, -4))
    bx = dev_u16(workloads.activations(rng, 64, 288))
    bw_fp8 = dev_u8(workloads.weight_codes(rng, (256, 288)))
    bws = dev_u8(workloads.scale_bytes(rng, (256, 288 // 32), -10, -4))
    bw = mx.mx_dequant_mxfp8_to_bf16(bw_fp8, bws)

    q = torch.empty((T, H * D), dtype=torch.uint8, device=dev)
    s = torch.empty((T, H * D // 128), dtype=torch.uint8, device=dev)
    o = torch.empty((T, G, N), dtype=torch.bfloat16, device=dev)
    lo = torch.empty((64, 256), dtype=torch.bfloat16, device=dev)
    lwsp = torch.empty(mx.mx_linear_workspace_bytes(64, 256, 1152, 1), dtype=torch.uint8, device=dev)
    bo = torch.empty((64, 256), dtype=torch.bfloat16, device=dev)

    def step():
        mx.mx_inv_rope_group_quant(x, pos, cosd, sind, H, D, 64, q=q, scale=s)
        mx.mx_bmm_a8w8_mxscale(q.view(T, G, K), s.view(T, G, K // 128), w, ws, out=o)
        mx.mx_linear(lx, lw, lws, out=lo, workspace=lwsp)
        mx.mx_linear(bx, bw, None, out=bo)

    say("graph: eager reference")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (q, s, o, lo, bo)]

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(g):
        step()
    scratch = torch.empty(1 << 20, dtype=torch.float32, device=dev)
    for r in range(4):
        for t in (q, s, o, lo, bo):
            t.zero_()                              # the replay must rewrite every output
        scratch.normal_()                          # unrelated eager work between replays
        torch.cuda.synchronize()
        say("graph: replay", r)
        g.replay()
        torch.cuda.synchronize()
        for name, t, rt in zip(("q", "scale", "bmm", "linear fp8", "linear bf16"), (q, s, o, lo, bo), ref):
            assert torch.equal(t.view(torch.uint8), rt.view(torch.uint8)), f"replay {r}: {name} differs"
