"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic (the one rounding it needs, float -> BF16 for the
inputs, is torch's own CPU cast).  Both the HIP path and the oracle receive
exactly these arrays.

Draw order is part of the recipe (numpy ``default_rng``, PCG64):

* tiny (seed 0): x (16, 512) std normal; W codes (2, 128, 256) uniform over
  the 254 non-NaN OCP e4m3 bytes; W scale exponents (2, 128, 2) uniform in
  [-8, -4].  Positions 0..15.
* prefill chunk (seed 1) / decode batch (seed 2): 655 outlier columns of the
  65,536 (1 % of the channels), for decode then the 64 positions uniform in
  [0, 32768); W codes (16, 1024, 4096); W scale exponents (16, 1024, 32) in
  [-8, -4]; last x (T, 65536) std normal with the outlier columns scaled by 20
  before rounding to BF16 (drawn last, so any prefix of rows is the same
  whatever T is).  Prefill positions are 0..8191.
* MXFP8 linear (seed 3): for K in (288, 576, 1152, 2304) in that order: x
  (64, K) std normal; W codes (4096, K); scale exponents (4096, K/32) in
  [-10, -4].
* shared-expert down_proj (seed 5): x (8, 2304) std normal; W codes
  (5120, 2304); scale exponents (5120, 72) in [-10, -4].  The TP-P shard is
  the first 2304/P columns of each (K = 2304, 1152, 576, 288 at TP1/2/4/8);
  decode batches of 1 and 8 rows take the first rows of x.
* long prefill (seed 4): outlier columns, W codes and scale exponents as the
  prefill chunk.  100,000 tokens = 12 chunks of 8192 + one of 1,696;
  positions 8192c + i.  Chunk c's activations are drawn on the GPU with
  torch's Philox generator seeded 4000 + c (13 GiB of BF16 would take minutes
  to draw on the host), std normal, outlier columns x 20, rounded to BF16;
  tests copy the rows they check back to the host for the oracle.

The rotary tables are the usual ones: omega_i = theta**(-2i/rope_dim), angle =
pos * omega_i in fp64, cos/sin rounded to float32 and then to BF16.
"""

import numpy as np
import torch

OCP_FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)

ROPE_DIM = 64
ROPE_THETA = 10000.0
TABLE_ROWS = 131072          # covers 100,008 prefill positions and 32,768 decode


def to_bf16_bits(x_f32):
    """float32 array -> BF16 bit patterns (uint16) via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rope_tables(rows=TABLE_ROWS, rope_dim=ROPE_DIM, theta=ROPE_THETA):
    """BF16 cos and sin tables [rows, rope_dim/2] (uint16 bits)."""
    i = np.arange(rope_dim // 2, dtype=np.float64)
    omega = theta ** (-2.0 * i / rope_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * omega[None, :]
    return to_bf16_bits(np.cos(ang).astype(np.float32)), to_bf16_bits(np.sin(ang).astype(np.float32))


def weight_codes(rng, shape):
    return OCP_FINITE_CODES[rng.integers(0, OCP_FINITE_CODES.size, size=shape)]


def scale_bytes(rng, shape, lo, hi):
    """E8M0 bytes of exponents uniform in [lo, hi]."""
    return (rng.integers(lo, hi + 1, size=shape) + 127).astype(np.uint8)


def activations(rng, T, width, outlier_cols=None):
    x = rng.standard_normal((T, width), dtype=np.float32)
    if outlier_cols is not None:
        x[:, outlier_cols] *= np.float32(20.0)
    return to_bf16_bits(x)


class WoA:
    """One ``wo_a`` problem: x [T, H*D] BF16 bits, positions, W [G,N,K], Ws [G,N,K/128]."""

    def __init__(self, name, T, H, D, G, N, x, positions, w, w_scale, rope_dim=ROPE_DIM):
        self.name, self.T, self.H, self.D, self.G, self.N = name, T, H, D, G, N
        self.K = H * D // G
        self.rope_dim = rope_dim
        self.x, self.positions, self.w, self.w_scale = x, positions, w, w_scale

    @property
    def flops(self):
        return 2 * self.T * self.G * self.N * self.K


def tiny():
    rng = np.random.default_rng(0)
    T, H, D, G, N = 16, 4, 128, 2, 128
    K = H * D // G
    x = activations(rng, T, H * D)
    w = weight_codes(rng, (G, N, K))
    ws = scale_bytes(rng, (G, N, K // 128), -8, -4)
    return WoA("tiny wo_a T=16 G=2 K=256 N=128", T, H, D, G, N, x,
               np.arange(T, dtype=np.int64), w, ws)


def _big(seed, T, decode, name, x_rows=None):
    rng = np.random.default_rng(seed)
    H, D, G, N = 128, 512, 16, 1024
    width = H * D
    K = width // G
    cols = rng.choice(width, size=round(0.01 * width), replace=False)
    if decode:
        positions = rng.integers(0, 32768, size=T).astype(np.int64)
    else:
        positions = np.arange(T, dtype=np.int64)
    w = weight_codes(rng, (G, N, K))
    ws = scale_bytes(rng, (G, N, K // 128), -8, -4)
    x = activations(rng, T if x_rows is None else x_rows, width, cols)
    return WoA(name, T, H, D, G, N, x, positions, w, ws)


def prefill_chunk():
    """T=8192, G=16, K=4096 (8 heads x 512), N=1024, seed 1."""
    return _big(1, 8192, False, "wo_a prefill chunk T=8192 G=16 K=4096 N=1024")


def decode_batch():
    """T=64 at random positions in [0, 32768), same shapes, seed 2."""
    return _big(2, 64, True, "wo_a decode batch T=64 G=16 K=4096 N=1024")


LINEAR_KS = (288, 576, 1152, 2304)


def mxfp8_linear():
    """{K: (x [64,K] BF16 bits, W [4096,K] codes, Ws [4096,K/32] bytes, Ws as FP32)}, seed 3."""
    rng = np.random.default_rng(3)
    M, N = 64, 4096
    out = {}
    for K in LINEAR_KS:
        x = activations(rng, M, K)
        w = weight_codes(rng, (N, K))
        ws = scale_bytes(rng, (N, K // 32), -10, -4)
        ws_f32 = np.ldexp(np.ones(ws.shape, dtype=np.float32), ws.astype(np.int32) - 127).astype(np.float32)
        out[K] = (x, w, ws, ws_f32)
    return out


DOWN_PROJ_N = 5120
DOWN_PROJ_K = 2304
DOWN_PROJ_TP = (1, 2, 4, 8)


def down_proj_shards():
    """{TP: (x [8, K] BF16 bits, W [5120, K] codes, Ws [5120, K/32] bytes)} with
    K = 2304 / TP: rank 0's share of the shared expert's row-parallel down_proj, seed 5."""
    rng = np.random.default_rng(5)
    x = activations(rng, 8, DOWN_PROJ_K)
    w = weight_codes(rng, (DOWN_PROJ_N, DOWN_PROJ_K))
    ws = scale_bytes(rng, (DOWN_PROJ_N, DOWN_PROJ_K // 32), -10, -4)
    out = {}
    for tp in DOWN_PROJ_TP:
        K = DOWN_PROJ_K // tp
        out[tp] = (np.ascontiguousarray(x[:, :K]), np.ascontiguousarray(w[:, :K]),
                   np.ascontiguousarray(ws[:, : K // 32]))
    return out


LONG_TOKENS = 100_000
CHUNK = 8192


def long_prefill_weights():
    """(outlier columns, W, Ws) of the 100,000-token stream, seed 4."""
    rng = np.random.default_rng(4)
    width, G, N = 128 * 512, 16, 1024
    K = width // G
    cols = rng.choice(width, size=round(0.01 * width), replace=False)
    w = weight_codes(rng, (G, N, K))
    ws = scale_bytes(rng, (G, N, K // 128), -8, -4)
    return cols, w, ws


def long_prefill_chunks(total=LONG_TOKENS, chunk=CHUNK):
    """[(start, length)] of the chunked 100,000-token prefill."""
    out, s = [], 0
    while s < total:
        n = min(chunk, total - s)
        out.append((s, n))
        s += n
    return out


def device_activations(c, T, width, outlier_cols, device):
    """Chunk c of the long prefill, drawn on `device`: BF16 [T, width] as int16 bits."""
    g = torch.Generator(device=device)
    g.manual_seed(4000 + c)
    x = torch.randn((T, width), generator=g, device=device, dtype=torch.float32)
    cols = torch.as_tensor(np.asarray(outlier_cols), device=device)
    x[:, cols] *= 20.0
    return x.to(torch.bfloat16).view(torch.int16)


def gemm_operands(seed, T, G, N, K, a_exp=(-12, -2), w_exp=(-8, -4)):
    """Stand-alone operands of the batched GEMM: uniform finite OCP codes for
    A and W, E8M0 bytes with exponents uniform in the given ranges."""
    rng = np.random.default_rng(seed)
    a = weight_codes(rng, (T, G, K))
    sa = scale_bytes(rng, (T, G, K // 128), *a_exp)
    w = weight_codes(rng, (G, N, K))
    sw = scale_bytes(rng, (G, N, K // 128), *w_exp)
    return a, sa, w, sw
