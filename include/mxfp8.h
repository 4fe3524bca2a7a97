/*
 * mxfp8.h -- C ABI of the MI355X (gfx950) FP8 wo_a library.
 *
 * The library implements the FP8 path of a DeepSeek-V4-style `wo_a` output
 * projection and the MXFP8 linear that feeds on the same formats:
 *
 *   attention output (BF16) --inverse RoPE + per-token group-128 E8M0 FP8 quant-->
 *   FP8 codes + E8M0 scales --batched a8w8 MX-scale GEMM with the FP8 weight--> BF16
 *
 * Sources (cited by page title and section):
 *  [WOA]   vLLM pull request 54894, "[ROCm][DSV4][Perf] Use FP8 WO_A output projection"
 *  [FNUZ]  vLLM pull request 45681, "[ROCm][DSv4] Functional fixes for DeepSeek V4 on MI300X/MI325X"
 *  [MXLIN] vLLM pull request 56560, "[ROCm][DSv4.1][Perf] Dequantize the MXFP8 weight once
 *          when dot_scaled cannot be used"
 *
 * Conventions for every entry point:
 *  - Tensor arguments are raw pointers.  "device" pointers must point to GPU
 *    memory of the current HIP device; "host" pointers to CPU memory.  The
 *    caller owns all memory (inputs, outputs, workspaces); the library
 *    allocates no device memory and keeps no tensor state (the one exception,
 *    mx_linear_noalloc's fixed scratch array, is part of the loaded code).
 *  - Layouts are dense, row-major, last index contiguous, exactly as written
 *    in each comment ([T, G, K] means element (t,g,k) at offset (t*G+g)*K+k).
 *  - BF16 is passed as 16-bit patterns, FP8 e4m3 codes and E8M0 scale bytes as
 *    bytes.  E8M0 byte b means 2^(b-127); 0xFF is NaN.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Device entry points
 *    only enqueue work and return; nothing synchronises.  Faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  - Every entry point validates its arguments before touching the GPU and
 *    returns an mx_status; nothing throws or aborts.  On failure no work is
 *    enqueued and mx_last_error() holds a per-thread description.
 *  - Device entry points require a gfx950 device; elsewhere they return
 *    MX_ERR_UNSUPPORTED, the caller's cue to take its own fallback ([WOA],
 *    Summary and Dependency: unsupported devices keep the BF16 path).
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MX_OK = 0,
  MX_ERR_INVALID_ARG = 1,   /* a pointer, size, alignment or layout is not accepted        */
  MX_ERR_UNSUPPORTED = 2,   /* no gfx950 device / no HIP runtime: take your fallback       */
  MX_ERR_NOT_LOSSLESS = 3,  /* FP32 -> E8M0: an input is not a power of two in range       */
  MX_ERR_HIP = 4            /* a HIP runtime call (launch) failed                          */
} mx_status;

/* FP8 e4m3 byte flavours ([FNUZ], Purpose): OCP (bias 7) saturates at 448,
 * FNUZ (bias 8, NaN 0x80, no -0) is used up to 224. */
typedef enum { MX_FP8_E4M3_OCP = 0, MX_FP8_E4M3_FNUZ = 1 } mx_fp8_format;

/* Pairing of the rotated dims: interleaved (2i, 2i+1) or split halves (i, i+R/2). */
typedef enum { MX_ROPE_INTERLEAVED = 0, MX_ROPE_NEOX = 1 } mx_rope_style;

/* The alignment that picks the MXFP8 linear's branch ([MXLIN], Purpose: the scaled
 * product needs K % 128 == 0).  Load-time preparation and the per-call dispatch
 * both key off this one constant. */
#define MX_LINEAR_K_ALIGN 128
/* MXFP8 block size along K of the linear's weight scales. */
#define MX_LINEAR_BLOCK 32
/* Quantisation group of the wo_a activations and weight ([WOA], Summary). */
#define MX_WOA_GROUP 128

/* Element type of checkpoint scales given to mx_woa_expand_scales. */
typedef enum { MX_SCALE_E8M0 = 0, MX_SCALE_F32 = 1 } mx_scale_kind;

/* ------------------------------------------------------------------ status */

/* Static text for a status code. */
const char* mx_status_string(int status);
/* Per-thread description of the last failure (empty string if none). */
const char* mx_last_error(void);
/* MX_OK if `device` is a gfx950 GPU the library can run on, else
 * MX_ERR_UNSUPPORTED.  Cached per device; with MX_LOG=1 in the environment the
 * first result per device is printed once to stderr ([WOA], Dependency: the
 * capability probe logs once). */
mx_status mx_probe(int device);
/* Library version string. */
const char* mx_version(void);

/* Dry-run mode (1 = on): device entry points validate and return MX_OK without
 * touching HIP.  For host-only tests of argument checking. */
void mx_set_dry_run(int on);

/* Launch counters, in this order: quant, bmm (large tiles), bmm (small T),
 * dequant, linear BF16 branch (prepared weight), linear FP8 branch, linear
 * per-call-dequant branch, f32->e8m0 device, e4m3 encode device, inverse RoPE
 * to BF16, BF16 bmm (large tiles), BF16 bmm (small T), wo_a scale expansion,
 * single-kernel wo_a.
 * `out` gets min(n, MX_NUM_COUNTERS) values; returns MX_NUM_COUNTERS. */
#define MX_NUM_COUNTERS 14
int mx_get_counters(uint64_t* out, int n);
void mx_reset_counters(void);

/* ------------------------------------------------------- wo_a hot path */

/*
 * mx_inv_rope_group_quant -- fused inverse RoPE + per-token group E8M0 FP8 quant
 * ([WOA], Summary item 1; Implementation: BF16 cos/sin caches).
 *
 * x         device BF16 [T, H*D]: the attention output, head h at columns h*D.
 * positions device int64 [T]: token positions, 0 <= pos < max_pos (a position
 *           outside that range is not read: its token gets scale 0xFF and NaN
 *           codes).
 * cos, sin  device BF16 [max_pos, rope_dim/2]: cos/sin(pos * omega_i).
 * rope_dim  rotated dims at the end of each head (0 = no rotation).  Pair i of
 *           a head is (D-R+2i, D-R+2i+1) (MX_ROPE_INTERLEAVED) or
 *           (D-R+i, D-R+R/2+i) (MX_ROPE_NEOX).  The rotation is by -pos*omega_i:
 *           (x, y) -> (x*c + y*s, y*c - x*s) in fp32, each product and sum
 *           rounded, result rounded to BF16 (nearest even).
 * group     128 (wo_a) or 32 (MX block); groups are consecutive along each row.
 * fmt       mx_fp8_format of the codes.
 * q         device u8 [T, H*D]: e4m3 codes of r * 2^-e, nearest even, saturating.
 * scale     device u8 [T, H*D/group]: E8M0 bytes e+127 with e = ceil(log2(amax/M)),
 *           M = 448 (OCP) / 224 (FNUZ), clamped to [-127, 127]; 0xFF (and NaN
 *           codes) for a group holding NaN/Inf.
 * Requires: T >= 0 (0 is a no-op), H, D > 0, D % 8 == 0, rope_dim % 16 == 0,
 * rope_dim <= D, (H*D) % group == 0, x and q 16-byte aligned, cos/sin 8-byte
 * aligned (16 for NEOX), max_pos >= 1 when rope_dim > 0 and T > 0.
 */
mx_status mx_inv_rope_group_quant(const void* x, const int64_t* positions,
                                  const void* cos, const void* sin, int64_t max_pos,
                                  int64_t T, int32_t H, int32_t D, int32_t rope_dim,
                                  int32_t rope_style, int32_t group, int32_t fmt,
                                  uint8_t* q, uint8_t* scale, void* stream);

/*
 * mx_bmm_a8w8_mxscale -- batched a8w8 GEMM with E8M0 block scales
 * ([WOA], Summary item 2; Implementation: group-128 weight and scale layouts).
 *
 * out[t,g,n] = bf16( sum_k  A[t,g,k]*2^(sa[t,g,k/128]-127) * W[g,n,k]*2^(sw[g,n,k/128]-127) )
 * accumulated in fp32, rounded to BF16 (nearest even).
 *
 * a        device u8 [T, G, K]: e4m3 codes in flavour a_fmt.
 * a_scale  device u8 [T, G, K/128].
 * a_fmt    MX_FP8_E4M3_OCP or MX_FP8_E4M3_FNUZ (an FNUZ code c times 2^s equals the OCP
 *          code c times 2^(s-1), so FNUZ blocks run on the OCP MFMA with their
 *          scale byte lowered by one; FNUZ 0x80 (NaN) is not expected in A).
 *          Exception: an FNUZ block with scale byte 0 (2^-127) would need the
 *          OCP scale 2^-128, which E8M0 lacks; the byte is kept, so such a
 *          block enters the sum at twice its value.  The quantiser writes byte
 *          0 only for FNUZ groups with 0 < amax <= 224 * 2^-127.
 * w        device u8 [G, N, K]: OCP e4m3 codes (the checkpoint format).
 * w_scale  device u8 [G, N, K/128].
 * out      device BF16 [T, G, N].
 * Requires: T >= 0 (0 is a no-op), G >= 1, N >= 1 with N % 16 == 0, K >= 128
 * with K % 128 == 0, a, w and out 16-byte aligned.
 */
mx_status mx_bmm_a8w8_mxscale(const uint8_t* a, const uint8_t* a_scale, int32_t a_fmt,
                              const uint8_t* w, const uint8_t* w_scale, void* out,
                              int64_t T, int32_t G, int32_t N, int32_t K, void* stream);

/*
 * mx_wo_a_fused -- the whole FP8 wo_a step in one kernel: inverse RoPE,
 * per-token group-128 E8M0 FP8 quantisation and the batched a8w8 MX-scale
 * GEMM, the quantised activation never leaving the compute unit ([WOA],
 * Summary: an inverse RoPE fused with per-token E8M0 group quantisation,
 * then the MX batched GEMM with the checkpoint's FP8 weight; here the two are
 * one pass).
 *
 * out = mx_bmm_a8w8_mxscale(q, scale, OCP, w, w_scale) with (q, scale) =
 * mx_inv_rope_group_quant(x, ..., group 128, OCP) -- the same codes and
 * scales, so the same values as the two calls (up to the order of the fp32
 * sums).  A token whose position is outside [0, max_pos) has NaN outputs.
 * x, positions, cos, sin, max_pos, T, H, D, rope_dim, rope_style: as for
 *           mx_inv_rope_group_quant; the token row [H*D] is read as [G, K]
 *           with K = H*D/G.
 * w        device u8 [G, N, K] OCP e4m3.   w_scale device u8 [G, N, K/128].
 * out      device BF16 [T, G, N].
 * Requires: T >= 0 (0 is a no-op), G >= 1, H*D % G == 0, K % 128 == 0,
 * K <= 4096, D % 128 == 0, rope_dim % 16 == 0 and rope_dim <= min(D, 64)
 * (split halves: rope_dim in {16, 32, 64}), N >= 1 with N % 16 == 0,
 * x, w, out, cos and sin 16-byte aligned, positions 8-byte aligned,
 * max_pos >= 1 when rope_dim > 0.  Other shapes, and tables of 2 GiB or
 * more (max_pos * rope_dim >= 2^31 bytes each), return MX_ERR_UNSUPPORTED
 * (the two calls serve them).
 */
mx_status mx_wo_a_fused(const void* x, const int64_t* positions, const void* cos,
                        const void* sin, int64_t max_pos, int64_t T, int32_t H, int32_t D,
                        int32_t rope_dim, int32_t rope_style, const uint8_t* w,
                        const uint8_t* w_scale, void* out, int32_t G, int32_t N, void* stream);

/*
 * mx_woa_expand_scales -- checkpoint weight scales of wo_a -> the layout the
 * GEMM reads, at load time ([WOA], Implementation: the group-128 weight and
 * scale layouts are validated before the fast path is used; power-of-two FP32
 * scales become E8M0 bytes without loss).
 *
 * out[g,n,kb] = E8M0 of scale[g, n / block_n, kb].
 * scale        device [G, ceil(N/block_n), K/128] of E8M0 bytes (MX_SCALE_E8M0) or
 *              FP32 (MX_SCALE_F32): block_n = 1 is one scale per (g, n, 128-K
 *              block), block_n = 128 one per 128 x 128 (n, k) block.
 * out          device u8 [G, N, K/128], the w_scale of mx_bmm_a8w8_mxscale.
 * reject_count device int32, caller-zeroed, or NULL: FP32 scales that are not
 *              2^n with -127 <= n <= 127 give 0xFF (NaN) bytes and are counted,
 *              once per source scale.  A nonzero count means the checkpoint
 *              cannot take the FP8 path (the caller falls back).  Asynchronous.
 * Requires: G, N >= 1, K % 128 == 0, G*N*K/128 < 2^31, FP32 scales 4-byte aligned.
 */
mx_status mx_woa_expand_scales(const void* scale, int32_t scale_kind, int32_t block_n,
                               int32_t G, int32_t N, int32_t K, uint8_t* out,
                               int32_t* reject_count, void* stream);

/* ------------------------------------------------ BF16 arm of wo_a */

/*
 * mx_inv_rope_bf16 -- inverse RoPE to BF16, the first step of the BF16 wo_a
 * path that the FP8 one replaces and keeps as its fallback ([WOA], Summary
 * and Related work: an inverse RoPE, then a BF16 grouped einsum over a BF16
 * copy of the weight).
 *
 * out = x with the last rope_dim dims of every head rotated exactly as in
 * mx_inv_rope_group_quant (same pairs, same fp32 arithmetic, BF16 nearest
 * even); the other dims are copied.
 * x, positions, cos, sin, max_pos, T, H, D, rope_dim, rope_style: as for
 *           mx_inv_rope_group_quant.  A token whose position is outside
 *           [0, max_pos) gets BF16 NaN (0x7FC0) in its rotated dims.
 * out       device BF16 [T, H*D].  out == x runs in place, reading and
 *           writing only the rotated dims (rope_dim/D of the tensor); any
 *           other overlap of out and x is rejected.
 * Requires: T >= 0 (0 is a no-op), H, D > 0, D % 8 == 0, rope_dim % 16 == 0,
 * rope_dim <= D, x and out 16-byte aligned, cos/sin 16-byte aligned,
 * positions 8-byte aligned, max_pos >= 1 when rope_dim > 0 and T > 0.
 */
mx_status mx_inv_rope_bf16(const void* x, const int64_t* positions, const void* cos,
                           const void* sin, int64_t max_pos, int64_t T, int32_t H, int32_t D,
                           int32_t rope_dim, int32_t rope_style, void* out, void* stream);

/*
 * mx_bmm_bf16 -- batched BF16 GEMM, the grouped einsum of the BF16 wo_a path
 * ([WOA], Summary and Related work).
 *
 * out[t,g,n] = bf16( sum_k x[t,g,k] * W[g,n,k] ), fp32 accumulation, nearest even.
 * x    device BF16 [T, G, K] (the rotated activation viewed per group).
 * w    device BF16 [G, N, K] (e.g. the FP8 weight dequantised once with
 *      mx_dequant_mxfp8_to_bf16 over [G*N, K] rows, block 128).
 * out  device BF16 [T, G, N].
 * Requires: T >= 0 (0 is a no-op), G >= 1, N >= 1 with N % 16 == 0, K >= 128
 * with K % 128 == 0, 512*G*K < 2^32, x, w and out 16-byte aligned.
 */
mx_status mx_bmm_bf16(const void* x, const void* w, void* out, int64_t T, int32_t G,
                      int32_t N, int32_t K, void* stream);

/* ------------------------------------------------------- MXFP8 linear */

/*
 * mx_dequant_mxfp8_to_bf16 -- one-pass MXFP8 -> BF16 weight dequantisation
 * ([MXLIN], Purpose and "Why it is worth a patch": the weight is constant, so
 * convert it once at load; one pass instead of a chain of pointwise kernels).
 *
 * out[n,k] = bf16(decode_ocp(w[n,k]) * 2^(s[n,k/block]-127)), nearest even.
 * w        device u8 [N, K] OCP e4m3.   w_scale device u8 [N, K/block].
 * out      device BF16 [N, K].
 * Requires: N, K >= 0, block in {32, 128}, K % block == 0, w 16-byte aligned,
 * out 16-byte aligned.
 */
mx_status mx_dequant_mxfp8_to_bf16(const uint8_t* w, const uint8_t* w_scale, void* out,
                                   int64_t N, int64_t K, int32_t block, void* stream);

/* 1 iff a weight with this K is converted to BF16 at load (K % MX_LINEAR_K_ALIGN != 0),
 * else 0 ([MXLIN], Purpose: load keys off K % 128). */
int mx_linear_dequant_at_load(int64_t K);

/* Workspace bytes mx_linear needs for this call shape and weight element size
 * (1 = FP8 weight, 2 = BF16 weight): FP8 with K % 128 != 0 (per-call dequant)
 * needs N*K*2; FP8 with K % 128 == 0 needs M*K + M*K/32 (x in MXFP8); BF16 needs 0. */
size_t mx_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t w_elem_bytes);

/*
 * mx_linear -- out = x @ W^T for an MXFP8 weight, dispatched per call on the
 * weight's element size, as in [MXLIN] (Purpose; review thread):
 *   w_elem_bytes == 2: W is BF16 [N,K] (dequantised at load) -> BF16 MFMA GEMM.
 *   w_elem_bytes == 1 and K % 128 == 0: x is quantised to MXFP8 (OCP, block 32,
 *        the quantiser's rule) into the workspace, then the block-scaled FP8
 *        MFMA GEMM with w_scale [N, K/32].
 *   w_elem_bytes == 1 and K % 128 != 0: the weight was not prepared; it is
 *        dequantised into the workspace on this call and the BF16 GEMM runs on
 *        it.  An unaligned FP8 weight never reaches the scaled GEMM.
 * x        device BF16 [M, K].      w  device FP8 [N, K] or BF16 [N, K].
 * w_scale  device u8 [N, K/32] (FP8 weight; ignored for BF16).
 * out      device BF16 [M, N], fp32 accumulation, nearest-even rounding.
 * workspace device, at least mx_linear_workspace_bytes(M, N, K, w_elem_bytes),
 *          16-byte aligned (may be NULL when that is 0).
 * Requires: M, N >= 0, K > 0, K % 32 == 0, N % 16 == 0, x/w 16-byte aligned,
 * out 8-byte aligned; M <= 2^30, N and K < 2^31, M*K, N*K and M*N < 2^40.
 * Any M: up to 64 rows (a decode batch) run on kernels that keep the weight
 * streaming, more rows (a prefill chunk) on tiles with operand reuse (256 x 256
 * block-scaled FP8 tiles; 128 x 256 or 128 x 128 BF16 tiles).
 */
mx_status mx_linear(const void* x, int64_t M, int64_t K, const void* w,
                    const uint8_t* w_scale, int32_t w_elem_bytes, int64_t N, void* out,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Scratch held by the library for mx_linear_noalloc: one copy per GPU the
 * library runs on, kept until the process ends. */
#define MX_LINEAR_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * mx_linear_noalloc -- mx_linear for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, branches, kernels and results as
 * mx_linear, without the workspace: the branches that need one (the MXFP8
 * copy of x on the block-scaled branch, the per-call BF16 weight of an
 * unprepared unaligned FP8 weight) use a scratch array inside the library,
 * MX_LINEAR_NOALLOC_SCRATCH_BYTES per GPU, whose device address is looked up
 * on the first call on each device.  The call allocates nothing (no hipMalloc,
 * no allocating library routine).
 * Returns MX_ERR_INVALID_ARG if mx_linear_workspace_bytes(M, N, K,
 * w_elem_bytes) exceeds the scratch size; otherwise as mx_linear.
 * The scratch is shared by every call on one GPU and keeps the last call's
 * contents (each call writes all it reads before reading it, so nothing needs
 * clearing): calls that overlap on one GPU -- on different streams, or from
 * different threads -- race on it and must be serialised by the caller.
 */
mx_status mx_linear_noalloc(const void* x, int64_t M, int64_t K, const void* w,
                            const uint8_t* w_scale, int32_t w_elem_bytes, int64_t N, void* out,
                            void* stream);

/* ---------------------------------------------------- format converters */

/*
 * FP32 power-of-two scales -> E8M0 bytes, losslessly ([WOA], Implementation;
 * [FNUZ], Purpose: the conversion uses no FP8 arithmetic).  A value converts iff
 * it is exactly 2^n, -127 <= n <= 127 (2^-127 is an FP32 subnormal); byte n+127.
 * Host: in/out host [n]; returns MX_ERR_NOT_LOSSLESS if any input does not
 * convert (its byte is 0xFF, the others are still written).
 * Device: in/out device [n]; rejected inputs get 0xFF and, when `reject_count`
 * (device int32, caller-zeroed) is not NULL, are counted into it.  Asynchronous.
 */
mx_status mx_f32_pow2_to_e8m0(const float* in, uint8_t* out, int64_t n);
mx_status mx_f32_pow2_to_e8m0_device(const float* in, uint8_t* out, int64_t n,
                                     int32_t* reject_count, void* stream);

/*
 * FP32 -> e4m3 bytes: nearest, ties to the even code, saturating at +-448 (OCP)
 * or +-224 (FNUZ) -- Inf included; NaN -> 0x7F (OCP) / 0x80 (FNUZ); OCP keeps
 * the sign of zero, FNUZ has no -0 ([FNUZ], Purpose).  Host and device variants.
 */
mx_status mx_f32_to_e4m3_ocp(const float* in, uint8_t* out, int64_t n);
mx_status mx_f32_to_e4m3_fnuz(const float* in, uint8_t* out, int64_t n);
mx_status mx_f32_to_e4m3_device(const float* in, uint8_t* out, int64_t n, int32_t fmt,
                                void* stream);

/* e4m3 / E8M0 bytes -> FP32 (host).  Exact; NaN codes give NaN.  The byte
 * meanings are those the encoders above produce: e4m3 in the OCP or FNUZ
 * encoding picked by `fmt` ([FNUZ], Purpose: gfx950 stores OCP bytes, gfx942
 * FNUZ bytes with largest finite 224, and its reference checks decode a byte
 * under the encoding the kernel wrote it in), E8M0 a biased power-of-two
 * exponent, 2^(byte - 127), 0xFF NaN ([WOA], Implementation: the scales are
 * biased E8M0 exponent bytes). */
mx_status mx_e4m3_to_f32(const uint8_t* in, float* out, int64_t n, int32_t fmt);
mx_status mx_e8m0_to_f32(const uint8_t* in, float* out, int64_t n);

/* ------------------------------------------------------------- measurement */

/*
 * Reads `bytes` (a multiple of 16) at device address `src` once and discards
 * them: the HBM floor that the weight-streaming calls (the decode-batch GEMM,
 * the MXFP8 linear at decode M) are timed against on the same buffers.  No
 * step of the FP8 path.  `sink` is a device uint32 that is written only when
 * the XOR of a lane's words hits one fixed value (so that the loads cannot be
 * dropped); its content means nothing.  src 16-byte aligned, sink 4-byte
 * aligned.  Asynchronous on `stream`.
 */
mx_status mx_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MXFP8_H */
