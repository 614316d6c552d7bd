/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 / W4A8 group-quantized linear layer.
 *
 * The operation (W4A16):  Y[M,N] = X[M,K] . dequant(W)^T, with fp16 X and Y and
 * 4-bit weights.  "Some fixes for AWQ" (neuralmagic/compressed-tensors PR 269), reply
 * defining W4A16: fp16 input vectors multiplied by int4-quantized weights give fp16
 * output vectors, with no activation-quantization argument.  Weights are quantized
 * asymmetrically per (output row n, group of G consecutive k) as in the opening
 * comment of that page (AutoAWQ's pseudo-quantize rule):
 *     s = fp16(max(fp32(max - min) / 15, 1e-5)),  z = clamp(rint(-min / s), 0, 15),
 *     q = clamp(rint(w / s) + z, 0, 15),  dequant(w) = (q - z) * s.
 * Per-channel weights (group_size -1) form one group over K per row (a reading of the
 * per-channel variant named on the lmdeploy QQQ page below).  Symmetric weights
 * (awq_pack_sym; the W4A16 preset named beside W4A16_ASYM on the compressed-tensors
 * page, read with the W4A8 per-channel constants) use s = fp16(max(max|w| / 7, 1e-5)),
 * q = clamp(rint(w / s), -8, 7), stored as the code q + 8 with zero point 8, so every
 * W4A16 entry point below serves them unchanged.
 *
 * The W4A8 stage ("[Feature] support qqq(w4a8) for lmdeploy", InternLM/lmdeploy issue
 * 2274, section "Modification"): per-token int8 activations produced by an online
 * quantization fused with RMSNorm, an int8 x int4 GEMM accumulating in int32, and an
 * epilogue that rescales by the activation and weight scales ("Some fixes for AWQ",
 * reply on 8-bit matmuls whose int32 output is rescaled by both scales).
 *
 * Memory layouts (row-major, contiguous; all pointers are DEVICE pointers owned by the
 * caller; the library never allocates, frees, synchronizes or changes the current
 * device; it only enqueues kernels on `stream`):
 *   X        fp16  [M, K]
 *   Y        fp16  [M, N]
 *   W        fp16  [N, K]            (out, in)
 *   qweight  int32 [ceil(N/16), K/128, 4, 16, 4]
 *                                    codes packed 8 per word along K, each word split by
 *                                    parity: element k = 8j+i of row n in nibble
 *                                    i/2 + 4(i%2) of that row's word j (the even i in the
 *                                    low half-word, the odd i in the high one, each half in
 *                                    element order: nibbles hold i = 0,2,4,6,1,3,5,7),
 *                                    words stored tiled: word j of row n sits at
 *                                    [n/16][j/16][(j%16)/4][n%16][j%4], i.e. 1 KB blocks of
 *                                    16 rows x 128 k; rows past N are padding (code 0)
 *   scales   fp16  [K/G, N]          per-group scales, group-major ([1, N] per-channel)
 *   qzeros   int32 [K/G, ceil(N/8)]  4-bit zero points packed along N, plain nibble
 *                                    order, pad nibbles 0 ([1, ceil(N/8)] per-channel)
 *   (W4A8)   qweight int32 [ceil(N/16), K/128, 4, 16, 4] (same tiling) of biased nibbles
 *            q + 8, each word split by halves (element 8j+i in nibble 2(i%4) + i/4 of
 *            word j: elements 0..3 in the even nibbles, 4..7 in the odd ones; q in
 *            [-8, 7]; padding rows q = 0),
 *            cscale fp16 [N] per-channel scale, gscale int8 [K/G, N] group scales
 *            (two-level variant only), xq int8 [M, K], s_a fp32 [M].
 *   (W8A8)   qweight int8 [ceil(N/16), K/128, 4, 2, 16, 16]: code (n, k) at
 *            [n/16][k/128][kc%4][kc/4][n%16][k%16] with kc = (k%128)/16 (2 KB per 16 rows
 *            x 128 k; padding rows 0), cscale fp16 [N].
 *
 * Sizes: M >= 0, N >= 0 (M == 0 or N == 0 is a no-op returning W4_OK), K a positive
 * multiple of 128.  group_size: 128, 64, 32 or -1 (per-channel) for W4A16 (the group
 * size is a parameter of the Triton AWQ format on the vLLM page: scales (K // group_size,
 * N)); 128 or -1 for W4A8; -1 for W8A8.  Every pointer must be 16-byte aligned and non-NULL unless stated otherwise.
 *
 * `stream` is a hipStream_t (NULL = the null stream).  All entry points are
 * asynchronous: they return after validation and launch; a fault inside a kernel
 * surfaces at the caller's next synchronization.  Argument checks happen before any
 * HIP call, so an invalid call returns without touching the device.
 *
 * Return value: one of the W4_* codes below; w4_last_error() gives a thread-local
 * message for the last failure on the calling thread.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  W4_OK = 0,
  W4_ERR_INVALID_ARG = 1,   /* NULL pointer, negative size, K not a multiple of G, misalignment */
  W4_ERR_UNSUPPORTED = 2,   /* group size or shape not implemented */
  W4_ERR_WORKSPACE = 3,     /* workspace missing or smaller than *_workspace_bytes() */
  W4_ERR_DEVICE = 4,        /* current device is not gfx950 */
  W4_ERR_HIP = 5            /* a HIP runtime call failed (see w4_last_error) */
};

/*
 * awq_pack -- quantize fp16 weights W [N, K] with the asymmetric group rule above and
 * write qweight, scales and qzeros.  Quantization decisions are taken in fp32 (IEEE
 * division, round-half-to-even), so the output is bit-exact and deterministic.
 * M is unused (accepted for a uniform signature; must be >= 0).  group_size -1 runs a
 * per-row statistics kernel first (two launches on `stream`).
 */
int awq_pack(const void* w, int32_t* qweight, void* scales, int32_t* qzeros,
             int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/*
 * awq_pack_sym -- as awq_pack with the symmetric rule: s = fp16(max(max|w| / 7, 1e-5))
 * per (row, group), code q + 8 with q = clamp(rint(w / s), -8, 7), every zero point 8
 * (the nibble of every real row is 8).  Same layouts, arguments and errors.
 */
int awq_pack_sym(const void* w, int32_t* qweight, void* scales, int32_t* qzeros,
                 int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/*
 * awq_unpack_dequant -- write fp16 W_deq [N, K] = fp16((q - z) * s) with exactly one
 * rounding per element (the dequantization step of the large-M GEMM).  Debug/export
 * path; bit-exact.
 */
int awq_unpack_dequant(const int32_t* qweight, const void* scales, const int32_t* qzeros,
                       void* w_out, int64_t N, int64_t K, int32_t group_size, void* stream);

/*
 * Plain (untiled) weight layouts accepted by the import calls below.  "Implement AWQ
 * quantization support for LLaMA" (vllm-project/vllm PR 1032) prints the Triton AWQ
 * weight format: codes packed 8 per 32-bit word along K (plain nibble order: element
 * k = 8j + i of a row in bits 4i..4i+3 of word j), per-group scales, and per-group zero
 * points packed 8 per word along the group axis (group g in bits 4 (g % 8).. of word
 * g / 8), stored K-major.  With ng = K / G (1 per-channel):
 *   W4_LAYOUT_ROWS  per output channel: qweight int32 [N, K/8], scales fp16 [N, ng],
 *                   qzeros int32 [N, ceil(ng/8)]; W4A8 gscale int8 [N, ng]
 *   W4_LAYOUT_COLS  the printed (K-major) orientation: qweight int32 [K/8, N], scales
 *                   fp16 [ng, N], qzeros int32 [ceil(ng/8), N]; W4A8 gscale int8 [ng, N]
 */
enum { W4_LAYOUT_ROWS = 0, W4_LAYOUT_COLS = 1 };

/*
 * awq_import_plain -- convert W4A16 weights quantized elsewhere from a plain layout
 * (see W4_LAYOUT_*) into the layout awq_gemm reads (parity-split words tiled into
 * qweight, scales [K/G, N], qzeros [K/G, ceil(N/8)], top of this file).  A pure
 * rearrangement of bits: the
 * outputs equal what awq_pack writes for the same codes, scales and zero points
 * (padding rows of qweight are code 0).  All six pointers are device pointers owned by
 * the caller, 16-byte aligned, non-NULL for N > 0; inputs and outputs must not overlap.
 * group_size 128, 64, 32 or -1; K a positive multiple of 128; N == 0 is a no-op.
 * Asynchronous on `stream` (a few small kernels).
 */
int awq_import_plain(const int32_t* qweight_plain, const void* scales_plain, const int32_t* qzeros_plain,
                     int32_t* qweight, void* scales, int32_t* qzeros, int64_t N, int64_t K, int32_t group_size,
                     int32_t layout, void* stream);

/*
 * w4a8_import_plain -- as awq_import_plain for W4A8 weights: qweight_plain holds biased
 * nibbles q + 8 ("[Feature] support qqq(w4a8) for lmdeploy", "Modification": exported
 * QQQ weights are converted to the serving format before the GEMM loads them) in the
 * plain nibble order; each word is split by halves on the way (the W4A8 qweight layout,
 * top of this file), and the tiled output's padding rows hold q = 0 (nibble 8).  group_size 128 (two-level: gscale_plain
 * int8 in the orientation of `layout` -> gscale [K/G, N]) or -1 (per-channel:
 * gscale_plain and gscale must be NULL).  cscale [N] is the same in every layout and is
 * not an argument.
 */
int w4a8_import_plain(const int32_t* qweight_plain, const int8_t* gscale_plain, int32_t* qweight, int8_t* gscale,
                      int64_t N, int64_t K, int32_t group_size, int32_t layout, void* stream);

/*
 * awq_gemm_workspace_bytes -- bytes of workspace awq_gemm needs for this shape (0 when
 * the chosen kernels do not split K).  The workspace holds split-K fp32 partial sums and
 * per-tile arrival counters.  It must be zero-filled before its first use; every
 * completed call leaves the counter region zeroed again, so a workspace can be reused
 * by later calls on the same stream.  Calls that overlap in time (different streams)
 * must not share a workspace.
 */
size_t awq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group_size);

/*
 * awq_gemm -- Y [M, N] = X [M, K] . dequant(qweight, scales, qzeros)^T, fp32 accumulate,
 * fp16 output (round to nearest even).  Dispatch: M <= 32 uses a bandwidth-bound skinny
 * kernel (16x16x32 fp16 MFMA on exact fp16 encodings of the codes, per-group scaling in
 * fp32; X staged in LDS at M = 1 on wide matrices with K <= 8192); larger M uses the
 * LDS-staged 32x32x16 fp16 MFMA GEMM with in-register dequantization.  Group sizes 64
 * and 32 take a dequantizing variant of the skinny kernel at M <= 32 (each lane scales
 * its own 32 k) and the MFMA GEMM above.  Results are deterministic (split-K partials
 * are summed in a fixed order).
 * The packed operands are in this library's layout (top of this file), not the
 * row-major qweight [N, K/8], scales [N, K/G], qzeros [N, ceil(K/G/8)] of a plain
 * export: with row-major words every wave load of the decode kernels touched 16
 * separate 64-byte pieces and ran ~40 % slower than the 1 KB tiles, and the
 * parity-split words expand to fp16 in five VALU operations with X in its natural
 * order (plain words take eight, or five plus a permutation of X).  Weights in a plain
 * layout come in once through awq_import_plain.
 */
int awq_gemm(const void* x, const int32_t* qweight, const void* scales, const int32_t* qzeros,
             void* y, void* workspace, size_t workspace_bytes,
             int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/*
 * awq_gemm_noalloc -- awq_gemm for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels and results as awq_gemm; the split-K workspace is a static device array
 * of W4_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until the process
 * ends, so the call makes no hipMalloc, hipFree or other allocating call.  The caller
 * passes inputs and outputs as for awq_gemm.  A shape whose workspace
 * (awq_gemm_workspace_bytes) exceeds the array returns W4_ERR_WORKSPACE before any
 * launch.  All calls on one GPU share the array and it keeps the last call's contents:
 * calls in stream order are safe, calls that overlap in time on one GPU (different
 * streams) race.  The first call on a device resolves the array's address and enqueues
 * one small kernel on `stream` that clears its counter region.
 */
#define W4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int awq_gemm_noalloc(const void* x, const int32_t* qweight, const void* scales, const int32_t* qzeros, void* y,
                     int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/*
 * w4a8_pack -- quantize fp16 W [N, K] to symmetric int4 for W4A8 and pack it.
 * group_size == -1: per-channel, cscale = fp16(max(max|w|/7, 1e-5)),
 *   q = clamp(rint(w / cscale), -8, 7); gscale must be NULL.
 * group_size == 128: two-level, cscale = fp16(max(max|w|/127, 1e-5)),
 *   w8 = clamp(rint(w / cscale), -127, 127), per group s_g = min(max(1, ceil(max|w8|/7)), 18),
 *   q = clamp(rint(w8 / s_g), -7, 7); gscale int8 [K/G, N] receives s_g.
 * qweight receives q + 8 (plain nibble order, tiled word layout above).  fp32 decisions;
 * bit-exact.
 */
int w4a8_pack(const void* w, int32_t* qweight, int8_t* gscale, void* cscale,
              int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/*
 * w4a8_quant_act -- per-token symmetric int8 quantization, optionally fused with RMSNorm
 * ("[Feature] support qqq(w4a8) for lmdeploy", "Modification": online quantization fused
 * with RMSNorm).  With gamma != NULL: y = x / sqrt(mean_k(x^2) + eps) * gamma (fp32, no
 * fp16 round trip); with gamma == NULL: y = x.  Then amax = max|y|,
 * xq = clamp(rint(y * fp32(127 / amax)), -127, 127), s_a = amax / 127; a zero row gives
 * xq = 0, s_a = 1.  N and group_size are unused (must be >= 0 / any value).
 */
int w4a8_quant_act(const void* x, const void* gamma, float eps, int8_t* xq, float* s_a,
                   int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/*
 * w4a8_silu_mul_quant -- the SiLU-gated input of the down projection, quantized per token
 * ("[Feature] support qqq(w4a8) for lmdeploy", "Modification": online quantization fused
 * with element-wise operations such as SiLU; gate and up weights fused into one weight).
 * gate_up: fp16 [M, 2K] row-major, the fused gate+up projection output, gate in columns
 * 0..K-1 and up in K..2K-1.  y = silu(gate) * up with silu(g) = g / (1 + exp(-g)), in
 * fp32 with no fp16 round trip; then the rule of w4a8_quant_act on y: xq int8 [M, K],
 * s_a fp32 [M]; a row gives xq = 0, s_a = 1 only where the rule has no value: max|y| = 0,
 * or fp32(127 / max|y|) not finite (max|y| below about 2^-121).  Tiny rows are kept
 * (y is formed scaled by 2^64 inside the kernel), so s_a may be an fp32 subnormal.
 * K must be a positive multiple of 8 (at most 2^29); N and group_size are unused.  The
 * caller owns every buffer; all pointers are device pointers, 16-byte aligned; the call
 * is asynchronous on `stream`.  y carries about 9 units of fp32 rounding (exp and the
 * reciprocal are the 1-ulp hardware approximations), so codes equal those of the exact
 * y except where y * 127 / max|y| lies within 2e-4 of a half-integer (a difference of 1
 * there).
 */
int w4a8_silu_mul_quant(const void* gate_up, int8_t* xq, float* s_a,
                        int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/*
 * w8a8_pack -- per-channel symmetric int8 weights for W8A8 (an 8-bit-weight method built
 * with SmoothQuant is reported on "Implement AWQ quantization support for LLaMA",
 * vllm-project/vllm PR 1032; "Some fixes for AWQ" names W8A8 as 8-bit weights and
 * activations; the constants are a reading, those of the first level of the two-level
 * W4A8 rule): cscale fp16 [N] = fp16(max(max|w| / 127, 1e-5)),
 * qweight (tiled int8 above) = clamp(rint(w / cscale), -127, 127).  fp32 decisions,
 * bit-exact.  group_size must be -1; M is unused (>= 0).  SmoothQuant's calibrated
 * smoothing is an offline rescaling of W and X that the caller applies beforehand.
 */
int w8a8_pack(const void* w, int8_t* qweight, void* cscale,
              int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/* w8a8_gemm_workspace_bytes -- as awq_gemm_workspace_bytes, for w8a8_gemm / _i32. */
size_t w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group_size);

/*
 * w8a8_gemm -- Y [M, N] = fp16(acc[m, n] * s_a[m] * cscale[n]) with
 * acc[m, n] = sum_k xq[m, k] * qweight[n, k] exact in int32, on the int8 MFMA kernels of
 * w4a8_gemm (M <= 16: 16x16x64; larger M: LDS-staged 32x32x32), the weights loaded as
 * they are.  xq, s_a from w4a8_quant_act or w4a8_silu_mul_quant.  group_size must be -1.
 * K a positive multiple of 128, at most 131072 (as for w4a8_gemm).
 */
int w8a8_gemm(const int8_t* xq, const float* s_a, const int8_t* qweight, const void* cscale, void* y,
              void* workspace, size_t workspace_bytes,
              int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/* w8a8_gemm_i32 -- the raw int32 accumulators acc [M, N] of w8a8_gemm.  Bit-exact. */
int w8a8_gemm_i32(const int8_t* xq, const int8_t* qweight, int32_t* acc, void* workspace, size_t workspace_bytes,
                  int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/* w4a8_gemm_workspace_bytes -- as awq_gemm_workspace_bytes, for w4a8_gemm / _i32. */
size_t w4a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group_size);

/*
 * w4a8_gemm -- Y [M, N] = fp16(acc[m, n] * s_a[m] * cscale[n]) where
 * acc[m, n] = sum_k xq[m, k] * q[n, k] * s_g[n, k / G] (s_g = 1 for group_size == -1) is
 * computed exactly in int32 on the int8 MFMA units (M <= 16: bandwidth-bound kernel on
 * 16x16x64 int8 MFMA; larger M: LDS-staged 32x32x32 int8 MFMA GEMM).  gscale is NULL iff
 * group_size == -1.  K is at most 131072 (2^17), which keeps every int32 partial sum
 * in range (127 * 128 per term); larger K returns W4_ERR_UNSUPPORTED.
 */
int w4a8_gemm(const int8_t* xq, const float* s_a, const int32_t* qweight, const int8_t* gscale,
              const void* cscale, void* y, void* workspace, size_t workspace_bytes,
              int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/*
 * w4a8_gemm_i32 -- the raw int32 accumulators acc [M, N] of w4a8_gemm (no rescaling).
 * Bit-exact; for verification of the integer pipeline.
 */
int w4a8_gemm_i32(const int8_t* xq, const int32_t* qweight, const int8_t* gscale, int32_t* acc,
                  void* workspace, size_t workspace_bytes,
                  int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream);

/*
 * w4_pack_codes -- pack 4-bit codes [R, C] (uint8, one code per byte, values 0..15; only the
 * low 4 bits of each byte are used) into int32 [R, ceil(C / 8)], row-major, plain nibble
 * order: element 8j + i of a row goes to bits 4i..4i+3 of word j, missing trailing
 * elements are 0.  The packing rule the pages fix for the AWQ weight format ("Implement
 * AWQ quantization support for LLaMA", vllm-project/vllm PR 1032: pack_num = 8 codes per
 * 32-bit word), without the tiling of qweight; for exporting codes or zero points in the
 * plain layout.  R, C >= 0 (R == 0 or C == 0 is a no-op); codes needs no alignment, out must
 * be 16-byte aligned.  Bit-exact.
 */
int w4_pack_codes(const uint8_t* codes, int32_t* out, int64_t R, int64_t C, void* stream);

/*
 * Measurement helpers: the measured ceilings that the GEMMs are reported against, next
 * to the specification figures (the pages' point is speed: "[Feature] support qqq(w4a8)
 * for lmdeploy", "Throughput").  Neither computes anything of the method.
 *
 * w4_ceiling_read -- read every byte of buf[0, bytes) once from device memory (16-byte
 * non-temporal vector loads, grid-stride over `blocks` workgroups of 256 threads, `unroll`
 * (4 or 8) loads in flight per thread) and store one xor-fold word per wave to sink (blocks * 4
 * uint32, device).  bytes a positive multiple of 16; 1 <= blocks <= 65536.
 *
 * w4_ceiling_mfma -- `blocks` workgroups of 4 waves, each wave running `iters` rounds of
 * 4 independent accumulator chains of v_mfma_f32_32x32x16_f16 (kind 0; 32768 flops per
 * instruction) or v_mfma_i32_32x32x32_i8 (kind 1; 65536 ops) with no memory traffic in
 * the loop.  A and B operands are 16-byte chunks of `operands` (device, operand_bytes a
 * positive multiple of 16; constant or random contents select the data the matrix cores
 * see); out receives one float per thread (blocks * 256, device).  Work per call:
 * blocks * 4 * iters * 4 instructions.
 */
int w4_ceiling_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks, int32_t unroll, void* stream);
int w4_ceiling_mfma(const void* operands, int64_t operand_bytes, int32_t kind, int32_t iters, float* out,
                    int32_t blocks, void* stream);

/* Human-readable name of a status code (static storage). */
const char* w4_status_string(int status);
/* Message for the last failure on the calling thread ("" if none). */
const char* w4_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_H */
