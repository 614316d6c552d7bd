"""Plain CPU oracle (numpy) for the W4A16 / W4A8 group-quantized linear layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` and by nothing else.  It shares no
code, header, table or constant generator with the GPU library.

Sources (web pages; cited by title and the part of the page):

* [AWQ-vLLM]  "Implement AWQ quantization support for LLaMA" (vllm-project/vllm
  PR 1032): the comment thread on the AWQ GEMM kernel, including the remark
  that dequantization is the tricky part and the rest is plain FP16 work, and
  the comment listing the Triton AWQ weight format (activations (M, K), packed
  weights along K with ``pack_num`` codes per word, per-group scales and
  zeros).
* [QQQ-lmdeploy]  "[Feature] support qqq(w4a8) for lmdeploy" (InternLM/lmdeploy
  issue 2274), section "Modification": a W4A8 GEMM, online (per-token)
  activation quantization fused with RMSNorm, fused gate+up weights; section
  "Benchmark": per-channel and g128 variants.
* [AWQ-fixes]  "Some fixes for AWQ" (neuralmagic/compressed-tensors PR 269):
  the opening comment (asymmetric quantization aligned with AutoAWQ's
  pseudo-quantize rule), the reply defining W4A16 (fp16 in, int4 weights,
  fp16 out, no activation quantization arguments) and the reply on 8-bit
  matmuls that output int32 and are rescaled by weight and activation scales,
  with activations quantized dynamically.

Readings where the pages are silent:

* R1 asymmetric rule: per (row n, group g) ``s = (max - min) / 15`` computed in
  fp32 (IEEE division), floored at 1e-5, stored as fp16 (RNE);
  ``z = clamp(rint(-min / s16), 0, 15)``; ``q = clamp(rint(w / s16) + z, 0, 15)``
  with the stored fp16 scale, in fp32.  Quantized codes are integers decided
  in fp32, the precision the GPU kernel uses.
* R2 rounding is round-half-to-even everywhere (``np.rint``).
* R3 dequantization is ``(q - z) * s16`` (exact in fp64; a single fp16
  rounding when exported as fp16).
* R4 packing is the plain nibble order: element ``8*j + i`` of a packed axis
  lives in bits ``4*i .. 4*i+3`` of word ``j``; pad nibbles are 0.
  Layouts: the codes of row n form words ``j = 0 .. K/8-1`` (packed along K);
  the W4A16 ``qweight`` holds each word with its codes split by parity (the even
  elements ``i = 0, 2, 4, 6`` in nibbles 0..3, the odd ones ``i = 1, 3, 5, 7``
  in nibbles 4..7: element i at nibble ``i // 2 + 4 * (i % 2)``), and stores the
  words tiled as int32 [ceil(N/16), K/128, 4, 16, 4]:
  word j of row n sits at ``[n // 16, j // 16, (j % 16) // 4, n % 16, j % 4]``
  (one 1 KB block holds 16 rows x 128 k; rows past N are padding with code 0,
  or q = 0 for W4A8).  ``scales`` fp16 [K/G, N]; ``qzeros`` int32
  [K/G, ceil(N/8)] (zero points packed along N).
* R5b The W4A8 ``qweight`` holds each word of biased nibbles split by halves: element
  ``i`` of the word in nibble ``2 * (i % 4) + i // 4`` (elements 0..3 in the even
  nibbles, 4..7 in the odd ones), tiled as the W4A16 words; a layout choice of the
  library (its int8 expansion then needs no byte permutation).
* R5 W4A8 weights (the pages print no constants): per-channel (group -1)
  ``s_c = fp16(max(max|w| / 7, 1e-5))``, ``q = clamp(rint(w / s_c), -8, 7)``;
  two-level g128: ``s_c = fp16(max(max|w| / 127, 1e-5))``,
  ``w8 = clamp(rint(w / s_c), -127, 127)``, per group ``m = max|w8|``,
  ``s_g = min(max(1, ceil(m / 7)), 18)`` (int8), ``q = clamp(rint(w8 / s_g), -7, 7)``.
  Stored nibble is ``q + 8``.  ``|q * s_g| <= 126`` so the int4 x int8-scale
  product always fits int8.  The constants are a reading; the implementation
  is pinned by exhaustive invariants, the reading itself is "parity unpinned"
  against the pages.
* R6 W4A8 activations: RMSNorm ``y = x / sqrt(mean(x^2) + eps) * gamma`` in
  fp64 with no fp16 round-trip of ``y``; the quantization decision is taken
  in fp32 on ``y32 = fp32(y)``: ``M = max|y32|``, ``inv = fp32(127 / M)``,
  ``xq = clamp(rint(fp32(y32 * inv)), -127, 127)``, ``s_a = fp32(M / 127)``;
  a zero row gives ``s_a = 1``, ``xq = 0``.  Without gamma (no-norm mode)
  ``y32 = x``.
* R13 W4A16 per-channel ([QQQ-lmdeploy] "Benchmark" and a reply in its thread
  name per-channel quantization, group_size = -1, beside g128): group_size -1
  means one group spanning all of K; the R1 rule then applies per row; scales
  are fp16 [1, N] and zero points int32 [1, ceil(N/8)].
* R16 group sizes 64 and 32 ([AWQ-vLLM], the Triton format comment sizes scales
  as (K // group_size, N): the group size is a parameter): the R1 / R14 rules apply
  per group of any G dividing K; the GPU library takes G in {32, 64, 128, -1}.
* R14 W4A16 symmetric ([AWQ-fixes], reply on preset schemes: a W4A16_ASYM preset
  beside W4A16, which is therefore the symmetric one): per (row, group)
  ``s = fp16(max(max|w| / 7, 1e-5))``, ``q = clamp(rint(w / s), -8, 7)`` (the R5
  per-channel constants), stored as the code ``q + 8`` with zero point 8, so
  ``(code - 8) * s = q * s`` dequantizes it with the asymmetric formula.
* R15 W8A8 ([AWQ-vLLM], reply on an 8-bit-weight method built with SmoothQuant
  that raised throughput; [AWQ-fixes], replies on presets: W8A8 quantizes weights
  and activations to 8 bits): weights per output channel symmetric int8 with the
  first level of R5's two-level rule, ``s = fp16(max(max|w| / 127, 1e-5))``,
  ``q = clamp(rint(w / s), -127, 127)``; activations per token as R6; the GEMM
  accumulates ``sum_k xq q`` exactly in int32 and outputs ``acc * s_a * s``.
  Layout (a design choice, like R4): int8 [ceil(N/16), K/128, 4, 2, 16, 16], code
  (n, k) at ``[n // 16, k // 128, kc % 4, kc // 4, n % 16, k % 16]`` with
  ``kc = (k % 128) // 16``: one 2 KB block per 16 rows x 128 k whose 16-byte chunks
  of one ``kc % 4`` lie together for all 16 rows and both ``kc // 4``.
  SmoothQuant's calibrated per-input-channel smoothing is an offline rescaling of
  X and W that leaves this GEMM unchanged; it needs calibration data and is not
  part of the oracle.
* R12 SiLU-gated activations ([QQQ-lmdeploy], "Modification": online
  quantization fused with element-wise operations such as SiLU; gate and up
  weights fused into one weight): the fused gate+up output ``[M, 2I]`` holds gate
  in columns ``0..I-1`` and up in ``I..2I-1``; ``y = silu(gate) * up`` with
  ``silu(g) = g / (1 + exp(-g))``, in fp64 with no fp16 round trip, then the R6
  quantization decision on ``fp32(y)``, unchanged: a row is a zero row
  (``xq = 0``, ``s_a = 1``) only when its fp32 ``max|y|`` is 0 or when
  ``fp32(127 / max|y|)`` is not finite, i.e. ``max|y|`` below about ``2^-121``,
  where the rule itself has no value (fp32 is normal down to ``2^-126``).
"""
from __future__ import annotations

import numpy as np

F16 = np.float16
F32 = np.float32
F64 = np.float64

__all__ = [
    "pack_nibbles", "unpack_nibbles", "split_parity", "merge_parity", "split_halves", "merge_halves",
    "tile_words", "untile_words",
    "quantize_asym", "quantize_sym", "pack_awq", "unpack_awq", "dequant_awq", "awq_reference",
    "linear_ref",
    "quantize_w4a8", "pack_w4a8", "unpack_w4a8", "w4a8_quant_act_ref", "quantize_w8a8",
    "tile_w8a8", "untile_w8a8",
    "w4a8_acc_ref", "w4a8_linear_ref", "silu_ref", "silu_mul_quant_ref",
]


# --------------------------------------------------------------------------
# Packing (R4).  [AWQ-vLLM], comment on the Triton AWQ weight format: codes are
# packed ``pack_num`` = 8 per 32-bit word along one axis.
# --------------------------------------------------------------------------
def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes [R, C] (values 0..15) into int32 [R, ceil(C/8)].

    Element ``8*j + i`` of a row goes to bits ``4*i .. 4*i+3`` of word ``j``.
    Missing trailing elements are treated as code 0.
    """
    codes = np.asarray(codes)
    if codes.ndim != 2:
        raise ValueError("codes must be 2-D")
    if codes.size and (codes.min() < 0 or codes.max() > 15):
        raise ValueError("codes must lie in [0, 15]")
    R, C = codes.shape
    W = (C + 7) // 8
    padded = np.zeros((R, W * 8), dtype=np.int64)
    padded[:, :C] = codes
    words = np.zeros((R, W), dtype=np.int64)
    for i in range(8):
        words += padded[:, i::8] << (4 * i)
    return words.astype(np.uint32).view(np.int32)


def unpack_nibbles(words: np.ndarray, C: int) -> np.ndarray:
    """Inverse of :func:`pack_nibbles`: int32 [R, W] -> uint8 codes [R, C]."""
    words = np.asarray(words)
    if words.dtype != np.int32:
        raise ValueError("words must be int32")
    u = words.view(np.uint32).astype(np.int64)
    R, W = u.shape
    if C > 8 * W:
        raise ValueError("C larger than the packed capacity")
    out = np.zeros((R, 8 * W), dtype=np.uint8)
    for i in range(8):
        out[:, i::8] = (u >> (4 * i)) & 0xF
    return out[:, :C]


def split_parity(words: np.ndarray) -> np.ndarray:
    """Plain words -> the W4A16 qweight's word format (R4): element ``i`` of each word
    (plain nibble i) moves to nibble ``i // 2 + 4 * (i % 2)``, so the even elements fill
    the low half-word and the odd ones the high half-word, each half in element order."""
    words = np.asarray(words)
    if words.dtype != np.int32:
        raise ValueError("words must be int32")
    u = words.view(np.uint32).astype(np.int64)
    out = np.zeros_like(u)
    for i in range(8):
        out |= ((u >> (4 * i)) & 0xF) << (4 * (i // 2 + 4 * (i % 2)))
    return out.astype(np.uint32).view(np.int32)


def merge_parity(words: np.ndarray) -> np.ndarray:
    """Inverse of :func:`split_parity`."""
    words = np.asarray(words)
    if words.dtype != np.int32:
        raise ValueError("words must be int32")
    u = words.view(np.uint32).astype(np.int64)
    out = np.zeros_like(u)
    for i in range(8):
        out |= ((u >> (4 * (i // 2 + 4 * (i % 2)))) & 0xF) << (4 * i)
    return out.astype(np.uint32).view(np.int32)


def split_halves(words: np.ndarray) -> np.ndarray:
    """Plain words -> the W4A8 qweight's word format (R5b): element ``i`` of each word
    (plain nibble i) moves to nibble ``2 * (i % 4) + i // 4``: elements 0..3 fill the
    even nibbles and elements 4..7 the odd ones, each in element order."""
    words = np.asarray(words)
    if words.dtype != np.int32:
        raise ValueError("words must be int32")
    u = words.view(np.uint32).astype(np.int64)
    out = np.zeros_like(u)
    for i in range(8):
        out |= ((u >> (4 * i)) & 0xF) << (4 * (2 * (i % 4) + i // 4))
    return out.astype(np.uint32).view(np.int32)


def merge_halves(words: np.ndarray) -> np.ndarray:
    """Inverse of :func:`split_halves`."""
    words = np.asarray(words)
    if words.dtype != np.int32:
        raise ValueError("words must be int32")
    u = words.view(np.uint32).astype(np.int64)
    out = np.zeros_like(u)
    for i in range(8):
        out |= ((u >> (4 * (2 * (i % 4) + i // 4))) & 0xF) << (4 * i)
    return out.astype(np.uint32).view(np.int32)


def tile_words(words: np.ndarray, pad_word: int = 0) -> np.ndarray:
    """Row-major code words [N, K/8] -> the tiled qweight [ceil(N/16), K/128, 4, 16, 4]
    (R4): word j of row n goes to ``[n // 16, j // 16, (j % 16) // 4, n % 16, j % 4]``.
    Rows past N are filled with ``pad_word``."""
    words = np.asarray(words)
    if words.dtype != np.int32 or words.ndim != 2:
        raise ValueError("words must be 2-D int32")
    N, W = words.shape
    if W % 16:
        raise ValueError("K must be a multiple of 128")
    Np = -(-N // 16) * 16
    full = np.full((Np, W), np.uint32(pad_word & 0xFFFFFFFF).view(np.int32), dtype=np.int32)
    full[:N] = words
    out = np.empty((Np // 16, W // 16, 4, 16, 4), dtype=np.int32)
    for n in range(16):
        for slot in range(4):
            for w in range(4):
                out[:, :, slot, n, w] = full[n::16, slot * 4 + w::16]
    return out


def untile_words(tiled: np.ndarray, N: int) -> np.ndarray:
    """Inverse of :func:`tile_words`: tiled qweight -> row-major words [N, K/8]."""
    tiled = np.asarray(tiled)
    if tiled.dtype != np.int32 or tiled.ndim != 5 or tiled.shape[2:] != (4, 16, 4):
        raise ValueError("tiled qweight must be int32 [N/16, K/128, 4, 16, 4]")
    T, G = tiled.shape[:2]
    if N > 16 * T:
        raise ValueError("N larger than the tiled capacity")
    full = np.empty((16 * T, 16 * G), dtype=np.int32)
    for n in range(16):
        for slot in range(4):
            for w in range(4):
                full[n::16, slot * 4 + w::16] = tiled[:, :, slot, n, w]
    return full[:N]


# --------------------------------------------------------------------------
# W4A16 asymmetric quantization (R1, R2).  [AWQ-fixes], opening comment.
# --------------------------------------------------------------------------
def _groups(w16: np.ndarray, group_size: int):
    """fp16 [N, K] -> fp32 [N, K/G, G]; group_size -1 is one group over K (R13)."""
    w16 = np.asarray(w16)
    if w16.dtype != F16 or w16.ndim != 2:
        raise ValueError("w16 must be a 2-D float16 array")
    N, K = w16.shape
    G = K if int(group_size) == -1 else int(group_size)
    if G <= 0 or K % G:
        raise ValueError("K must be a multiple of group_size")
    return w16.astype(F32).reshape(N, K // G, G), N, K


def quantize_asym(w16: np.ndarray, group_size: int = 128):
    """Group-wise asymmetric uint4 quantization of fp16 weights [N, K] (R1;
    group_size -1: per row, R13).

    Returns ``(codes uint8 [N, K], scales fp16 [N, K/G], zeros uint8 [N, K/G])``
    in the natural (row, group) orientation.  All decisions in fp32.
    """
    w, N, K = _groups(w16, group_size)
    mn = w.min(axis=2)
    mx = w.max(axis=2)
    s32 = (mx - mn) / F32(15.0)
    s32 = np.maximum(s32, F32(1e-5))
    s16 = s32.astype(F16)
    s = s16.astype(F32)
    z = np.clip(np.rint(-mn / s), F32(0), F32(15))
    q = np.clip(np.rint(w / s[:, :, None]) + z[:, :, None], F32(0), F32(15))
    return (q.reshape(N, K).astype(np.uint8), s16, z.astype(np.uint8))


def quantize_sym(w16: np.ndarray, group_size: int = 128):
    """Group-wise symmetric int4 quantization for W4A16 (R14): per (row, group)
    ``s = fp16(max(max|w| / 7, 1e-5))``, ``q = clamp(rint(w / s), -8, 7)`` with the
    stored scale, in fp32.  Returns ``(codes uint8 [N, K] = q + 8, scales fp16
    [N, K/G], zeros uint8 [N, K/G] = 8)``, the orientation of :func:`quantize_asym`."""
    w, N, K = _groups(w16, group_size)
    amax = np.abs(w).max(axis=2)
    s16 = np.maximum(amax / F32(7.0), F32(1e-5)).astype(F16)
    s = s16.astype(F32)
    q = np.clip(np.rint(w / s[:, :, None]), F32(-8), F32(7))
    codes = (q + F32(8)).reshape(N, K).astype(np.uint8)
    return codes, s16, np.full(s16.shape, 8, dtype=np.uint8)


def pack_awq(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray):
    """Natural-orientation quantized weights -> the packed layout of R4.

    ``codes`` uint8 [N, K], ``scales`` fp16 [N, K/G], ``zeros`` uint8 [N, K/G]
    -> ``(qweight int32 [ceil(N/16), K/128, 4, 16, 4], scales fp16 [K/G, N],
    qzeros int32 [K/G, ceil(N/8)])``.
    """
    N, K = codes.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    qweight = tile_words(split_parity(pack_nibbles(codes)))
    scales_gn = np.ascontiguousarray(np.asarray(scales, dtype=F16).T)
    qzeros = pack_nibbles(np.ascontiguousarray(np.asarray(zeros).T))
    return qweight, scales_gn, qzeros


def unpack_awq(qweight: np.ndarray, scales_gn: np.ndarray, qzeros: np.ndarray, K: int):
    """Packed layout -> ``(codes [N, K], scales fp16 [N, K/G], zeros [N, K/G])``."""
    N = scales_gn.shape[1]
    codes = unpack_nibbles(merge_parity(untile_words(qweight, N)), K)
    scales = np.ascontiguousarray(scales_gn.T)
    zeros = np.ascontiguousarray(unpack_nibbles(qzeros, N).T)
    return codes, scales, zeros


def dequant_awq(qweight, scales_gn, qzeros, K: int, group_size: int = 128) -> np.ndarray:
    """Dequantized weights ``(q - z) * s`` in fp64, [N, K] (R3).

    [AWQ-vLLM], comment that dequantization is the tricky part; the product of
    a small integer and an fp16 scale is exact in fp64.
    """
    codes, scales, zeros = unpack_awq(qweight, scales_gn, qzeros, K)
    G = K if int(group_size) == -1 else int(group_size)
    N = codes.shape[0]  # the number of real rows (scales_gn.shape[1])
    s = np.repeat(scales.astype(F64), G, axis=1)
    z = np.repeat(zeros.astype(F64), G, axis=1)
    assert s.shape == (N, K)
    return (codes.astype(F64) - z) * s


def linear_ref(x16: np.ndarray, w_deq: np.ndarray) -> np.ndarray:
    """``Y = X @ w_deq^T`` in fp64 ([AWQ-fixes], reply defining W4A16: fp16
    inputs multiplied by int4-quantized weights give fp16 outputs)."""
    return np.asarray(x16, dtype=F64) @ np.asarray(w_deq, dtype=F64).T


def awq_reference(w16: np.ndarray, x16: np.ndarray, group_size: int = 128, symmetric: bool = False):
    """The whole W4A16 chain: quantize (R1, or R14 when symmetric) -> pack -> unpack
    -> dequant -> fp64 matmul.

    Returns a dict with the packed tensors, the fp64 dequantized weights and
    the fp64 outputs.
    """
    codes, scales, zeros = (quantize_sym if symmetric else quantize_asym)(w16, group_size)
    qweight, scales_gn, qzeros = pack_awq(codes, scales, zeros)
    w_deq = dequant_awq(qweight, scales_gn, qzeros, w16.shape[1], group_size)
    y = linear_ref(x16, w_deq) if x16 is not None else None
    return dict(qweight=qweight, scales=scales_gn, qzeros=qzeros, w_deq=w_deq, y=y)


# --------------------------------------------------------------------------
# W4A8 (R5, R6).  [QQQ-lmdeploy] "Modification" and "Benchmark";
# [AWQ-fixes] reply on int32 matmul output rescaled by both scales.
# --------------------------------------------------------------------------
def quantize_w4a8(w16: np.ndarray, group_size: int = -1):
    """Symmetric int4 weights for W4A8 (R5).

    ``group_size == -1``: per-channel, returns ``(q int8 [N,K] in [-8,7],
    cscale fp16 [N], None)``.  ``group_size == G > 0``: two-level, returns
    ``(q int8 [N,K] in [-7,7], cscale fp16 [N], gscale int8 [N, K/G])``.
    Decisions in fp32.
    """
    w16 = np.asarray(w16)
    if w16.dtype != F16 or w16.ndim != 2:
        raise ValueError("w16 must be a 2-D float16 array")
    N, K = w16.shape
    w = w16.astype(F32)
    amax = np.abs(w).max(axis=1)
    if group_size == -1:
        s32 = np.maximum(amax / F32(7.0), F32(1e-5))
        s16 = s32.astype(F16)
        q = np.clip(np.rint(w / s16.astype(F32)[:, None]), F32(-8), F32(7))
        return q.astype(np.int8), s16, None
    G = int(group_size)
    if G <= 0 or K % G:
        raise ValueError("K must be a multiple of group_size")
    s32 = np.maximum(amax / F32(127.0), F32(1e-5))
    s16 = s32.astype(F16)
    w8 = np.clip(np.rint(w / s16.astype(F32)[:, None]), F32(-127), F32(127))
    w8g = w8.reshape(N, K // G, G)
    m = np.abs(w8g).max(axis=2)
    sg = np.minimum(np.maximum(F32(1), np.ceil(m / F32(7))), F32(18))
    q = np.clip(np.rint(w8g / sg[:, :, None]), F32(-7), F32(7))
    return q.reshape(N, K).astype(np.int8), s16, sg.astype(np.int8)


def quantize_w8a8(w16: np.ndarray):
    """Per-channel symmetric int8 weights for W8A8 (R15): ``(q int8 [N, K] in
    [-127, 127], s fp16 [N])`` with ``s = fp16(max(max|w| / 127, 1e-5))`` and
    ``q = clamp(rint(w / s), -127, 127)``, decisions in fp32.  The integer GEMM and the
    output are :func:`w4a8_acc_ref` (no group scales) and :func:`w4a8_linear_ref`."""
    w16 = np.asarray(w16)
    if w16.dtype != F16 or w16.ndim != 2:
        raise ValueError("w16 must be a 2-D float16 array")
    w = w16.astype(F32)
    s16 = np.maximum(np.abs(w).max(axis=1) / F32(127.0), F32(1e-5)).astype(F16)
    q = np.clip(np.rint(w / s16.astype(F32)[:, None]), F32(-127), F32(127))
    return q.astype(np.int8), s16


def tile_w8a8(q: np.ndarray) -> np.ndarray:
    """int8 codes [N, K] -> the tiled W8A8 qweight int8 [ceil(N/16), K/128, 4, 2, 16, 16]
    (R15 layout): with ``kc = (k % 128) // 16``, code (n, k) goes to
    ``[n // 16, k // 128, kc % 4, kc // 4, n % 16, k % 16]``; rows past N hold 0."""
    q = np.asarray(q)
    if q.dtype != np.int8 or q.ndim != 2 or q.shape[1] % 128:
        raise ValueError("q must be int8 [N, K] with K a multiple of 128")
    N, K = q.shape
    Np = -(-N // 16) * 16
    full = np.zeros((Np, K), np.int8)
    full[:N] = q
    # [n16, r, g, h, c, b] -> [n16, g, c, h, r, b]
    return np.ascontiguousarray(full.reshape(Np // 16, 16, K // 128, 2, 4, 16).transpose(0, 2, 4, 3, 1, 5))


def untile_w8a8(tiled: np.ndarray, N: int) -> np.ndarray:
    """Inverse of :func:`tile_w8a8`: tiled int8 -> codes [N, K]."""
    t = np.asarray(tiled)
    n16, ng = t.shape[0], t.shape[1]
    return np.ascontiguousarray(t.transpose(0, 4, 1, 3, 2, 5)).reshape(n16 * 16, ng * 128)[:N]


def pack_w4a8(q: np.ndarray, cscale: np.ndarray, gscale):
    """-> ``(qweight int32 [ceil(N/16), K/128, 4, 16, 4] of biased nibbles q+8 in words
    split by halves (R5b; pad rows q = 0), cscale fp16 [N], gscale int8 [K/G, N] or None)``."""
    qweight = tile_words(split_halves(pack_nibbles(np.asarray(q, dtype=np.int64) + 8)), pad_word=0x88888888)
    gs = None if gscale is None else np.ascontiguousarray(np.asarray(gscale, dtype=np.int8).T)
    return qweight, np.asarray(cscale, dtype=F16), gs


def unpack_w4a8(qweight: np.ndarray, N: int, K: int) -> np.ndarray:
    """Tiled biased-nibble words -> signed int4 values [N, K] (int64)."""
    return unpack_nibbles(merge_halves(untile_words(qweight, N)), K).astype(np.int64) - 8


def w4a8_quant_act_ref(x16: np.ndarray, gamma16=None, eps: float = 1e-5):
    """Per-token symmetric int8 activation quantization, optionally fused with
    RMSNorm (R6).  Returns ``(xq int8 [M,K], s_a fp32 [M], t fp64 [M,K])`` where
    ``t`` is the fp32 value that was rounded to give ``xq`` (for near-tie
    accounting in tests)."""
    x = np.asarray(x16)
    if x.dtype != F16 or x.ndim != 2:
        raise ValueError("x16 must be a 2-D float16 array")
    M, K = x.shape
    if gamma16 is None:
        y32 = x.astype(F32)
    else:
        x64 = x.astype(F64)
        r = 1.0 / np.sqrt(np.mean(x64 * x64, axis=1) + float(eps))
        y64 = x64 * r[:, None] * np.asarray(gamma16, dtype=F16).astype(F64)[None, :]
        y32 = y64.astype(F32)
    return _quant_rows_int8(y32)


def _quant_rows_int8(y32: np.ndarray):
    """Per-row symmetric int8 quantization of fp32 values (R6): ``amax = max|y|``,
    ``inv = fp32(127 / amax)``, ``xq = clamp(rint(fp32(y * inv)), -127, 127)``,
    ``s_a = fp32(amax / 127)``.  A row for which the rule has no value -- ``amax == 0``,
    or ``inv`` not finite in fp32 (``amax`` below about ``2^-121``) -- gives ``xq = 0,
    s_a = 1``.  Returns ``(xq, s_a, t)`` with ``t`` the fp32 values that were rounded."""
    M, K = y32.shape
    amax = np.abs(y32).max(axis=1) if K else np.zeros(M, F32)
    xq = np.zeros((M, K), dtype=np.int8)
    s_a = np.ones(M, dtype=F32)
    t_all = np.zeros((M, K), dtype=F64)
    for m in range(M):
        if amax[m] == 0:
            continue
        with np.errstate(over="ignore"):
            inv = F32(127.0) / amax[m]
        if not np.isfinite(inv):
            continue
        t = y32[m] * inv
        xq[m] = np.clip(np.rint(t), -127, 127).astype(np.int8)
        s_a[m] = amax[m] / F32(127.0)
        t_all[m] = t
    return xq, s_a, t_all


def silu_ref(g: np.ndarray) -> np.ndarray:
    """SiLU in fp64: ``g / (1 + exp(-g))`` (written as ``g * sigmoid(g)`` with the
    overflow-safe branch for negative g)."""
    g = np.asarray(g, dtype=F64)
    e = np.exp(-np.abs(g))
    sig = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return g * sig


def silu_mul_quant_ref(gate_up16: np.ndarray):
    """The SiLU-gated input of the down projection quantized per token (R12): the fused
    gate+up output ``[M, 2I]`` holds gate in columns ``0..I-1`` and up in ``I..2I-1``;
    ``y = silu(gate) * up`` in fp64 (no fp16 round trip), then the per-token int8 rule
    of :func:`_quant_rows_int8` on ``fp32(y)``.  Returns ``(xq int8 [M, I], s_a fp32 [M],
    t fp64 [M, I])``."""
    gu = np.asarray(gate_up16)
    if gu.dtype != F16 or gu.ndim != 2 or gu.shape[1] % 2:
        raise ValueError("gate_up16 must be a 2-D float16 array with an even number of columns")
    I = gu.shape[1] // 2
    g = gu[:, :I].astype(F64)
    u = gu[:, I:].astype(F64)
    return _quant_rows_int8((silu_ref(g) * u).astype(F32))


def w4a8_acc_ref(xq: np.ndarray, q: np.ndarray, gscale_ng, group_size: int) -> np.ndarray:
    """Exact integer accumulators ``acc[m,n] = sum_k xq[m,k] * q[n,k] * s_g[n, k//G]``
    (int64).  ``gscale_ng`` is int8 [N, K/G] or None (per-channel)."""
    xq = np.asarray(xq, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    if gscale_ng is not None:
        G = int(group_size)
        q = q * np.repeat(np.asarray(gscale_ng, dtype=np.int64), G, axis=1)
    return xq @ q.T


def w4a8_linear_ref(acc: np.ndarray, s_a: np.ndarray, cscale: np.ndarray) -> np.ndarray:
    """fp64 outputs ``acc * s_a[m] * s_c[n]``."""
    return (np.asarray(acc, dtype=F64) * np.asarray(s_a, dtype=F64)[:, None]
            * np.asarray(cscale, dtype=F16).astype(F64)[None, :])

