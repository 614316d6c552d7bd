"""MI355X (gfx950) W4A16 / W4A8 group-quantized linear layer.

Python binding of the C ABI in ``include/w4a16.h`` (``libw4a16.so``); the
functions carry the names of the C entry points.
"""
from ._lib import (  # noqa: F401
    W4Error,
    awq_gemm,
    awq_gemm_noalloc,
    awq_gemm_workspace_bytes,
    awq_import_plain,
    awq_pack,
    awq_pack_sym,
    awq_unpack_dequant,
    bind_awq_gemm,
    bind_w4a8_gemm,
    bind_w4a8_quant_act,
    bind_w4a8_silu_mul_quant,
    lib_path,
    qweight_shape,
    load,
    w4a8_gemm,
    w4a8_gemm_i32,
    w4a8_gemm_workspace_bytes,
    w4a8_import_plain,
    w4a8_pack,
    w4a8_quant_act,
    w4a8_silu_mul_quant,
    w4_pack_codes,
    w8a8_pack,
    w8a8_qweight_shape,
    w8a8_gemm,
    w8a8_gemm_i32,
    w8a8_gemm_workspace_bytes,
    bind_w8a8_gemm,
    bind_ceiling_read,
    bind_ceiling_mfma,
)
