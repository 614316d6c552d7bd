"""CPU: the Python binding validates every tensor's shape against (M, N, K, group_size)
before any C call, so a mismatched argument raises ValueError instead of becoming an
out-of-bounds device access.  Tensors live on the ``meta`` device (shapes and dtypes
only, no storage): a call whose shapes are all consistent gets as far as the device
check and fails there, which shows that no C entry point was reached either way."""
import pytest
import torch

import w4a16_gemm_amd as w4

M, N, K = 4, 40, 512
f16, i32, i8, u8, f32 = torch.float16, torch.int32, torch.int8, torch.uint8, torch.float32


def t(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="meta")


def awq_args(group_size=128, ng=None):
    ng = ng if ng is not None else (1 if group_size == -1 else K // group_size)
    return dict(x=t((M, K), f16), qweight=t(w4.qweight_shape(N, K), i32), scales=t((ng, N), f16),
                qzeros=t((ng, (N + 7) // 8), i32))


def w4a8_args(group_size=-1):
    gs = None if group_size == -1 else t((K // 128, N), i8)
    return dict(xq=t((M, K), i8), s_a=t((M,), f32), qweight=t(w4.qweight_shape(N, K), i32), gscale=gs,
                cscale=t((N,), f16))


def raises_shape(fn, *args, match, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def reaches_device_check(fn, *args, **kw):
    with pytest.raises(ValueError, match="GPU device"):
        fn(*args, **kw)


# ---------------------------------------------------------------- W4A16
def test_awq_gemm_consistent_shapes_reach_the_device_check():
    for g in (128, 64, 32, -1):
        a = awq_args(g)
        reaches_device_check(w4.awq_gemm, a["x"], a["qweight"], a["scales"], a["qzeros"], group_size=g)
        reaches_device_check(w4.awq_gemm, a["x"], a["qweight"], a["scales"], a["qzeros"], group_size=g,
                             out=t((M, N), f16))
        reaches_device_check(w4.bind_awq_gemm, a["x"], a["qweight"], a["scales"], a["qzeros"], t((M, N), f16),
                             group_size=g)
        reaches_device_check(w4.awq_unpack_dequant, a["qweight"], a["scales"], a["qzeros"], group_size=g)


def test_awq_gemm_scales_of_another_group_size():
    a = awq_args(128)  # g128 scales [4, N] passed as g64: 8 rows would be read
    raises_shape(w4.awq_gemm, a["x"], a["qweight"], a["scales"], a["qzeros"], group_size=64, match="scales")
    raises_shape(w4.awq_unpack_dequant, a["qweight"], a["scales"], a["qzeros"], group_size=64, match="scales")
    raises_shape(w4.bind_awq_gemm, a["x"], a["qweight"], a["scales"], a["qzeros"], t((M, N), f16), group_size=64,
                 match="scales")


def test_awq_gemm_each_mismatch():
    a = awq_args(128)
    cases = [
        ("qzeros", dict(qzeros=t((K // 128, (N + 7) // 8 - 1), i32))),
        ("qzeros", dict(qzeros=t((K // 64, (N + 7) // 8), i32))),
        ("qweight", dict(qweight=t(w4.qweight_shape(N + 16, K), i32))),
        ("qweight", dict(qweight=t(w4.qweight_shape(N, K - 128), i32))),
        ("scales", dict(scales=t((K // 128 + 1, N), f16))),
    ]
    for match, over in cases:
        b = {**a, **over}
        raises_shape(w4.awq_gemm, b["x"], b["qweight"], b["scales"], b["qzeros"], match=match)
        raises_shape(w4.bind_awq_gemm, b["x"], b["qweight"], b["scales"], b["qzeros"], t((M, N), f16), match=match)
    for bad in ((M + 1, N), (M, N - 1), (N, M)):
        raises_shape(w4.awq_gemm, a["x"], a["qweight"], a["scales"], a["qzeros"], out=t(bad, f16), match="out")
        raises_shape(w4.bind_awq_gemm, a["x"], a["qweight"], a["scales"], a["qzeros"], t(bad, f16), match="out")
    raises_shape(w4.awq_gemm, a["x"], a["qweight"], a["scales"], a["qzeros"], group_size=256, match="group_size")
    raises_shape(w4.awq_gemm, t((M, K + 8), f16), a["qweight"], a["scales"], a["qzeros"], match="K=")
    raises_shape(w4.awq_gemm, a["x"], a["qweight"], a["scales"], a["qzeros"], workspace=t((64, 64), u8),
                 match="workspace")
    with pytest.raises(TypeError, match="out"):
        w4.awq_gemm(a["x"], a["qweight"], a["scales"], a["qzeros"], out=t((M, N), f32))


def test_pack_group_and_k_checks():
    raises_shape(w4.awq_pack, t((N, K + 64), f16), match="K=")
    raises_shape(w4.awq_pack, t((N, K), f16), group_size=16, match="group_size")
    raises_shape(w4.w4a8_pack, t((N, K), f16), group_size=64, match="group_size")
    reaches_device_check(w4.awq_pack, t((N, K), f16), group_size=-1)
    reaches_device_check(w4.w4a8_pack, t((N, K), f16), group_size=128)
    reaches_device_check(w4.w8a8_pack, t((N, K), f16))


# ----------------------------------------------------------------- W4A8
def test_w4a8_consistent_shapes_reach_the_device_check():
    for g in (-1, 128):
        a = w4a8_args(g)
        reaches_device_check(w4.w4a8_gemm, a["xq"], a["s_a"], a["qweight"], a["gscale"], a["cscale"], group_size=g)
        reaches_device_check(w4.w4a8_gemm, a["xq"], a["s_a"], a["qweight"], a["gscale"], a["cscale"], group_size=g,
                             out=t((M, N), f16))
        reaches_device_check(w4.bind_w4a8_gemm, a["xq"], a["s_a"], a["qweight"], a["gscale"], a["cscale"],
                             t((M, N), f16), group_size=g)
        reaches_device_check(w4.w4a8_gemm_i32, a["xq"], a["qweight"], a["gscale"], group_size=g, N=N)


def test_w4a8_each_mismatch():
    for g in (-1, 128):
        a = w4a8_args(g)
        for bad in ((M, N + 1), (M - 1, N)):
            raises_shape(w4.w4a8_gemm, a["xq"], a["s_a"], a["qweight"], a["gscale"], a["cscale"], group_size=g,
                         out=t(bad, f16), match="out")
            raises_shape(w4.bind_w4a8_gemm, a["xq"], a["s_a"], a["qweight"], a["gscale"], a["cscale"], t(bad, f16),
                         group_size=g, match="out")
        raises_shape(w4.w4a8_gemm, a["xq"], t((M + 1,), f32), a["qweight"], a["gscale"], a["cscale"], group_size=g,
                     match="s_a")
        raises_shape(w4.bind_w4a8_gemm, a["xq"], t((1,), f32), a["qweight"], a["gscale"], a["cscale"],
                     t((M, N), f16), group_size=g, match="s_a")
        raises_shape(w4.w4a8_gemm, a["xq"], a["s_a"], a["qweight"], a["gscale"], t((N + 16,), f16), group_size=g,
                     match="qweight")
    a = w4a8_args(128)
    raises_shape(w4.w4a8_gemm, a["xq"], a["s_a"], a["qweight"], t((K // 128, N - 1), i8), a["cscale"],
                 group_size=128, match="gscale")
    raises_shape(w4.w4a8_gemm, a["xq"], a["s_a"], a["qweight"], t((K // 64, N), i8), a["cscale"],
                 group_size=128, match="gscale")
    raises_shape(w4.w4a8_gemm, a["xq"], a["s_a"], a["qweight"], None, a["cscale"], group_size=128, match="gscale")
    raises_shape(w4.w4a8_gemm, a["xq"], a["s_a"], a["qweight"], a["gscale"], a["cscale"], group_size=-1,
                 match="gscale")
    raises_shape(w4.w4a8_gemm_i32, a["xq"], a["qweight"], t((1, N), i8), group_size=128, N=N, match="gscale")


def test_activation_quantizers():
    x = t((M, K), f16)
    reaches_device_check(w4.w4a8_quant_act, x, t((K,), f16))
    raises_shape(w4.w4a8_quant_act, x, t((K - 8,), f16), match="gamma")
    reaches_device_check(w4.bind_w4a8_quant_act, x, t((K,), f16), t((M, K), i8), t((M,), f32))
    raises_shape(w4.bind_w4a8_quant_act, x, t((K + 8,), f16), t((M, K), i8), t((M,), f32), match="gamma")
    raises_shape(w4.bind_w4a8_quant_act, x, None, t((M, K - 8), i8), t((M,), f32), match="xq")
    raises_shape(w4.bind_w4a8_quant_act, x, None, t((M, K), i8), t((M + 1,), f32), match="s_a")
    gu = t((M, 2 * K), f16)
    reaches_device_check(w4.bind_w4a8_silu_mul_quant, gu, t((M, K), i8), t((M,), f32))
    raises_shape(w4.bind_w4a8_silu_mul_quant, gu, t((M, 2 * K), i8), t((M,), f32), match="xq")
    raises_shape(w4.bind_w4a8_silu_mul_quant, gu, t((M, K), i8), t((2 * M,), f32), match="s_a")
    raises_shape(w4.w4a8_silu_mul_quant, t((M, 2 * K + 1), f16), match="even")


# ----------------------------------------------------------------- W8A8
def test_w8a8_checks():
    xq, s_a, cs = t((M, K), i8), t((M,), f32), t((N,), f16)
    qw = t(w4.w8a8_qweight_shape(N, K), i8)
    reaches_device_check(w4.w8a8_gemm, xq, s_a, qw, cs)
    reaches_device_check(w4.bind_w8a8_gemm, xq, s_a, qw, cs, t((M, N), f16))
    reaches_device_check(w4.w8a8_gemm_i32, xq, qw, N)
    raises_shape(w4.w8a8_gemm, xq, s_a, qw, cs, out=t((M, N + 1), f16), match="out")
    raises_shape(w4.bind_w8a8_gemm, xq, s_a, qw, cs, t((M + 1, N), f16), match="out")
    raises_shape(w4.w8a8_gemm, xq, t((M - 1,), f32), qw, cs, match="s_a")
    raises_shape(w4.bind_w8a8_gemm, xq, t((M - 1,), f32), qw, cs, t((M, N), f16), match="s_a")
    raises_shape(w4.w8a8_gemm, xq, s_a, t(w4.w8a8_qweight_shape(N, K + 128), i8), cs, match="qweight")
    raises_shape(w4.w8a8_gemm_i32, xq, qw, N + 16, match="qweight")


def test_devices_must_match():
    # a CPU tensor among meta tensors: the device check names it (first non-GPU one)
    a = awq_args(128)
    with pytest.raises(ValueError, match="x must be on a GPU device"):
        w4.awq_gemm(torch.empty((M, K), dtype=f16), a["qweight"], a["scales"], a["qzeros"])
