"""CPU: plant plausible mistakes in a copy of the oracle and check that at least
one pin fails for each.  This shows the pins can catch a dropped term, a wrong
sign, index or constant, or a transposed operand."""
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "ref.py")

MUTANTS = [
    ("scale divisor 16", "s32 = (mx - mn) / F32(15.0)", "s32 = (mx - mn) / F32(16.0)"),
    ("scale from unrounded fp32", "s = s16.astype(F32)\n", "s = s32\n"),
    ("zero sign flipped", "np.rint(-mn / s)", "np.rint(mn / s)"),
    ("zero not added", "np.rint(w / s[:, :, None]) + z[:, :, None]", "np.rint(w / s[:, :, None])"),
    ("code clamp 14", "+ z[:, :, None], F32(0), F32(15))", "+ z[:, :, None], F32(0), F32(14))"),
    ("min/max swapped", "mn = w.min(axis=2)\n    mx = w.max(axis=2)", "mn = w.max(axis=2)\n    mx = w.min(axis=2)"),
    ("dequant adds zero", "(codes.astype(F64) - z) * s", "(codes.astype(F64) + z) * s"),
    ("dequant drops zero", "(codes.astype(F64) - z) * s", "codes.astype(F64) * s"),
    ("pack nibble order reversed", "words += padded[:, i::8] << (4 * i)", "words += padded[:, i::8] << (4 * (7 - i))"),
    ("unpack nibble order reversed", "out[:, i::8] = (u >> (4 * i)) & 0xF", "out[:, i::8] = (u >> (4 * (7 - i))) & 0xF"),
    ("parity split reversed", "out |= ((u >> (4 * i)) & 0xF) << (4 * (i // 2 + 4 * (i % 2)))", "out |= ((u >> (4 * i)) & 0xF) << (4 * (4 * (i % 2) + 3 - i // 2))"),
    ("parity merge identity", "out |= ((u >> (4 * (i // 2 + 4 * (i % 2)))) & 0xF) << (4 * i)", "out |= ((u >> (4 * i)) & 0xF) << (4 * i)"),
    ("awq qweight without the parity split", "qweight = tile_words(split_parity(pack_nibbles(codes)))", "qweight = tile_words(pack_nibbles(codes))"),
    ("halves split reversed", "out |= ((u >> (4 * i)) & 0xF) << (4 * (2 * (i % 4) + i // 4))", "out |= ((u >> (4 * i)) & 0xF) << (4 * (2 * (i // 4) + i % 4))"),
    ("halves merge identity", "out |= ((u >> (4 * (2 * (i % 4) + i // 4))) & 0xF) << (4 * i)", "out |= ((u >> (4 * i)) & 0xF) << (4 * i)"),
    ("w4a8 qweight without the halves split", "qweight = tile_words(split_halves(pack_nibbles(np.asarray(q, dtype=np.int64) + 8)), pad_word=0x88888888)", "qweight = tile_words(pack_nibbles(np.asarray(q, dtype=np.int64) + 8), pad_word=0x88888888)"),
    ("tile rows and slots swapped", "out[:, :, slot, n, w] = full[n::16, slot * 4 + w::16]", "out[:, :, slot, n, w] = full[n::16, (w * 4 + slot)::16]"),
    ("untile rows and slots swapped", "full[n::16, slot * 4 + w::16] = tiled[:, :, slot, n, w]", "full[n::16, (w * 4 + slot)::16] = tiled[:, :, slot, n, w]"),
    ("scales not transposed", "scales = np.ascontiguousarray(scales_gn.T)", "scales = np.ascontiguousarray(scales_gn).reshape(scales_gn.shape[::-1])"),
    ("group index off by one", "s = np.repeat(scales.astype(F64), G, axis=1)", "s = np.roll(np.repeat(scales.astype(F64), G, axis=1), 1, axis=1)"),
    ("matmul transposed operand", "np.asarray(w_deq, dtype=F64).T", "np.asarray(w_deq, dtype=F64).T[::-1]"),
    ("w4a8 s_g cap 19", "np.ceil(m / F32(7))), F32(18))", "np.ceil(m / F32(7))), F32(19))"),
    ("w4a8 s_g rint", "np.ceil(m / F32(7))", "np.rint(m / F32(7))"),
    ("w4a8 first level /128", "amax / F32(127.0)", "amax / F32(128.0)"),
    ("w4a8 bias 7", "np.asarray(q, dtype=np.int64) + 8)", "np.asarray(q, dtype=np.int64) + 7)"),
    ("act eps dropped", "np.mean(x64 * x64, axis=1) + float(eps)", "np.mean(x64 * x64, axis=1)"),
    ("act gamma dropped", "y64 = x64 * r[:, None] * np.asarray(gamma16, dtype=F16).astype(F64)[None, :]", "y64 = x64 * r[:, None]"),
    ("act s_a over 128", "s_a[m] = amax[m] / F32(127.0)", "s_a[m] = amax[m] / F32(128.0)"),
    ("act truncation", "xq[m] = np.clip(np.rint(t), -127, 127)", "xq[m] = np.clip(np.trunc(t), -127, 127)"),
    ("act rounds half away from zero", "xq[m] = np.clip(np.rint(t), -127, 127)", "xq[m] = np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127)"),
    ("weight codes round half away from zero", "q = np.clip(np.rint(w / s[:, :, None])", "q = np.clip(np.sign(w) * np.floor(np.abs(w / s[:, :, None]) + 0.5)"),
    ("silu returns the sigmoid", "    return g * sig\n", "    return sig\n"),
    ("silu sigmoid of -g", "sig = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))", "sig = np.where(g >= 0, e / (1.0 + e), 1.0 / (1.0 + e))"),
    ("silu gate and up swapped", "g = gu[:, :I].astype(F64)\n    u = gu[:, I:].astype(F64)", "u = gu[:, :I].astype(F64)\n    g = gu[:, I:].astype(F64)"),
    ("silu gate and up interleaved", "g = gu[:, :I].astype(F64)\n    u = gu[:, I:].astype(F64)", "g = gu[:, 0::2].astype(F64)\n    u = gu[:, 1::2].astype(F64)"),
    ("tiny rows zeroed below 2^-64", "        if amax[m] == 0:\n", "        if amax[m] < 2.0 ** -64:\n"),
    ("rows with an infinite 127/amax quantized", "        if not np.isfinite(inv):\n            continue\n", ""),
    ("sym divisor 8", "s16 = np.maximum(amax / F32(7.0), F32(1e-5)).astype(F16)", "s16 = np.maximum(amax / F32(8.0), F32(1e-5)).astype(F16)"),
    ("sym max without abs", "amax = np.abs(w).max(axis=2)", "amax = w.max(axis=2)"),
    ("sym zero point 7", "codes = (q + F32(8)).reshape(N, K).astype(np.uint8)", "codes = (q + F32(7)).reshape(N, K).astype(np.uint8)"),
    ("per-channel as g128", "G = K if int(group_size) == -1 else int(group_size)\n    if G <= 0", "G = 128 if int(group_size) == -1 else int(group_size)\n    if G <= 0"),
    ("w8a8 divisor 128", "s16 = np.maximum(np.abs(w).max(axis=1) / F32(127.0), F32(1e-5)).astype(F16)", "s16 = np.maximum(np.abs(w).max(axis=1) / F32(128.0), F32(1e-5)).astype(F16)"),
    ("w8a8 clamp 126", "q = np.clip(np.rint(w / s16.astype(F32)[:, None]), F32(-127), F32(127))\n    return q.astype(np.int8), s16", "q = np.clip(np.rint(w / s16.astype(F32)[:, None]), F32(-126), F32(126))\n    return q.astype(np.int8), s16"),
    ("w8a8 tile c and h swapped", "transpose(0, 2, 4, 3, 1, 5))\n", "transpose(0, 2, 3, 4, 1, 5)).reshape(-1, (q.shape[1]) // 128, 4, 2, 16, 16)\n"),
    ("acc ignores group scale", "q = q * np.repeat(np.asarray(gscale_ng, dtype=np.int64), G, axis=1)", "q = q"),
]


def _build(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mut = _build(old, new)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mut)
        except Exception as e:  # AssertionError or a shape/type error the mistake causes
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutant {name!r}"
