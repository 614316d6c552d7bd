"""Pins that tie the CPU oracle to facts outside itself.

Every pin takes an oracle module (the real ``oracle.ref`` or a mutant built by
``test_oracle_mutants.py``) and raises ``AssertionError`` when the oracle
disagrees with:

* hand-worked examples of the stated rules (``tests/golden/``),
* constructed inputs whose exact answer is known by construction,
* mathematical bounds and invariants of the rules,
* brute force in exact rational / integer arithmetic on tiny inputs,
* algebraic special cases that reduce to a plain matrix identity.

None of the pins re-types an oracle formula and compares it with itself.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import synth
from golden_io import read_cases, read_pack_words, read_silu_cases, read_variant_cases

F16, F32, F64 = np.float16, np.float32, np.float64


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- packing
def pin_pack_words(ora):
    """Worked words of the plain nibble order (tests/golden/pack_words.txt)."""
    for codes, word in read_pack_words():
        got = ora.pack_nibbles(np.array([codes], dtype=np.uint8))
        assert got.dtype == np.int32 and got.shape == (1, 1)
        assert int(got.view(np.uint32)[0, 0]) == word, (codes, hex(int(got.view(np.uint32)[0, 0])), hex(word))
        back = ora.unpack_nibbles(np.array([[np.uint32(word)]], dtype=np.uint32).view(np.int32), 8)
        assert back.tolist() == [codes]


def pin_pack_bijection(ora):
    """pack o unpack = id on words, unpack o pack = id on codes, pad nibbles 0."""
    # all 8 x 16 one-hot nibbles: the word equals code << 4i, unsigned
    for i in range(8):
        for c in range(16):
            codes = np.zeros((1, 8), np.uint8)
            codes[0, i] = c
            w = ora.pack_nibbles(codes)
            assert int(w.view(np.uint32)[0, 0]) == (c << (4 * i))
    rng = _rng(7)
    words = rng.integers(0, 2**32, size=(1000, 37), dtype=np.uint64).astype(np.uint32).view(np.int32)
    codes = ora.unpack_nibbles(words, 37 * 8)
    assert codes.max() <= 15
    assert np.array_equal(ora.pack_nibbles(codes), words)
    c2 = rng.integers(0, 16, size=(33, 21), dtype=np.int64).astype(np.uint8)  # ragged: 21 % 8 != 0
    w2 = ora.pack_nibbles(c2)
    assert w2.shape == (33, 3)
    assert np.array_equal(ora.unpack_nibbles(w2, 21), c2)
    assert np.all((w2.view(np.uint32)[:, 2] >> 20) == 0)  # 3 pad nibbles are zero


def pin_parity_words(ora):
    """Worked words of the W4A16 qweight's parity-split word format
    (tests/golden/parity_words.txt): the plain word of the codes, split, gives the
    listed word; merging it gives the plain word back; and a single code at element i
    of a word lands, after pack_awq, in nibble i // 2 + 4 (i % 2) of the one nonzero
    qweight word (element 8 j + i of a row)."""
    for codes, word in read_pack_words("parity_words.txt"):
        plain = ora.pack_nibbles(np.array([codes], dtype=np.uint8))
        got = ora.split_parity(plain)
        assert int(got.view(np.uint32)[0, 0]) == word, (codes, hex(int(got.view(np.uint32)[0, 0])), hex(word))
        back = ora.merge_parity(np.array([[np.uint32(word)]], dtype=np.uint32).view(np.int32))
        assert np.array_equal(back, plain)
    nib = {0: 0, 1: 4, 2: 1, 3: 5, 4: 2, 5: 6, 6: 3, 7: 7}  # element -> nibble, by hand
    N, K = 3, 128
    for k in range(0, 16):
        codes = np.zeros((N, K), np.uint8)
        codes[1, k] = 11
        qw, _, _ = ora.pack_awq(codes, np.ones((N, 1), F16), np.zeros((N, 1), np.uint8))
        flat = qw.reshape(-1).view(np.uint32)
        off = ((k % 128) // 32) * 64 + 1 * 4 + (k % 32) // 8
        assert np.count_nonzero(flat) == 1 and int(flat[off]) == 11 << (4 * nib[k % 8]), k
    rng = _rng(9)
    words = rng.integers(0, 2**32, size=(64, 5), dtype=np.uint64).astype(np.uint32).view(np.int32)
    assert np.array_equal(ora.merge_parity(ora.split_parity(words)), words)
    assert np.array_equal(ora.split_parity(ora.merge_parity(words)), words)


def pin_halves_words(ora):
    """Worked words of the W4A8 qweight's split-halves word format
    (tests/golden/halves_words.txt): the plain word of the codes, split, gives the
    listed word; merging it gives the plain word back; and a single nonzero q at element
    i of a word lands, after pack_w4a8, as the biased nibble q + 8 in nibble
    2 (i % 4) + i // 4 of the only word that is not 0x88888888."""
    for codes, word in read_pack_words("halves_words.txt"):
        plain = ora.pack_nibbles(np.array([codes], dtype=np.uint8))
        got = ora.split_halves(plain)
        assert int(got.view(np.uint32)[0, 0]) == word, (codes, hex(int(got.view(np.uint32)[0, 0])), hex(word))
        back = ora.merge_halves(np.array([[np.uint32(word)]], dtype=np.uint32).view(np.int32))
        assert np.array_equal(back, plain)
    nib = {0: 0, 1: 2, 2: 4, 3: 6, 4: 1, 5: 3, 6: 5, 7: 7}  # element -> nibble, by hand
    N, K = 3, 128
    for k in range(16):
        q = np.zeros((N, K), np.int64)
        q[2, k] = -5
        qw, _, _ = ora.pack_w4a8(q, np.ones(N, F16), None)
        flat = qw.reshape(-1).view(np.uint32)
        off = ((k % 128) // 32) * 64 + 2 * 4 + (k % 32) // 8
        others = np.delete(flat, off)
        assert np.all(others == 0x88888888), k
        expect = (0x88888888 & ~(0xF << (4 * nib[k % 8]))) | (3 << (4 * nib[k % 8]))
        assert int(flat[off]) == expect, (k, hex(int(flat[off])))
    rng = _rng(10)
    words = rng.integers(0, 2**32, size=(64, 5), dtype=np.uint64).astype(np.uint32).view(np.int32)
    assert np.array_equal(ora.merge_halves(ora.split_halves(words)), words)
    assert np.array_equal(ora.split_halves(ora.merge_halves(words)), words)


def pin_tile_layout(ora):
    """Tiled word order: a single code placed at (n, k) lands in exactly one word of
    the flat qweight, at the offset computed by hand from the layout rule
    ((n/16 * K/128 + k/128) * 4 + (k % 128)/32) * 64 + (n % 16) * 4 + (k % 32)/8,
    nibble k % 8; tile/untile are inverse bijections; pad rows carry the pad word."""
    N, K = 37, 256
    for (n, k, c) in ((17, 200, 9), (0, 0, 15), (36, 255, 1), (15, 127, 6), (16, 128, 3)):
        codes = np.zeros((N, K), np.uint8)
        codes[n, k] = c
        flat = ora.tile_words(ora.pack_nibbles(codes)).reshape(-1).view(np.uint32)
        off = ((n // 16 * (K // 128) + k // 128) * 4 + (k % 128) // 32) * 64 + (n % 16) * 4 + (k % 32) // 8
        assert flat.size == 48 * K // 8
        assert int(flat[off]) == c << (4 * (k % 8)), (n, k)
        assert np.count_nonzero(flat) == 1
    rng = _rng(5)
    words = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    t = ora.tile_words(words, pad_word=0x88888888)
    assert t.shape == (3, 2, 4, 16, 4)
    assert np.array_equal(ora.untile_words(t, N), words)
    assert np.all(ora.untile_words(t, 48)[N:].view(np.uint32) == 0x88888888)


# ------------------------------------------------------- asymmetric rule
def pin_asym_worked(ora):
    """Hand-worked groups (tests/golden/asym_g128_worked.txt)."""
    for case in read_cases("asym_g128_worked.txt"):
        vals = case["values"]
        assert vals.size == 128
        # place the group at row 1, group 1 of a [3, 384] matrix; other entries random
        w = (np.random.default_rng(3).standard_normal((3, 384)) * 0.02).astype(F16)
        w[1, 128:256] = vals
        codes, scales, zeros = ora.quantize_asym(w, 128)
        assert scales.shape == (3, 3) and zeros.shape == (3, 3)
        assert scales[1, 1].view(np.uint16) == case["scale"].view(np.uint16), case["name"]
        assert int(zeros[1, 1]) == case["zero"], case["name"]
        hexes = [format(int(v.view(np.uint16)), "04X") for v in vals]
        for j, hx in enumerate(hexes):
            assert int(codes[1, 128 + j]) == case["code"][hx], (case["name"], hx)
        qw, sg, qz = ora.pack_awq(codes, scales, zeros)
        wd = ora.dequant_awq(qw, sg, qz, 384, 128)
        for j, hx in enumerate(hexes):
            assert Fraction(wd[1, 128 + j]) == Fraction(case["deq"][hx]), (case["name"], hx)


def pin_asym_constructed(ora):
    """Weights built as (q - z) * 2^e with q spanning 0..15 are recovered exactly."""
    rng = _rng(11)
    N, K, G = 6, 512, 128
    q = rng.integers(0, 16, size=(N, K))
    ng = K // G
    q[:, 3::G] = 0          # every group spans the full code range 0..15
    q[:, 77::G] = 15
    z = rng.integers(0, 16, size=(N, ng))
    e = rng.integers(-10, -3, size=(N, ng))
    s = np.ldexp(1.0, e)
    w = ((q - np.repeat(z, G, axis=1)) * np.repeat(s, G, axis=1)).astype(F16)
    codes, scales, zeros = ora.quantize_asym(w, G)
    assert np.array_equal(codes.astype(np.int64), q)
    assert np.array_equal(zeros.astype(np.int64), z)
    assert np.array_equal(scales.astype(F64), s)


def pin_asym_roundtrip_bound(ora):
    """|w - w_deq| <= s16/2 + 15*|s_exact - s16| (+ fp32 slack) for groups with
    min <= 0 <= max, where s_exact = (max - min)/15 in exact arithmetic; codes and
    zeros stay in [0, 15]; scales are positive."""
    inp = synth.make_linear(0, 256, 1024, seed=5, outliers=True)
    w = inp.w.numpy()
    G = 128
    codes, scales, zeros = ora.quantize_asym(w, G)
    assert codes.max() <= 15 and zeros.max() <= 15
    assert np.all(scales.astype(F64) > 0)
    qw, sg, qz = ora.pack_awq(codes, scales, zeros)
    wd = ora.dequant_awq(qw, sg, qz, w.shape[1], G)
    wg = w.astype(F64).reshape(w.shape[0], -1, G)
    mn, mx = wg.min(axis=2), wg.max(axis=2)
    ok = (mn <= 0) & (mx >= 0)
    assert ok.mean() > 0.99
    s16 = scales.astype(F64)
    bound = s16 / 2 + 15 * np.abs((mx - mn) / 15 - s16) + 1e-6 * s16
    err = np.abs(wg - wd.reshape(wg.shape)).max(axis=2)
    assert np.all(err[ok] <= bound[ok]), float((err / bound)[ok].max())
    # and the error is not trivially small: the bound is nearly attained
    assert (err[ok] / s16[ok]).max() > 0.45


# ----------------------------------------------------------------- GEMM
def _frac16(v):
    return Fraction(float(v))


def pin_fraction_bruteforce(ora):
    """Tiny GEMMs in exact rational arithmetic from the natural-orientation
    quantizer outputs, against the packed -> dequant -> fp64 matmul chain."""
    for (M, N, K, G, seed) in ((2, 5, 256, 128, 1), (3, 9, 128, 128, 2), (1, 16, 384, 128, 3)):
        inp = synth.make_linear(M, N, K, seed=seed, outliers=True)
        w, x = inp.w.numpy(), inp.x.numpy()
        codes, scales, zeros = ora.quantize_asym(w, G)
        ref = ora.awq_reference(w, x, G)
        for m in range(M):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    acc += _frac16(x[m, k]) * (int(codes[n, k]) - int(zeros[n, k // G])) * _frac16(scales[n, k // G])
                got = Fraction(float(ref["y"][m, n]))
                scale = sum(abs(_frac16(x[m, k])) for k in range(K)) * max(abs(_frac16(s)) for s in scales[n]) * 15
                assert abs(got - acc) <= scale * Fraction(1, 2**50), (M, N, K, m, n)


def pin_identity_probe(ora):
    """Unit-vector rows e_k: Y[m, n] equals the dequantized weight w_deq[n, k],
    which is (code - zero) * scale of the natural-orientation outputs."""
    N, K, G = 24, 384, 128
    w = synth.make_linear(0, N, K, seed=9, outliers=True).w.numpy()
    ks = np.array([0, 1, 7, 8, 127, 128, 200, 383])
    x = np.zeros((len(ks), K), F16)
    x[np.arange(len(ks)), ks] = 1
    codes, scales, zeros = ora.quantize_asym(w, G)
    y = ora.awq_reference(w, x, G)["y"]
    for m, k in enumerate(ks):
        expect = (codes[:, k].astype(F64) - zeros[:, k // G]) * scales[:, k // G].astype(F64)
        assert np.array_equal(y[m], expect), k


def pin_per_channel_special_case(ora):
    """G = K: W_deq = diag(s) (Q - z 1^T), so Y = (X Q^T - (X 1) z^T) diag(s)."""
    M, N, K = 5, 12, 256
    inp = synth.make_linear(M, N, K, seed=4, outliers=True)
    w, x = inp.w.numpy(), inp.x.numpy()
    codes, scales, zeros = ora.quantize_asym(w, K)
    assert scales.shape == (N, 1)
    y = ora.awq_reference(w, x, K)["y"]
    X = x.astype(F64)
    alt = (X @ codes.astype(F64).T - X.sum(axis=1, keepdims=True) * zeros[:, 0].astype(F64)[None, :]) \
        * scales[:, 0].astype(F64)[None, :]
    assert np.allclose(y, alt, rtol=1e-12, atol=1e-12)


def pin_constructed_exact_gemm(ora):
    """Integer activations and power-of-two scales: every sum is an exact dyadic
    number, so the fp64 chain must equal an integer computation exactly."""
    rng = _rng(21)
    M, N, K, G = 4, 10, 512, 128
    q = rng.integers(0, 16, size=(N, K))
    q[:, ::G] = 0
    q[:, 1::G] = 15
    z = rng.integers(0, 16, size=(N, K // G))
    w = ((q - np.repeat(z, G, axis=1)) * 0.125).astype(F16)
    x = rng.integers(-4, 5, size=(M, K)).astype(F16)
    y = ora.awq_reference(w, x, G)["y"]
    exact = (x.astype(np.int64) @ (q - np.repeat(z, G, axis=1)).T)  # times 1/8
    assert np.array_equal(y * 8, exact.astype(F64))


# ------------------------------------------------------------------ W4A8
def pin_w4a8_worked(ora):
    """Hand-worked rows (tests/golden/w4a8_worked.txt)."""
    for case in read_cases("w4a8_worked.txt"):
        w = case["values"][None, :]
        q, cs, gs = ora.quantize_w4a8(w, case["group"])
        assert cs[0].view(np.uint16) == case["cscale"].view(np.uint16), case["name"]
        if case["group"] == -1:
            assert gs is None
            assert q[0].tolist() == case["q"]
        else:
            assert gs[0].tolist() == case["gscale"]
            G = case["group"]
            for g, head in enumerate(case["q_head"]):
                assert q[0, g * G:g * G + len(head)].tolist() == head, (case["name"], g)


def pin_w4a8_exhaustive(ora):
    """Every group maximum m in 0..127 and every w8 in [-m, m]: the two-level rule
    keeps |q * s_g| <= 127 (the int8 product never overflows), q in [-7, 7],
    s_g in [1, 18], and |w8 - q * s_g| <= s_g / 2."""
    G = 256
    rows = np.zeros((128, G), np.int64)
    for m in range(128):
        vals = np.arange(-m, m + 1)
        rows[m, :vals.size] = vals
    w8 = rows.reshape(1, -1)
    w = (w8 * 2.0**-7).astype(F16)          # exact; row max 127 * 2^-7 -> s_c = 2^-7
    q, cs, gs = ora.quantize_w4a8(w, G)
    assert float(cs[0]) == 2.0**-7
    qv = q.astype(np.int64).reshape(128, G)
    sg = gs.astype(np.int64).reshape(128)
    assert np.all((sg >= 1) & (sg <= 18))
    assert np.all(np.abs(qv) <= 7)
    prod = qv * sg[:, None]
    assert np.all(np.abs(prod) <= 127)
    err = np.abs(rows - prod)
    assert np.all(2 * err <= sg[:, None]), int((2 * err - sg[:, None]).max())
    # per-channel: q in [-8, 7] and |w - q s_c| <= s_c / 2 within the range
    w2 = synth.make_linear(0, 64, 512, seed=8, outliers=True).w.numpy()
    q2, c2, _ = ora.quantize_w4a8(w2, -1)
    assert q2.min() >= -8 and q2.max() <= 7
    c = c2.astype(F64)[:, None]
    assert np.all(np.abs(w2.astype(F64) - q2 * c) <= c / 2 + 7 * np.abs(np.abs(w2.astype(F64)).max(1, keepdims=True) / 7 - c) + 1e-9)


def pin_quant_act_closed_forms(ora):
    """Closed forms of per-token int8 quantization with and without RMSNorm."""
    K = 512
    # no-norm, one-hot rows: code +-127 at k, zero elsewhere; s_a = |a| / 127
    a = np.array([0.5, -3.0, 1.0, 65504.0], F16)
    x = np.zeros((4, K), F16)
    x[np.arange(4), [0, 5, 511, 300]] = a
    xq, sa, _ = ora.w4a8_quant_act_ref(x, None)
    for m in range(4):
        row = np.zeros(K, np.int64)
        row[[0, 5, 511, 300][m]] = 127 if a[m] > 0 else -127
        assert np.array_equal(xq[m].astype(np.int64), row)
        assert abs(float(sa[m]) - abs(float(a[m])) / 127) <= 1e-7 * abs(float(a[m]))
    # half-way codes round to even: x = [127, 62.5, -0.5, 1.5] -> [127, 62, 0, 2]
    x2 = np.zeros((1, K), F16)
    x2[0, :4] = [127, 62.5, -0.5, 1.5]
    xq2, sa2, _ = ora.w4a8_quant_act_ref(x2, None)
    assert xq2[0, :4].tolist() == [127, 62, 0, 2] and float(sa2[0]) == 1.0
    # RMSNorm on constant rows with unit gamma: y = c / sqrt(c^2 + eps) for every k
    gamma = np.ones(K, F16)
    cs = np.array([0.001, -0.25, 2.0], F16)
    xc = np.repeat(cs[:, None], K, axis=1)
    xq3, sa3, _ = ora.w4a8_quant_act_ref(xc, gamma, 1e-5)
    for m, c in enumerate(cs.astype(F64)):
        y = c / np.sqrt(c * c + 1e-5)
        assert np.all(xq3[m] == (127 if c > 0 else -127))
        assert abs(float(sa3[m]) - abs(y) / 127) <= 1e-6 * abs(y) / 127
    # RMSNorm with gamma, one row: y_k = x_k * gamma_k / rms; codes follow
    inp = synth.make_linear(3, 8, K, seed=12, rms_spread=True, with_gamma=True)
    xr, gr = inp.x.numpy(), inp.gamma.numpy()
    xq4, sa4, _ = ora.w4a8_quant_act_ref(xr, gr, 1e-5)
    for m in range(3):
        rms = np.sqrt((xr[m].astype(F64) ** 2).sum() / K + 1e-5)
        y = xr[m].astype(F64) * gr.astype(F64) / rms
        assert abs(float(sa4[m]) * 127 - np.abs(y).max()) <= 1e-6 * np.abs(y).max()
        assert np.abs(xq4[m]).max() == 127
        assert np.all(np.abs(xq4[m] - y / (np.abs(y).max() / 127)) <= 0.5 + 1e-4)
    # a zero row: s_a = 1, codes 0
    xz, sz, _ = ora.w4a8_quant_act_ref(np.zeros((1, K), F16), gamma)
    assert float(sz[0]) == 1.0 and not xz.any()


def pin_silu_worked(ora):
    """Hand-worked SiLU-gated row (tests/golden/silu_mul_quant_worked.txt)."""
    for case in read_silu_cases():
        xq, sa, _ = ora.silu_mul_quant_ref(case["gate_up"][None, :])
        assert xq[0].tolist() == case["xq"], case["name"]
        assert abs(float(sa[0]) - case["s_a"]) <= 1e-7 * case["s_a"], case["name"]


def pin_silu_closed_forms(ora):
    """silu(0) = 0; silu(g) - silu(-g) = g; silu(ln 3) = 0.75 ln 3; silu(g) -> g for
    large g and -> 0 for very negative g (no overflow at the fp16 extremes)."""
    g = np.concatenate([np.linspace(-30, 30, 601), [0.0, 1e-3, -1e-3, 65504.0, -65504.0]])
    s = ora.silu_ref(g)
    assert s[-5] == 0.0
    assert np.all(np.abs((s - ora.silu_ref(-g)) - g) <= 1e-14 * np.maximum(1, np.abs(g)))
    assert abs(ora.silu_ref(np.log(3.0)) - 0.75 * np.log(3.0)) <= 1e-15
    assert s[-2] == 65504.0 and s[-1] == 0.0 and np.all(np.isfinite(s))
    # the minimum of silu is about -0.2785 at g = -1.2785 (root of 1 + g (1 - sigmoid(g)) = 0)
    assert abs(s.min() - (-0.27846454)) < 1e-3


def pin_silu_special_cases(ora):
    """Gate values >= 40 make silu(g) = g exactly in fp64 (exp(-40) < 2^-53), so with
    up = 1 the SiLU-gated quantization equals the plain per-token rule on the gate,
    and with up = -1 its codes are negated; a zero gate row gives s_a = 1, codes 0."""
    rng = _rng(31)
    M, I = 6, 384
    gate = rng.uniform(40, 2000, size=(M, I)).astype(F16)
    gate[:, ::7] = rng.uniform(40, 60000, size=(M, (I + 6) // 7)).astype(F16)
    ones = np.ones((M, I), F16)
    xq, sa, _ = ora.silu_mul_quant_ref(np.concatenate([gate, ones], axis=1))
    rq, rsa, _ = ora.w4a8_quant_act_ref(gate, None)
    assert np.array_equal(xq, rq) and np.array_equal(sa, rsa)
    xn, san, _ = ora.silu_mul_quant_ref(np.concatenate([gate, -ones], axis=1))
    assert np.array_equal(xn, -rq) and np.array_equal(san, rsa)
    z = np.zeros((1, 2 * I), F16)
    z[0, I:] = 5.0
    xz, sz, _ = ora.silu_mul_quant_ref(z)
    assert float(sz[0]) == 1.0 and not xz.any()
    # a row with up = 0 except one element: only that element is non-zero, code +-127
    r = np.zeros((1, 2 * I), F16)
    r[0, :I] = rng.uniform(-4, 4, size=I).astype(F16)
    r[0, I + 17] = 2.0
    xo, so, _ = ora.silu_mul_quant_ref(r)
    expect = np.zeros(I, np.int64)
    sv = ora.silu_ref(float(r[0, 17]))
    expect[17] = 127 if sv > 0 else -127
    assert np.array_equal(xo[0].astype(np.int64), expect)
    assert abs(float(so[0]) - abs(2.0 * sv) / 127) <= 1e-7 * abs(2.0 * sv) / 127
    # Tiny rows keep the plain rule (no threshold of their own): all of a row's y share
    # the factor silu(g) when the gate is constant, so y / max|y| = u / max|u| and the
    # codes are -rint(127 u / max u) up to near-ties.  g = -50: max|y| = 50 e^-50 u_max
    # ~ 1e-20 and g = -45: ~ 1.3e-18, both far above 2^-121, are live rows; g = -90 with
    # u = 8: max|y| = 720 e^-90 ~ 5.9e-37 >= 127 / (2^128 - 2^104) ~ 3.7e-37, live, and
    # s_a = max|y| / 127 ~ 4.6e-39 lies in the fp32 subnormal range; g = -90 with u <= 1:
    # max|y| <= 90 e^-90 ~ 7.4e-38, where fp32(127 / max|y|) overflows: a zero row.
    lo = np.zeros((4, 2 * I), F16)
    lo[0, :I] = -50.0
    lo[1, :I] = -45.0
    lo[2, :I] = -90.0
    lo[3, :I] = -90.0
    lo[:2, I:] = rng.uniform(0.5, 1.0, size=(2, I)).astype(F16)
    lo[:2, I + 3] = 1.0
    lo[2, I:] = rng.uniform(4.0, 8.0, size=I).astype(F16)
    lo[2, I + 5] = 8.0
    lo[3, I:] = rng.uniform(0.5, 1.0, size=I).astype(F16)
    lo[3, I + 5] = 1.0
    xl, sl, _ = ora.silu_mul_quant_ref(lo)
    for m, gv in ((0, -50.0), (1, -45.0), (2, -90.0)):
        u = lo[m, I:].astype(F64)
        amax = abs(gv) / (1.0 + np.exp(-gv)) * u.max()
        assert abs(float(sl[m]) - amax / 127) <= 1e-6 * amax / 127, (m, float(sl[m]), amax / 127)
        target = 127.0 * u / u.max()
        assert np.all(xl[m] < 0) and xl[m].min() == -127
        assert np.all(np.abs(xl[m].astype(F64) + target) <= 0.5 + 1e-5)
    assert 0.0 < float(sl[2]) < np.finfo(F32).tiny
    assert float(sl[3]) == 1.0 and not xl[3].any()


# ------------------------------------------------------- W4A16 variants
def pin_variants_worked(ora):
    """Hand-worked per-channel and symmetric rows (tests/golden/w4a16_variants_worked.txt)."""
    for case in read_variant_cases():
        quant = ora.quantize_sym if case["rule"] == "sym" else ora.quantize_asym
        codes, sc, z = quant(case["values"][None, :], case["group"])
        assert sc[0].view(np.uint16).tolist() == case["scales"].view(np.uint16).tolist(), case["name"]
        assert z[0].tolist() == case["zeros"], case["name"]
        for b, head in enumerate(case.get("codes_head", [])):
            assert codes[0, 128 * b:128 * b + len(head)].tolist() == head, (case["name"], b)
        for k, c in case.get("codes_at", {}).items():
            assert int(codes[0, k]) == c, (case["name"], k)


def pin_sym_properties(ora):
    """Symmetric rule: codes in [1, 15] (|w| / s <= 7 (1 + 2^-11) never rounds past 7),
    |w - (code - 8) s| <= s / 2, negating W maps every code c to 16 - c with the same
    scales (rint is odd), and zeros are 8; per-channel is one scale per row."""
    rng = _rng(41)
    w = (rng.standard_normal((24, 512)) * 0.02).astype(F16)
    w[3, 17] = 0.3
    for G in (128, -1):
        c, sc, z = ora.quantize_sym(w, G)
        assert c.min() >= 1 and c.max() <= 15 and np.all(z == 8)
        Gk = 512 if G == -1 else G
        sv = np.repeat(sc.astype(F64), Gk, axis=1)
        assert np.all(np.abs(w.astype(F64) - (c.astype(F64) - 8) * sv) <= sv / 2 + 1e-12)
        cn, scn, _ = ora.quantize_sym(-w, G)
        assert np.array_equal(cn.astype(np.int64), 16 - c.astype(np.int64)) and np.array_equal(scn, sc)
        assert sc.shape == (24, 512 // Gk)


def pin_variants_constructed_exact(ora):
    """Weights q * 2^-6 with q in [-7, 7] and each group (or row) holding +-7 come back
    exactly from the symmetric rule (s = fp16(7 * 2^-6 / 7) = 2^-6), and asymmetric
    per-channel weights (c - z) * 2^-4 with each row spanning codes 0..15 come back
    exactly; X of small integers then gives exact outputs through the whole chain."""
    rng = _rng(43)
    M, N, K = 3, 16, 384
    x = rng.integers(-4, 5, size=(M, K)).astype(F16)
    q = rng.integers(-7, 8, size=(N, K))
    q[:, ::128] = 7
    w = (q * 2.0**-6).astype(F16)
    for G in (128, -1):
        ref = ora.awq_reference(w, x, G, symmetric=True)
        exact = x.astype(np.int64) @ q.T
        assert np.array_equal(ref["y"] * 64, exact.astype(F64)), G
    z = rng.integers(0, 16, size=N)
    c = rng.integers(0, 16, size=(N, K))
    c[:, 0] = 0
    c[:, 1] = 15
    c = np.minimum(np.maximum(c, 0), 15)
    w2 = ((c - z[:, None]) * 2.0**-4).astype(F16)
    ref2 = ora.awq_reference(w2, x, -1)
    assert np.array_equal(ref2["y"] * 16, (x.astype(np.int64) @ (c - z[:, None]).T).astype(F64))
    assert ref2["scales"].shape == (1, N) and ref2["qzeros"].shape == (1, 2)


# ----------------------------------------------------------------- W8A8
def pin_w8a8_worked(ora):
    """The first level of the hand-worked two-level row TL (tests/golden/w4a8_worked.txt)
    is the W8A8 rule: s = 0x2008 and codes 127, 6, -13 | 32."""
    case = [c for c in read_cases("w4a8_worked.txt") if c["name"] == "TL"][0]
    q, s = ora.quantize_w8a8(case["values"][None, :])
    assert s[0].view(np.uint16) == case["cscale"].view(np.uint16)
    assert q[0, :3].tolist() == [127, 6, -13] and q[0, 128] == 32 and not q[0, 3:128].any()


def pin_w8a8_tile_layout(ora):
    """Tiled int8 order: a single code placed at (n, k) lands at the flat byte offset
    computed by hand from the layout rule, with kc = (k % 128) / 16,
    ((n/16 * K/128 + k/128) * 4 + kc % 4) * 512 + (kc / 4) * 256 + (n % 16) * 16 + k % 16;
    tile/untile are inverse bijections; pad rows are 0."""
    N, K = 37, 256
    for (n, k, c) in ((17, 200, 9), (0, 0, -127), (36, 255, 1), (15, 127, 64), (16, 128, -3)):
        q = np.zeros((N, K), np.int8)
        q[n, k] = c
        flat = ora.tile_w8a8(q).reshape(-1)
        kc = (k % 128) // 16
        off = ((n // 16 * (K // 128) + k // 128) * 4 + kc % 4) * 512 + (kc // 4) * 256 + (n % 16) * 16 + k % 16
        assert flat.size == 48 * K
        assert int(flat[off]) == c and np.count_nonzero(flat) == 1, (n, k)
    rng = _rng(7)
    q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    t = ora.tile_w8a8(q)
    assert t.shape == (3, 2, 4, 2, 16, 16)
    assert np.array_equal(ora.untile_w8a8(t, N), q)
    assert not ora.untile_w8a8(t, 48)[N:].any()


def pin_w8a8_properties(ora):
    """Codes in [-127, 127], |w - q s| <= s / 2, the row maximum maps to +-127, negating
    W negates the codes; with w = q' 2^-7 and each row holding +-127 the codes are q'
    exactly, so the integer accumulator is the exact product."""
    rng = _rng(51)
    w = (rng.standard_normal((40, 640)) * 0.02).astype(F16)
    q, s = ora.quantize_w8a8(w)
    sv = s.astype(F64)[:, None]
    assert q.min() >= -127 and q.max() <= 127
    assert np.all(np.abs(w.astype(F64) - q * sv) <= sv / 2 + 1e-12)
    am = np.argmax(np.abs(w.astype(F64)), axis=1)
    assert np.all(np.abs(q[np.arange(40), am]) == 127)
    qn, sn = ora.quantize_w8a8(-w)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    qp = rng.integers(-127, 128, size=(16, 256))
    qp[:, 5] = -127
    q2, s2 = ora.quantize_w8a8((qp * 2.0**-7).astype(F16))
    assert np.all(s2.astype(F64) == 2.0**-7) and np.array_equal(q2.astype(np.int64), qp)
    xq = rng.integers(-127, 128, size=(3, 256))
    assert np.array_equal(ora.w4a8_acc_ref(xq, q2, None, 128), xq @ qp.T)


def pin_w4a8_acc_bruteforce(ora):
    """Integer accumulators against Python-int loops, both weight variants."""
    rng = _rng(31)
    M, N, K, G = 3, 7, 256, 128
    xq = rng.integers(-127, 128, size=(M, K))
    for group in (-1, G):
        w = synth.make_linear(0, N, K, seed=13, outliers=True).w.numpy()
        q, cs, gs = ora.quantize_w4a8(w, group)
        qw, cs2, gs_gn = ora.pack_w4a8(q, cs, gs)
        qq = ora.unpack_w4a8(qw, N, K)
        assert np.array_equal(qq, q.astype(np.int64))
        acc = ora.w4a8_acc_ref(xq.astype(np.int8), qq, gs, G)
        for m in range(M):
            for n in range(N):
                tot = 0
                for k in range(K):
                    sgk = 1 if gs is None else int(gs_gn[k // G, n])
                    tot += int(xq[m, k]) * int(q[n, k]) * sgk
                assert int(acc[m, n]) == tot
        sa = np.array([0.5, 0.375, 3.0], F32)
        y = ora.w4a8_linear_ref(acc, sa, cs2)
        for m in range(M):
            for n in range(N):
                assert Fraction(float(y[m, n])) == int(acc[m, n]) * Fraction(float(sa[m])) * Fraction(float(cs2[n]))


ALL_PINS = [
    pin_pack_words, pin_pack_bijection, pin_parity_words, pin_halves_words, pin_tile_layout,
    pin_asym_worked, pin_asym_constructed, pin_asym_roundtrip_bound,
    pin_fraction_bruteforce, pin_identity_probe, pin_per_channel_special_case,
    pin_constructed_exact_gemm,
    pin_w4a8_worked, pin_w4a8_exhaustive, pin_quant_act_closed_forms, pin_w4a8_acc_bruteforce,
    pin_silu_worked, pin_silu_closed_forms, pin_silu_special_cases,
    pin_variants_worked, pin_sym_properties, pin_variants_constructed_exact,
    pin_w8a8_worked, pin_w8a8_properties, pin_w8a8_tile_layout,
]
