"""CPU: the C-ABI library loads, exports every symbol include/w4a16.h declares, and
rejects invalid arguments before touching a device (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import w4a16_gemm_amd as w4
    if not os.path.exists(w4.lib_path()):
        pytest.fail("libw4a16.so is not built: run python -m w4a16_gemm_amd.build")
    return w4.load()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("awq_pack", "awq_gemm", "w4a8_quant_act", "w4a8_gemm", "awq_unpack_dequant", "w4a8_pack",
              "w4a8_gemm_i32", "awq_gemm_workspace_bytes", "w4a8_gemm_workspace_bytes", "w4_status_string",
              "w4_last_error", "w4_pack_codes", "w4a8_silu_mul_quant", "awq_pack_sym", "w8a8_pack", "w8a8_gemm",
              "w8a8_gemm_i32", "w8a8_gemm_workspace_bytes", "awq_import_plain", "w4a8_import_plain"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.w4_status_string(0) == b"W4_OK"
    assert lib.w4_status_string(3) == b"W4_ERR_WORKSPACE"
    assert lib.w4_status_string(99) == b"W4_ERR_UNKNOWN"


FAKE = 0x10000  # a non-NULL, 16-byte aligned address that is never dereferenced


@pytest.mark.parametrize("args,code,msg", [
    ((None, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 64, 256, 128, None), 1, "x is NULL"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 64, 200, 128, None), 1, "multiple of 128"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 64, 0, 128, None), 1, "multiple of 128"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, -1, 64, 256, 128, None), 1, "negative"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 64, 256, 16, None), 2, "group_size"),
    ((FAKE + 4, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 64, 256, 128, None), 1, "aligned"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 64, 1 << 31, 128, None), 2, "2^30"),
    # a narrow-N shape splits K and needs a workspace (per-channel alike)
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 1, 256, 5120, 128, None), 3, "workspace"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 1, 256, 5120, -1, None), 3, "workspace"),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 64, 256, 0, None), 2, "group_size"),
])
def test_awq_gemm_validation(lib, args, code, msg):
    P = ctypes.c_void_p
    conv = [P(a) if (i < 6 and a is not None) else a for i, a in enumerate(args)]
    assert lib.awq_gemm(*conv) == code
    assert msg in lib.w4_last_error().decode()


def test_empty_shapes_are_noops(lib):
    # M == 0 or N == 0 return OK before any pointer or device check
    assert lib.awq_gemm(None, None, None, None, None, None, 0, 0, 64, 256, 128, None) == 0
    assert lib.awq_gemm(None, None, None, None, None, None, 0, 4, 0, 256, 128, None) == 0
    assert lib.w4a8_gemm(None, None, None, None, None, None, None, 0, 0, 64, 256, -1, None) == 0
    assert lib.w4a8_quant_act(None, None, ctypes.c_float(1e-5), None, None, 0, 0, 256, 0, None) == 0
    assert lib.w4a8_silu_mul_quant(None, None, None, 0, 0, 256, 0, None) == 0


def test_pack_codes_validation(lib):
    P = ctypes.c_void_p
    assert lib.w4_pack_codes(None, None, 0, 5, None) == 0  # empty: no pointer or device check
    assert lib.w4_pack_codes(P(FAKE), P(FAKE), -1, 8, None) == 1
    assert "negative" in lib.w4_last_error().decode()
    assert lib.w4_pack_codes(None, P(FAKE), 3, 8, None) == 1
    assert "codes is NULL" in lib.w4_last_error().decode()
    assert lib.w4_pack_codes(P(FAKE), P(FAKE + 4), 3, 8, None) == 1
    assert "aligned" in lib.w4_last_error().decode()


def test_w4a8_validation(lib):
    P = ctypes.c_void_p
    f = P(FAKE)
    # gscale must be NULL for per-channel and non-NULL for g128
    assert lib.w4a8_gemm(f, f, f, f, f, f, None, 0, 4, 64, 256, -1, None) == 1
    assert "gscale" in lib.w4_last_error().decode()
    assert lib.w4a8_gemm(f, f, f, None, f, f, None, 0, 4, 64, 256, 128, None) == 1
    assert lib.w4a8_gemm(f, f, f, None, f, f, None, 0, 4, 64, 256, 32, None) == 2
    assert lib.w4a8_quant_act(f, None, ctypes.c_float(1e-5), f, f, 4, 0, 100, 0, None) == 1
    assert lib.w4a8_quant_act(f, None, ctypes.c_float(-1.0), f, f, 4, 0, 128, 0, None) == 1
    assert lib.w4a8_silu_mul_quant(f, f, f, 4, 0, 100, 0, None) == 1
    assert "multiple of 8" in lib.w4_last_error().decode()
    assert lib.w4a8_silu_mul_quant(f, f, f, -1, 0, 128, 0, None) == 1
    assert lib.w4a8_silu_mul_quant(f, None, f, 4, 0, 128, 0, None) == 1
    assert "xq is NULL" in lib.w4_last_error().decode()
    assert lib.w4a8_silu_mul_quant(f, f, f, 4, 0, 1 << 30, 0, None) == 2
    assert lib.w4a8_pack(f, f, None, f, 0, 64, 256, 128, None) == 1
    assert lib.awq_pack(f, f, f, f, 0, 64, 256, 16, None) == 2
    assert lib.awq_pack_sym(f, f, f, f, 0, 64, 256, 16, None) == 2
    assert "group_size" in lib.w4_last_error().decode()
    assert lib.awq_pack_sym(f, None, f, f, 0, 64, 256, -1, None) == 1
    assert "qweight is NULL" in lib.w4_last_error().decode()
    assert lib.awq_pack_sym(None, None, None, None, 0, 0, 256, -1, None) == 0
    assert lib.awq_unpack_dequant(f, f, f, f, 64, 200, -1, None) == 1
    assert lib.w8a8_pack(f, f, f, 0, 64, 256, 128, None) == 2
    assert lib.w8a8_pack(f, f, None, 0, 64, 256, -1, None) == 1
    assert "cscale is NULL" in lib.w4_last_error().decode()
    assert lib.w8a8_gemm(f, f, f, f, f, None, 0, 4, 64, 256, 128, None) == 2
    assert lib.w8a8_gemm(f, None, f, f, f, None, 0, 4, 64, 256, -1, None) == 1
    assert "s_a is NULL" in lib.w4_last_error().decode()
    assert lib.w8a8_gemm_i32(f, f, None, None, 0, 4, 64, 256, -1, None) == 1
    assert lib.w8a8_gemm(f, f, f, f, f, None, 0, 4, 64, 1 << 18, -1, None) == 2
    assert "131072" in lib.w4_last_error().decode()
    assert lib.w4a8_gemm(f, f, f, None, f, f, None, 0, 4, 64, 1 << 18, -1, None) == 2
    assert lib.w8a8_gemm(None, None, None, None, None, None, 0, 0, 64, 256, -1, None) == 0
    assert lib.w8a8_gemm(f, f, f, f, f, None, 0, 1, 256, 5120, -1, None) == 3  # narrow N splits K


def test_import_validation(lib):
    P = ctypes.c_void_p
    f = P(FAKE)
    assert lib.awq_import_plain(None, None, None, None, None, None, 0, 256, 128, 0, None) == 0  # N == 0
    assert lib.awq_import_plain(f, f, f, f, f, f, 64, 256, 128, 2, None) == 1
    assert "layout" in lib.w4_last_error().decode()
    assert lib.awq_import_plain(f, f, None, f, f, f, 64, 256, 128, 1, None) == 1
    assert "qzeros_plain is NULL" in lib.w4_last_error().decode()
    assert lib.awq_import_plain(f, f, f, f, f, P(FAKE + 2), 64, 256, 128, 0, None) == 1
    assert "aligned" in lib.w4_last_error().decode()
    assert lib.awq_import_plain(f, f, f, f, f, f, 64, 200, 128, 0, None) == 1
    assert lib.awq_import_plain(f, f, f, f, f, f, 64, 256, 16, 0, None) == 2
    assert lib.w4a8_import_plain(f, f, f, f, 64, 256, -1, 0, None) == 1
    assert "gscale" in lib.w4_last_error().decode()
    assert lib.w4a8_import_plain(f, None, f, f, 64, 256, 128, 0, None) == 1
    assert "gscale_plain is NULL" in lib.w4_last_error().decode()
    assert lib.w4a8_import_plain(f, None, f, None, 64, 256, 64, 0, None) == 2
    assert lib.w4a8_import_plain(f, None, f, None, -1, 256, -1, 0, None) == 1


def test_workspace_sizes(lib):
    # empty shapes need no workspace (and are never planned)
    for fn in (lib.awq_gemm_workspace_bytes, lib.w4a8_gemm_workspace_bytes):
        assert fn(0, 64, 256, -1) == 0 and fn(4, 0, 256, -1) == 0 and fn(0, 0, 256, 128) == 0
    assert lib.w8a8_gemm_workspace_bytes(0, 64, 256, -1) == 0 and lib.w8a8_gemm_workspace_bytes(4, 0, 256, -1) == 0
    # decode shapes split K; prefill shapes do not; invalid shapes report 0
    assert lib.awq_gemm_workspace_bytes(1, 256, 5120, 128) > 0
    assert lib.awq_gemm_workspace_bytes(4096, 27648, 5120, 128) == 0
    assert lib.awq_gemm_workspace_bytes(16, 5120, 200, 128) == 0
    assert lib.awq_gemm_workspace_bytes(1, 256, 5120, -1) == lib.awq_gemm_workspace_bytes(1, 256, 5120, 128)
    assert lib.awq_gemm_workspace_bytes(1, 256, 5120, 16) == 0
    # group sizes 64 and 32 take the MFMA GEMM at every M (its own split-K plan)
    assert lib.awq_gemm_workspace_bytes(1, 256, 5120, 64) == lib.awq_gemm_workspace_bytes(1, 256, 5120, 32) > 0
    assert lib.w8a8_gemm_workspace_bytes(1, 256, 5120, -1) > 0
    assert lib.w8a8_gemm_workspace_bytes(1, 256, 5120, 128) == 0
    assert lib.w8a8_gemm_workspace_bytes(1, 256, 1 << 18, -1) == 0
    assert lib.w4a8_gemm_workspace_bytes(1, 256, 5120, -1) > 0  # narrow N splits K
    assert lib.w4a8_gemm_workspace_bytes(4096, 13824, 5120, 128) == 0


def test_plans_of_many_shapes(lib):
    """The tile planners run on the host for every call: seeded shapes over every dispatch
    boundary, group size and K must plan without a host fault and report a workspace
    that covers the counter region whenever K is split."""
    import numpy as np
    rng = np.random.default_rng(7)
    Ms = [1, 2, 3, 4, 5, 8, 9, 16, 17, 31, 32, 33, 48, 64, 65, 128, 129, 255, 256, 257, 511, 512, 513, 4096, 5000]
    for _ in range(600):
        M = int(rng.choice(Ms))
        N = int(rng.integers(1, 40000))
        K = 128 * int(rng.integers(1, 120))
        for g in (128, 64, 32, -1):
            b = lib.awq_gemm_workspace_bytes(M, N, K, g)
            assert b == 0 or b >= 16384
        for g in (128, -1):
            b = lib.w4a8_gemm_workspace_bytes(M, N, K, g)
            assert b == 0 or b >= 16384
        b = lib.w8a8_gemm_workspace_bytes(M, N, K, -1)
        assert b == 0 or b >= 16384
