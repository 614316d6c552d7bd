"""ctypes binding of ``libw4a16.so`` (the C ABI declared in ``include/w4a16.h``).

Argument marshalling only: every function checks dtypes, devices, shapes and
contiguity, allocates its outputs (and, where a kernel splits K, a cached
zero-filled workspace) with torch on the input's device, and calls the C entry
point of the same name on torch's current stream.  All computation happens in the
HIP kernels; there is no CPU or PyTorch fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

W4_OK = 0
_lib = None
_lock = threading.Lock()


class W4Error(RuntimeError):
    """A non-zero status returned by the C library."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib_path() -> str:
    return LIB_PATH


def load():
    """Load (once) and return the ctypes handle of libw4a16.so."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m w4a16_gemm_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        sig = {
            "awq_pack": [P, P, P, P, I64, I64, I64, I32, P],
            "awq_pack_sym": [P, P, P, P, I64, I64, I64, I32, P],
            "awq_unpack_dequant": [P, P, P, P, I64, I64, I32, P],
            "awq_gemm": [P, P, P, P, P, P, SZ, I64, I64, I64, I32, P],
            "w4a8_pack": [P, P, P, P, I64, I64, I64, I32, P],
            "w4a8_quant_act": [P, P, F, P, P, I64, I64, I64, I32, P],
            "w4a8_silu_mul_quant": [P, P, P, I64, I64, I64, I32, P],
            "w4a8_gemm": [P, P, P, P, P, P, P, SZ, I64, I64, I64, I32, P],
            "w4a8_gemm_i32": [P, P, P, P, P, SZ, I64, I64, I64, I32, P],
            "w4_pack_codes": [P, P, I64, I64, P],
            "w8a8_pack": [P, P, P, I64, I64, I64, I32, P],
            "w8a8_gemm": [P, P, P, P, P, P, SZ, I64, I64, I64, I32, P],
            "w8a8_gemm_i32": [P, P, P, P, SZ, I64, I64, I64, I32, P],
            "awq_import_plain": [P, P, P, P, P, P, I64, I64, I32, I32, P],
            "w4a8_import_plain": [P, P, P, P, I64, I64, I32, I32, P],
            "awq_gemm_noalloc": [P, P, P, P, P, I64, I64, I64, I32, P],
            "w4_ceiling_read": [P, I64, P, I32, I32, P],
            "w4_ceiling_mfma": [P, I64, I32, I32, P, I32, P],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        for name in ("awq_gemm_workspace_bytes", "w4a8_gemm_workspace_bytes", "w8a8_gemm_workspace_bytes"):
            fn = getattr(lib, name)
            fn.argtypes = [I64, I64, I64, I32]
            fn.restype = ctypes.c_size_t
        lib.w4_status_string.argtypes = [ctypes.c_int]
        lib.w4_status_string.restype = ctypes.c_char_p
        lib.w4_last_error.argtypes = []
        lib.w4_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(fn: str, status: int):
    if status != W4_OK:
        lib = load()
        raise W4Error(fn, status, f"{lib.w4_status_string(status).decode()}: {lib.w4_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype, shape=None, ndim=None):
    """Type, dtype, rank, shape and contiguity of one tensor argument.  Devices are
    checked afterwards by :func:`_gpu`, so that every shape of a call is validated
    before anything else (and before any C call)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is None and shape is not None:
        ndim = len(shape)
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gpu(**tensors):
    """All given tensors (None entries skipped) on one GPU device; returns it."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    return dev


def _groups(K: int, group_size: int, allowed) -> int:
    """Rows of the scale / zero-point arrays (K / G; 1 per-channel)."""
    if group_size not in allowed:
        raise ValueError(f"group_size={group_size} is not one of {sorted(allowed)}")
    if K <= 0 or K % 128:
        raise ValueError(f"K={K} must be a positive multiple of 128")
    return 1 if group_size == -1 else K // group_size


W4A16_GROUPS = (128, 64, 32, -1)
W4A8_GROUPS = (128, -1)


# Workspaces: one zero-filled buffer per (device, stream), grown on demand.  The
# kernels leave its counter region zeroed after every completed call, so it can be
# reused by later calls on the same stream.
_ws_cache: dict = {}


def _workspace(dev, nbytes: int):
    if nbytes == 0:
        return None, 0
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf, buf.numel()


def qweight_shape(N: int, K: int):
    """Shape of the tiled packed weights: int32 [ceil(N/16), K/128, 4, 16, 4] -- 1 KB
    blocks of 16 rows x 128 k; word j of row n at [n//16, j//16, (j%16)//4, n%16, j%4]."""
    return ((N + 15) // 16, K // 128, 4, 16, 4)


def _need_qweight(qweight, N, K):
    _need(qweight, "qweight", torch.int32, qweight_shape(N, K))


def _need_w4a16(qweight, scales, qzeros, N, K, group_size):
    """qweight, scales [K/G, N] and qzeros [K/G, ceil(N/8)] of an N x K W4A16 matrix."""
    ng = _groups(K, group_size, W4A16_GROUPS)
    _need_qweight(qweight, N, K)
    _need(scales, "scales", torch.float16, (ng, N))
    _need(qzeros, "qzeros", torch.int32, (ng, (N + 7) // 8))


# ------------------------------------------------------------------ W4A16
def awq_pack(w: torch.Tensor, group_size: int = 128):
    """fp16 W [N, K] -> (qweight int32 [ceil(N/16), K/128, 4, 16, 4], scales fp16 [K/G, N],
    qzeros int32 [K/G, ceil(N/8)]); group_size -1: per-channel (scales [1, N])."""
    return _pack_w4a16("awq_pack", w, group_size)


def awq_pack_sym(w: torch.Tensor, group_size: int = 128):
    """As awq_pack with the symmetric rule (codes q + 8, zero points 8)."""
    return _pack_w4a16("awq_pack_sym", w, group_size)


def _pack_w4a16(name, w, group_size):
    _need(w, "w", torch.float16, ndim=2)
    N, K = w.shape
    _groups(K, group_size, W4A16_GROUPS)
    dev = _gpu(w=w)
    G = group_size if group_size > 0 else K
    qweight = torch.empty(qweight_shape(N, K), dtype=torch.int32, device=dev)
    scales = torch.empty((K // G, N), dtype=torch.float16, device=dev)
    qzeros = torch.empty((K // G, (N + 7) // 8), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        _check(name, getattr(load(), name)(_ptr(w), _ptr(qweight), _ptr(scales), _ptr(qzeros), 0, N, K,
                                           group_size, _stream(dev)))
    return qweight, scales, qzeros


def w4_pack_codes(codes):
    """uint8 codes [R, C] (values 0..15) -> int32 [R, ceil(C/8)], plain nibble order."""
    _need(codes, "codes", torch.uint8, ndim=2)
    dev = _gpu(codes=codes)
    R, C = codes.shape
    out = torch.empty((R, (C + 7) // 8), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        _check("w4_pack_codes", load().w4_pack_codes(_ptr(codes), _ptr(out), R, C, _stream(dev)))
    return out


def awq_unpack_dequant(qweight, scales, qzeros, group_size: int = 128):
    """Packed weights -> fp16 W_deq [N, K] = fp16((q - z) * s)."""
    _need(scales, "scales", torch.float16, ndim=2)
    _need(qweight, "qweight", torch.int32, ndim=5)
    N, K = scales.shape[1], qweight.shape[1] * 128
    _need_w4a16(qweight, scales, qzeros, N, K, group_size)
    dev = _gpu(qweight=qweight, scales=scales, qzeros=qzeros)
    out = torch.empty((N, K), dtype=torch.float16, device=dev)
    with torch.cuda.device(dev):
        _check("awq_unpack_dequant", load().awq_unpack_dequant(_ptr(qweight), _ptr(scales), _ptr(qzeros), _ptr(out),
                                                               N, K, group_size, _stream(dev)))
    return out


LAYOUTS = {"rows": 0, "cols": 1}


def _plain_dims(qweight_plain, layout):
    """(N, K) of plain packed words: rows [N, K/8], cols [K/8, N]."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}, got {layout!r}")
    _need(qweight_plain, "qweight_plain", torch.int32, ndim=2)
    a, b = qweight_plain.shape
    return (a, 8 * b) if layout == "rows" else (b, 8 * a)


def _plain_groups(t, name, dtype, N, rows_per_n, layout):
    _need(t, name, dtype, (N, rows_per_n) if layout == "rows" else (rows_per_n, N))


def awq_import_plain(qweight_plain, scales_plain, qzeros_plain, group_size: int = 128, layout: str = "rows"):
    """Plain W4A16 weights -> (qweight tiled, scales [K/G, N], qzeros [K/G, ceil(N/8)]).
    layout "rows": qweight [N, K/8], scales [N, K/G], qzeros [N, ceil(K/G/8)]; "cols" (the
    K-major Triton AWQ orientation): qweight [K/8, N], scales [K/G, N], qzeros
    [ceil(K/G/8), N]."""
    N, K = _plain_dims(qweight_plain, layout)
    ng = _groups(K, group_size, W4A16_GROUPS)
    _plain_groups(scales_plain, "scales_plain", torch.float16, N, ng, layout)
    _plain_groups(qzeros_plain, "qzeros_plain", torch.int32, N, (ng + 7) // 8, layout)
    dev = _gpu(qweight_plain=qweight_plain, scales_plain=scales_plain, qzeros_plain=qzeros_plain)
    qweight = torch.empty(qweight_shape(N, K), dtype=torch.int32, device=dev)
    scales = torch.empty((ng, N), dtype=torch.float16, device=dev)
    qzeros = torch.empty((ng, (N + 7) // 8), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        _check("awq_import_plain", load().awq_import_plain(
            _ptr(qweight_plain), _ptr(scales_plain), _ptr(qzeros_plain), _ptr(qweight), _ptr(scales), _ptr(qzeros),
            N, K, group_size, LAYOUTS[layout], _stream(dev)))
    return qweight, scales, qzeros


def awq_gemm_workspace_bytes(M: int, N: int, K: int, group_size: int = 128) -> int:
    return int(load().awq_gemm_workspace_bytes(M, N, K, group_size))


def awq_gemm(x, qweight, scales, qzeros, group_size: int = 128, out=None, workspace=None):
    """Y [M, N] = X [M, K] . dequant(W)^T  (fp16 in, fp16 out, fp32 accumulate)."""
    _need(x, "x", torch.float16, ndim=2)
    _need(scales, "scales", torch.float16, ndim=2)
    M, K = x.shape
    N = scales.shape[1]
    _need_w4a16(qweight, scales, qzeros, N, K, group_size)
    if out is not None:
        _need(out, "out", torch.float16, (M, N))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, ndim=1)
    dev = _gpu(x=x, qweight=qweight, scales=scales, qzeros=qzeros, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
    lib = load()
    with torch.cuda.device(dev):
        if workspace is None:
            ws, nb = _workspace(dev, lib.awq_gemm_workspace_bytes(M, N, K, group_size))
        else:
            ws, nb = workspace, workspace.numel() * workspace.element_size()
        _check("awq_gemm", lib.awq_gemm(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(qzeros), _ptr(out), _ptr(ws),
                                        nb, M, N, K, group_size, _stream(dev)))
    return out


def awq_gemm_noalloc(x, qweight, scales, qzeros, out, group_size: int = 128):
    """awq_gemm on the library's static device workspace (no allocation anywhere: the
    output is the caller's).  Raises W4Error (W4_ERR_WORKSPACE) for a shape whose
    workspace exceeds the static array."""
    _need(x, "x", torch.float16, ndim=2)
    _need(scales, "scales", torch.float16, ndim=2)
    M, K = x.shape
    N = scales.shape[1]
    _need_w4a16(qweight, scales, qzeros, N, K, group_size)
    _need(out, "out", torch.float16, (M, N))
    dev = _gpu(x=x, qweight=qweight, scales=scales, qzeros=qzeros, out=out)
    with torch.cuda.device(dev):
        _check("awq_gemm_noalloc", load().awq_gemm_noalloc(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(qzeros),
                                                           _ptr(out), M, N, K, group_size, _stream(dev)))
    return out


# ------------------------------------------------------------------- W4A8
def w4a8_pack(w: torch.Tensor, group_size: int = -1):
    """fp16 W [N, K] -> (qweight int32 [ceil(N/16), K/128, 4, 16, 4] of biased nibbles,
    gscale int8 [K/G, N] or None, cscale fp16 [N])."""
    _need(w, "w", torch.float16, ndim=2)
    N, K = w.shape
    _groups(K, group_size, W4A8_GROUPS)
    dev = _gpu(w=w)
    qweight = torch.empty(qweight_shape(N, K), dtype=torch.int32, device=dev)
    cscale = torch.empty((N,), dtype=torch.float16, device=dev)
    gscale = torch.empty((K // group_size, N), dtype=torch.int8, device=dev) if group_size > 0 else None
    with torch.cuda.device(dev):
        _check("w4a8_pack", load().w4a8_pack(_ptr(w), _ptr(qweight), _ptr(gscale), _ptr(cscale), 0, N, K,
                                             group_size, _stream(dev)))
    return qweight, gscale, cscale


def w4a8_import_plain(qweight_plain, gscale_plain=None, group_size: int = -1, layout: str = "rows"):
    """Plain W4A8 weights (biased nibbles q + 8) -> (qweight tiled, gscale [K/G, N] or
    None).  layout "rows": qweight [N, K/8], gscale [N, K/G]; "cols": [K/8, N], [K/G, N]."""
    N, K = _plain_dims(qweight_plain, layout)
    ng = _groups(K, group_size, W4A8_GROUPS)
    if group_size == -1:
        if gscale_plain is not None:
            raise ValueError("gscale_plain must be None for per-channel weights (group_size -1)")
    else:
        if gscale_plain is None:
            raise ValueError("gscale_plain is required for group_size 128")
        _plain_groups(gscale_plain, "gscale_plain", torch.int8, N, ng, layout)
    dev = _gpu(qweight_plain=qweight_plain, gscale_plain=gscale_plain)
    qweight = torch.empty(qweight_shape(N, K), dtype=torch.int32, device=dev)
    gscale = torch.empty((ng, N), dtype=torch.int8, device=dev) if group_size > 0 else None
    with torch.cuda.device(dev):
        _check("w4a8_import_plain", load().w4a8_import_plain(
            _ptr(qweight_plain), _ptr(gscale_plain), _ptr(qweight), _ptr(gscale), N, K, group_size,
            LAYOUTS[layout], _stream(dev)))
    return qweight, gscale


def w4a8_quant_act(x: torch.Tensor, gamma=None, eps: float = 1e-5):
    """fp16 X [M, K] (and optional RMSNorm gamma [K]) -> (xq int8 [M, K], s_a fp32 [M])."""
    _need(x, "x", torch.float16, ndim=2)
    M, K = x.shape
    if gamma is not None:
        _need(gamma, "gamma", torch.float16, (K,))
    dev = _gpu(x=x, gamma=gamma)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    s_a = torch.empty((M,), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check("w4a8_quant_act", load().w4a8_quant_act(_ptr(x), _ptr(gamma), float(eps), _ptr(xq), _ptr(s_a), M, 0,
                                                       K, 0, _stream(dev)))
    return xq, s_a


def w4a8_silu_mul_quant(gate_up: torch.Tensor):
    """fp16 fused gate+up output [M, 2I] (gate columns first) -> (xq int8 [M, I] of
    silu(gate) * up, s_a fp32 [M])."""
    _need(gate_up, "gate_up", torch.float16, ndim=2)
    M, K2 = gate_up.shape
    if K2 % 2:
        raise ValueError("gate_up must have an even number of columns")
    dev = _gpu(gate_up=gate_up)
    xq = torch.empty((M, K2 // 2), dtype=torch.int8, device=dev)
    s_a = torch.empty((M,), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check("w4a8_silu_mul_quant", load().w4a8_silu_mul_quant(_ptr(gate_up), _ptr(xq), _ptr(s_a), M, 0,
                                                                 K2 // 2, 0, _stream(dev)))
    return xq, s_a


def w4a8_gemm_workspace_bytes(M: int, N: int, K: int, group_size: int = -1) -> int:
    return int(load().w4a8_gemm_workspace_bytes(M, N, K, group_size))


def _w4a8_args(xq, qweight, gscale, group_size, N):
    """Shapes of the integer operands: xq [M, K], tiled qweight, gscale [K/G, N] for the
    two-level format (group_size 128) and None per-channel (-1)."""
    _need(xq, "xq", torch.int8, ndim=2)
    M, K = xq.shape
    ng = _groups(K, group_size, W4A8_GROUPS)
    _need_qweight(qweight, N, K)
    if group_size == -1:
        if gscale is not None:
            raise ValueError("gscale must be None for per-channel weights (group_size -1)")
    else:
        if gscale is None:
            raise ValueError("gscale is required for group_size 128")
        _need(gscale, "gscale", torch.int8, (ng, N))
    return M, N, K


def _w4a8_scales(s_a, cscale, out, M, N):
    _need(s_a, "s_a", torch.float32, (M,))
    _need(cscale, "cscale", torch.float16, (N,))
    if out is not None:
        _need(out, "out", torch.float16, (M, N))


def w4a8_gemm(xq, s_a, qweight, gscale, cscale, group_size: int = -1, out=None):
    """Y [M, N] = fp16(acc * s_a[m] * cscale[n]), acc the exact int32 sum of xq * q * s_g."""
    _need(cscale, "cscale", torch.float16, ndim=1)
    M, N, K = _w4a8_args(xq, qweight, gscale, group_size, cscale.shape[0])
    _w4a8_scales(s_a, cscale, out, M, N)
    dev = _gpu(xq=xq, s_a=s_a, qweight=qweight, gscale=gscale, cscale=cscale, out=out)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
    lib = load()
    with torch.cuda.device(dev):
        ws, nb = _workspace(dev, lib.w4a8_gemm_workspace_bytes(M, N, K, group_size))
        _check("w4a8_gemm", lib.w4a8_gemm(_ptr(xq), _ptr(s_a), _ptr(qweight), _ptr(gscale), _ptr(cscale), _ptr(out),
                                          _ptr(ws), nb, M, N, K, group_size, _stream(dev)))
    return out


def w4a8_gemm_i32(xq, qweight, gscale, group_size: int = -1, N: int | None = None):
    """Raw int32 accumulators acc [M, N] of w4a8_gemm (N defaults to 16 * qweight.shape[0];
    give it when N is not a multiple of 16)."""
    if N is None:
        N = 16 * qweight.shape[0]
    M, N, K = _w4a8_args(xq, qweight, gscale, group_size, N)
    dev = _gpu(xq=xq, qweight=qweight, gscale=gscale)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    lib = load()
    with torch.cuda.device(dev):
        ws, nb = _workspace(dev, lib.w4a8_gemm_workspace_bytes(M, N, K, group_size))
        _check("w4a8_gemm_i32", lib.w4a8_gemm_i32(_ptr(xq), _ptr(qweight), _ptr(gscale), _ptr(acc), _ptr(ws), nb, M,
                                                  N, K, group_size, _stream(dev)))
    return acc


def bind_awq_gemm(x, qweight, scales, qzeros, out, group_size: int = 128):
    """Validate once and return a zero-argument callable that enqueues awq_gemm on the
    current stream with pre-marshalled arguments (for tight launch loops: benchmarks,
    stream capture).  The workspace is allocated here, not at call time."""
    _need(x, "x", torch.float16, ndim=2)
    _need(scales, "scales", torch.float16, ndim=2)
    M, K = x.shape
    N = scales.shape[1]
    _need_w4a16(qweight, scales, qzeros, N, K, group_size)
    _need(out, "out", torch.float16, (M, N))
    dev = _gpu(x=x, qweight=qweight, scales=scales, qzeros=qzeros, out=out)
    lib = load()
    with torch.cuda.device(dev):
        ws, nb = _workspace(dev, lib.awq_gemm_workspace_bytes(M, N, K, group_size))
        stream = _stream(dev)
    args = (_ptr(x), _ptr(qweight), _ptr(scales), _ptr(qzeros), _ptr(out), _ptr(ws), nb, M, N, K, group_size, stream)
    fn = lib.awq_gemm
    keep = (x, qweight, scales, qzeros, out, ws)

    def call():
        rc = fn(*args)
        if rc != W4_OK:
            _check("awq_gemm", rc)
        return keep
    return call


def bind_w4a8_gemm(xq, s_a, qweight, gscale, cscale, out, group_size: int = -1):
    """As bind_awq_gemm, for w4a8_gemm."""
    _need(cscale, "cscale", torch.float16, ndim=1)
    M, N, K = _w4a8_args(xq, qweight, gscale, group_size, cscale.shape[0])
    if out is None:
        raise ValueError("out is required")
    _w4a8_scales(s_a, cscale, out, M, N)
    dev = _gpu(xq=xq, s_a=s_a, qweight=qweight, gscale=gscale, cscale=cscale, out=out)
    lib = load()
    with torch.cuda.device(dev):
        ws, nb = _workspace(dev, lib.w4a8_gemm_workspace_bytes(M, N, K, group_size))
        stream = _stream(dev)
    args = (_ptr(xq), _ptr(s_a), _ptr(qweight), _ptr(gscale), _ptr(cscale), _ptr(out), _ptr(ws), nb, M, N, K,
            group_size, stream)
    fn = lib.w4a8_gemm
    keep = (xq, s_a, qweight, gscale, cscale, out, ws)

    def call():
        rc = fn(*args)
        if rc != W4_OK:
            _check("w4a8_gemm", rc)
        return keep
    return call


def bind_w4a8_quant_act(x, gamma, xq, s_a, eps: float = 1e-5):
    """As bind_awq_gemm, for w4a8_quant_act."""
    _need(x, "x", torch.float16, ndim=2)
    M, K = x.shape
    if gamma is not None:
        _need(gamma, "gamma", torch.float16, (K,))
    _need(xq, "xq", torch.int8, (M, K))
    _need(s_a, "s_a", torch.float32, (M,))
    dev = _gpu(x=x, gamma=gamma, xq=xq, s_a=s_a)
    lib = load()
    with torch.cuda.device(dev):
        stream = _stream(dev)
    args = (_ptr(x), _ptr(gamma), ctypes.c_float(eps), _ptr(xq), _ptr(s_a), M, 0, K, 0, stream)
    fn = lib.w4a8_quant_act
    keep = (x, gamma, xq, s_a)

    def call():
        rc = fn(*args)
        if rc != W4_OK:
            _check("w4a8_quant_act", rc)
        return keep
    return call


def bind_w4a8_silu_mul_quant(gate_up, xq, s_a):
    """As bind_awq_gemm, for w4a8_silu_mul_quant."""
    _need(gate_up, "gate_up", torch.float16, ndim=2)
    M, K2 = gate_up.shape
    if K2 % 2:
        raise ValueError("gate_up must have an even number of columns")
    _need(xq, "xq", torch.int8, (M, K2 // 2))
    _need(s_a, "s_a", torch.float32, (M,))
    dev = _gpu(gate_up=gate_up, xq=xq, s_a=s_a)
    lib = load()
    with torch.cuda.device(dev):
        stream = _stream(dev)
    args = (_ptr(gate_up), _ptr(xq), _ptr(s_a), M, 0, K2 // 2, 0, stream)
    fn = lib.w4a8_silu_mul_quant
    keep = (gate_up, xq, s_a)

    def call():
        rc = fn(*args)
        if rc != W4_OK:
            _check("w4a8_silu_mul_quant", rc)
        return keep
    return call


# ------------------------------------------------------------------- W8A8
def w8a8_qweight_shape(N: int, K: int):
    """Shape of the tiled W8A8 weights: int8 [ceil(N/16), K/128, 4, 2, 16, 16]."""
    return ((N + 15) // 16, K // 128, 4, 2, 16, 16)


def w8a8_pack(w: torch.Tensor):
    """fp16 W [N, K] -> (qweight int8 tiled [ceil(N/16), K/128, 4, 2, 16, 16], cscale fp16
    [N]), per-channel."""
    _need(w, "w", torch.float16, ndim=2)
    N, K = w.shape
    _groups(K, -1, (-1,))
    dev = _gpu(w=w)
    qweight = torch.empty(w8a8_qweight_shape(N, K), dtype=torch.int8, device=dev)
    cscale = torch.empty((N,), dtype=torch.float16, device=dev)
    with torch.cuda.device(dev):
        _check("w8a8_pack", load().w8a8_pack(_ptr(w), _ptr(qweight), _ptr(cscale), 0, N, K, -1, _stream(dev)))
    return qweight, cscale


def w8a8_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().w8a8_gemm_workspace_bytes(M, N, K, -1))


def _w8a8_args(xq, qweight, N):
    _need(xq, "xq", torch.int8, ndim=2)
    M, K = xq.shape
    _groups(K, -1, (-1,))
    _need(qweight, "qweight", torch.int8, w8a8_qweight_shape(N, K))
    return M, N, K


def w8a8_gemm(xq, s_a, qweight, cscale, out=None):
    """Y [M, N] = fp16(acc * s_a[m] * cscale[n]), acc = xq . qweight^T exact in int32."""
    _need(cscale, "cscale", torch.float16, ndim=1)
    M, N, K = _w8a8_args(xq, qweight, cscale.shape[0])
    _w4a8_scales(s_a, cscale, out, M, N)
    dev = _gpu(xq=xq, s_a=s_a, qweight=qweight, cscale=cscale, out=out)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
    lib = load()
    with torch.cuda.device(dev):
        ws, nb = _workspace(dev, lib.w8a8_gemm_workspace_bytes(M, N, K, -1))
        _check("w8a8_gemm", lib.w8a8_gemm(_ptr(xq), _ptr(s_a), _ptr(qweight), _ptr(cscale), _ptr(out), _ptr(ws), nb,
                                          M, N, K, -1, _stream(dev)))
    return out


def w8a8_gemm_i32(xq, qweight, N: int):
    """The raw int32 accumulators [M, N] of w8a8_gemm."""
    M, N, K = _w8a8_args(xq, qweight, N)
    dev = _gpu(xq=xq, qweight=qweight)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    lib = load()
    with torch.cuda.device(dev):
        ws, nb = _workspace(dev, lib.w8a8_gemm_workspace_bytes(M, N, K, -1))
        _check("w8a8_gemm_i32", lib.w8a8_gemm_i32(_ptr(xq), _ptr(qweight), _ptr(acc), _ptr(ws), nb, M, N, K, -1,
                                                  _stream(dev)))
    return acc


def bind_w8a8_gemm(xq, s_a, qweight, cscale, out):
    """As bind_awq_gemm, for w8a8_gemm."""
    _need(cscale, "cscale", torch.float16, ndim=1)
    M, N, K = _w8a8_args(xq, qweight, cscale.shape[0])
    if out is None:
        raise ValueError("out is required")
    _w4a8_scales(s_a, cscale, out, M, N)
    dev = _gpu(xq=xq, s_a=s_a, qweight=qweight, cscale=cscale, out=out)
    lib = load()
    with torch.cuda.device(dev):
        ws, nb = _workspace(dev, lib.w8a8_gemm_workspace_bytes(M, N, K, -1))
        stream = _stream(dev)
    args = (_ptr(xq), _ptr(s_a), _ptr(qweight), _ptr(cscale), _ptr(out), _ptr(ws), nb, M, N, K, -1, stream)
    fn = lib.w8a8_gemm
    keep = (xq, s_a, qweight, cscale, out, ws)

    def call():
        rc = fn(*args)
        if rc != W4_OK:
            _check("w8a8_gemm", rc)
        return keep
    return call


# ------------------------------------------------------ measurement helpers
def bind_ceiling_read(buf, nbytes: int, blocks: int = 1024, unroll: int = 4):
    """Zero-argument callable that enqueues w4_ceiling_read over the first `nbytes` of
    the device buffer `buf` (a read-only HBM stream, the measured bandwidth ceiling)."""
    _need(buf, "buf", torch.uint8, ndim=1)
    if nbytes <= 0 or nbytes % 16 or nbytes > buf.numel():
        raise ValueError(f"nbytes={nbytes} must be a positive multiple of 16 within the buffer")
    dev = _gpu(buf=buf)
    sink = torch.empty((blocks * 4,), dtype=torch.int32, device=dev)
    lib = load()
    with torch.cuda.device(dev):
        stream = _stream(dev)
    args = (_ptr(buf), nbytes, _ptr(sink), blocks, unroll, stream)
    fn = lib.w4_ceiling_read
    keep = (buf, sink)

    def call():
        rc = fn(*args)
        if rc != W4_OK:
            _check("w4_ceiling_read", rc)
        return keep
    return call


def bind_ceiling_mfma(operands, kind: int, iters: int, blocks: int = 512):
    """Zero-argument callable that enqueues w4_ceiling_mfma (kind 0 fp16, 1 int8); returns
    (callable, flops per call)."""
    _need(operands, "operands", torch.uint8, ndim=1)
    if operands.numel() < 16 or operands.numel() % 16:
        raise ValueError("operands must hold a positive multiple of 16 bytes")
    if kind not in (0, 1):
        raise ValueError("kind must be 0 (fp16) or 1 (int8)")
    dev = _gpu(operands=operands)
    out = torch.empty((blocks * 256,), dtype=torch.float32, device=dev)
    lib = load()
    with torch.cuda.device(dev):
        stream = _stream(dev)
    args = (_ptr(operands), operands.numel(), kind, iters, _ptr(out), blocks, stream)
    fn = lib.w4_ceiling_mfma
    keep = (operands, out)

    def call():
        rc = fn(*args)
        if rc != W4_OK:
            _check("w4_ceiling_mfma", rc)
        return keep
    flops = blocks * 4 * iters * 4 * (65536 if kind == 1 else 32768)
    return call, flops
