"""Thin Python binding of the MI355X FPx weight-only linear library.

Argument marshalling only: every step runs in ``libfp6amd.so`` (host packer
and quantiser in C++, de-quantisation and the fused GEMM in HIP kernels for
gfx950).  Host arrays are NumPy; device buffers are torch CUDA (ROCm) tensors
used purely as memory, with the current torch stream passed to the library.

The names follow the C ABI in ``include/fp6.h`` and ``include/fpx.h``; every
call takes ``fmt`` ("e3m2" -- the default, FP6 -- "e2m3", "e2m2" or "e2m1"):
"e3m2" goes through the fp6_* entry points, the others through fpx_*.

* :func:`packed_bytes`, :func:`pack_version`, :func:`bits`
* :func:`quantize_rows` (host) -> ``(codes uint8 [N,K], scales fp16 [N])``
* :func:`prepack` (host) -> ``uint8 [N*K*bits/8]`` packed layout v3
* :func:`linear` (device) -> ``Y fp16 [M,N] = X . dequant(W)^T``
* :func:`linear_plan` (device, forced schedule), :func:`dequant` (device export)
* 2:4-sparse FP6 (``include/fp6s.h``): :func:`sparse_packed_bytes`,
  :func:`prune_quantize`, :func:`sparse_prepack`, :func:`sparse_linear`,
  :func:`sparse_linear_plan`, :func:`sparse_dequant`

There is no fallback: if the shared library is missing or fails to load,
importing this package raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp6amd.so")

FP6_OK = 0
STATUS_NAMES = {
    0: "FP6_OK", 1: "FP6_E_NULL", 2: "FP6_E_SHAPE", 3: "FP6_E_ALIGN", 4: "FP6_E_CODE",
    5: "FP6_E_SCALE", 6: "FP6_E_SIZE", 7: "FP6_E_HIP", 8: "FP6_E_VALUE",
}
EXPORTED = (
    "fp6_pack_version", "fp6_status_string", "fp6_packed_bytes", "fp6_quantize_rows",
    "fp6_prepack", "fp6_linear", "fp6_linear_noalloc", "fp6_linear_plan", "fp6_linear_plan_query", "fp6_dequant",
    "fp6_release", "fpx_bits", "fpx_packed_bytes", "fpx_quantize_rows", "fpx_prepack",
    "fpx_linear", "fpx_linear_plan", "fpx_dequant", "fp6s_packed_bytes", "fp6s_prune_quantize",
    "fp6s_prepack", "fp6s_linear", "fp6s_linear_plan", "fp6s_linear_plan_query", "fp6s_dequant",
)
FORMATS = {"e3m2": 0, "e2m3": 1, "e2m2": 2, "e2m1": 3}


class FP6Error(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, func: str, status: int):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{func}: {self.name} ({_lib.fp6_status_string(status).decode()})")


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime (same SONAME as the system one).  Import
    # torch first so the dynamic linker binds this library to that runtime:
    # loading the library first would bring in a second HIP runtime, whose
    # streams and launches do not interoperate with torch's.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python weight_only_fp6_amd/build_lib.py` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, sz, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    sig = {
        "fp6_pack_version": ([], i32),
        "fp6_status_string": ([i32], ctypes.c_char_p),
        "fp6_packed_bytes": ([i64, i64], sz),
        "fp6_quantize_rows": ([vp, i64, i64, vp, vp], i32),
        "fp6_prepack": ([vp, vp, i64, i64, vp, sz], i32),
        "fp6_linear": ([vp, vp, vp, vp, i64, i64, i64, vp], i32),
        "fp6_linear_noalloc": ([vp, vp, vp, vp, i64, i64, i64, vp], i32),
        "fp6_linear_plan": ([vp, vp, vp, vp, i64, i64, i64, i32, i32, vp], i32),
        "fp6_linear_plan_query": ([i64, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)], i32),
        "fp6_dequant": ([vp, vp, vp, i64, i64, vp], i32),
        "fp6_release": ([], i32),
        "fpx_bits": ([i32], i32),
        "fpx_packed_bytes": ([i32, i64, i64], sz),
        "fpx_quantize_rows": ([i32, vp, i64, i64, vp, vp], i32),
        "fpx_prepack": ([i32, vp, vp, i64, i64, vp, sz], i32),
        "fpx_linear": ([i32, vp, vp, vp, vp, i64, i64, i64, vp], i32),
        "fpx_linear_plan": ([i32, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp], i32),
        "fpx_dequant": ([i32, vp, vp, vp, i64, i64, vp], i32),
        "fp6s_packed_bytes": ([i64, i64], sz),
        "fp6s_prune_quantize": ([vp, i64, i64, vp, vp, vp], i32),
        "fp6s_prepack": ([vp, vp, vp, i64, i64, vp, sz], i32),
        "fp6s_linear": ([vp, vp, vp, vp, i64, i64, i64, vp], i32),
        "fp6s_linear_plan": ([vp, vp, vp, vp, i64, i64, i64, i32, i32, vp], i32),
        "fp6s_linear_plan_query": ([i64, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)], i32),
        "fp6s_dequant": ([vp, vp, vp, i64, i64, vp], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


_lib = _load()
lib = _lib


def _check(func: str, status: int) -> None:
    if status != FP6_OK:
        raise FP6Error(func, status)


def _fmt_id(fmt: str) -> int:
    if fmt not in FORMATS:
        raise ValueError(f"unknown weight format {fmt!r}; expected one of {sorted(FORMATS)}")
    return FORMATS[fmt]


def pack_version() -> int:
    return int(_lib.fp6_pack_version())


def bits(fmt: str = "e3m2") -> int:
    return int(_lib.fpx_bits(_fmt_id(fmt)))


def packed_bytes(N: int, K: int, fmt: str = "e3m2") -> int:
    if fmt == "e3m2":
        return int(_lib.fp6_packed_bytes(N, K))
    return int(_lib.fpx_packed_bytes(_fmt_id(fmt), N, K))


def _host_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def quantize_rows(W: np.ndarray, fmt: str = "e3m2"):
    """Host quantiser: float32 [N,K] -> (codes uint8 [N,K], scales float16 [N])."""
    f = _fmt_id(fmt)
    W = np.ascontiguousarray(W, dtype=np.float32)
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    N, K = W.shape
    codes = np.empty((N, K), dtype=np.uint8)
    scales = np.empty(N, dtype=np.uint16)
    if fmt == "e3m2":
        st = _lib.fp6_quantize_rows(_host_ptr(W), N, K, _host_ptr(codes), _host_ptr(scales))
    else:
        st = _lib.fpx_quantize_rows(f, _host_ptr(W), N, K, _host_ptr(codes), _host_ptr(scales))
    _check("quantize_rows", st)
    return codes, scales.view(np.float16)


def prepack(codes: np.ndarray, scales: np.ndarray, fmt: str = "e3m2") -> np.ndarray:
    """Host packer: codes uint8 [N,K] + scales fp16 [N] -> packed uint8 [N*K*bits/8]."""
    f = _fmt_id(fmt)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float16).view(np.uint16)
    if codes.ndim != 2 or scales.shape != (codes.shape[0],):
        raise ValueError("codes [N,K] and scales [N] expected")
    N, K = codes.shape
    nbytes = packed_bytes(N, K, fmt)
    out = np.empty(max(nbytes, 1), dtype=np.uint8)
    if fmt == "e3m2":
        st = _lib.fp6_prepack(_host_ptr(codes), _host_ptr(scales), N, K, _host_ptr(out), nbytes)
    else:
        st = _lib.fpx_prepack(f, _host_ptr(codes), _host_ptr(scales), N, K, _host_ptr(out), nbytes)
    _check("prepack", st)
    return out[:nbytes]


def _stream_handle(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _dev_ptr(t) -> int:
    return int(t.data_ptr()) if t is not None else 0


_PACKED = "packed (the prepack output for N, K and this format)"
_SPARSE_PACKED = "packed (the sparse_prepack output for N, K)"


def _check_device_tensors(*specs) -> None:
    """Each (tensor, dtype, shape or element count, name) must be a contiguous
    GPU tensor of that dtype and shape, else ValueError -- before anything
    reaches the library, which takes raw pointers and cannot check buffer
    sizes.  Dtypes, shapes and layouts are checked for every tensor before
    devices."""
    import torch
    for t, dtype, shape, what in specs:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{what} must be a torch tensor")
        if t.dtype != dtype:
            raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
        if isinstance(shape, int):
            if t.numel() != shape:
                raise ValueError(f"{what} must hold {shape} elements, got {t.numel()}")
        elif tuple(t.shape) != tuple(shape):
            raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous")
    for t, _, _, what in specs:
        if not t.is_cuda:
            raise ValueError(f"{what} must be on the GPU")


def linear(X, packed, scales, N: int, K: int, out=None, stream=None, fmt: str = "e3m2"):
    """Y[M,N] fp16 = X[M,K] . dequant(W)^T on the GPU (asynchronous)."""
    return linear_plan(X, packed, scales, N, K, variant=0, splits=0, out=out, stream=stream, fmt=fmt)


def linear_plan(X, packed, scales, N: int, K: int, variant: int = 0, splits: int = 0,
                out=None, stream=None, fmt: str = "e3m2"):
    import torch
    f = _fmt_id(fmt)
    if not isinstance(X, torch.Tensor) or X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be an fp16 [M,K] tensor")
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _check_device_tensors((X, torch.float16, (M, K), "X"),
                          (packed, torch.uint8, packed_bytes(N, K, fmt), _PACKED),
                          (scales, torch.float16, N, "scales"),
                          (out, torch.float16, (M, N), "out"))
    args = (_dev_ptr(X), _dev_ptr(packed), _dev_ptr(scales), _dev_ptr(out), M, N, K, variant, splits,
            _stream_handle(stream))
    st = _lib.fp6_linear_plan(*args) if fmt == "e3m2" else _lib.fpx_linear_plan(f, *args)
    _check("linear_plan", st)
    return out


KERNEL_NAMES = {
    1: "fp6_gemm_stream<1,1,4>", 2: "fp6_gemm_stream<1,4,2>", 3: "fp6_gemm_stream<2,1,4>",
    4: "fp6_gemm_stream<4,1,2>", 5: "fp6_gemm_tiled<4,4,4>", 6: "fp6_gemm_tiled<8,4,4>",
    7: "fp6_gemm_stream<1,1,8>", 8: "fp6_gemm_stream<2,1,6>", 9: "fp6_gemm_ksplit<8 waves>",
    10: "fp6_gemm_tiled<8,2,8>", 11: "fp6_gemm_tiled<4,2,8>", 12: "fp6_gemm_ksplit<16 waves>",
    13: "fp6_gemm_kslice", 14: "fp6_gemm_xlds<2,4,4>", 15: "fp6_gemm_xlds<1,4,4>",
    16: "fp6_gemm_xlds<2,4,8>", 17: "fp6_gemm_tiledw<4,2,8>", 18: "fp6_gemm_xlds<1,4,8>",
    19: "fp6_gemm_xlds<2,2,8,MB=2>", 20: "fp6_gemm_xlds<2,2,8,MB=4>", 21: "fp6_gemm_xlds<1,4,8,MB=2>",
    22: "fp6_gemm_xlds<1,2,8,MB=4>", 23: "fp6_gemm_tiledl<8,2,8>", 24: "fp6_gemm_tiledl<4,2,8>",
    25: "fp6_gemm_tiled_sk<8,2,8>", 26: "fp6_gemm_kring",
}


def plan_query(M: int, N: int, K: int):
    """(variant, splits) that fp6_linear picks for this shape on the current GPU."""
    v, s = ctypes.c_int(0), ctypes.c_int(0)
    _check("fp6_linear_plan_query", _lib.fp6_linear_plan_query(M, N, K, ctypes.byref(v), ctypes.byref(s)))
    return v.value, s.value


def dequant(packed, scales, N: int, K: int, out=None, stream=None, fmt: str = "e3m2"):
    """Wdq fp16 [N,K] from the packed weights (same device splice as linear)."""
    import torch
    f = _fmt_id(fmt)
    if out is None:
        out = torch.empty((N, K), dtype=torch.float16, device=packed.device)
    _check_device_tensors((packed, torch.uint8, packed_bytes(N, K, fmt), _PACKED),
                          (scales, torch.float16, N, "scales"),
                          (out, torch.float16, (N, K), "out"))
    args = (_dev_ptr(packed), _dev_ptr(scales), _dev_ptr(out), N, K, _stream_handle(stream))
    st = _lib.fp6_dequant(*args) if fmt == "e3m2" else _lib.fpx_dequant(f, *args)
    _check("dequant", st)
    return out


# ---------------------------------------------------------------------------
# 2:4-sparse FP6
# ---------------------------------------------------------------------------
SPARSE_KERNEL_NAMES = {1: "sp_gemm_kslice", 2: "sp_gemm_xlds<1,4,4>", 3: "sp_gemm_xlds<2,4,4>",
                       4: "sp_gemm_tiled<4,2,8>", 5: "sp_gemm_tiled<8,2,8>", 6: "sp_gemm_ksplit",
                       7: "sp_gemm_xlds<1,4,8,MB=2>", 8: "sp_gemm_xlds<2,2,8,MB=2>", 9: "sp_gemm_kring"}


def sparse_packed_bytes(N: int, K: int) -> int:
    return int(_lib.fp6s_packed_bytes(N, K))


def prune_quantize(W: np.ndarray):
    """Host 2:4 magnitude pruning + quantisation: float32 [N,K] ->
    (codes uint8 [N,K/2], pos uint8 [N,K/2], scales float16 [N])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    N, K = W.shape
    codes = np.empty((N, max(K // 2, 1)), dtype=np.uint8)
    pos = np.empty((N, max(K // 2, 1)), dtype=np.uint8)
    scales = np.empty(N, dtype=np.uint16)
    _check("fp6s_prune_quantize",
           _lib.fp6s_prune_quantize(_host_ptr(W), N, K, _host_ptr(codes), _host_ptr(pos), _host_ptr(scales)))
    return codes, pos, scales.view(np.float16)


def sparse_prepack(codes: np.ndarray, pos: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """Host packer: compressed (codes, pos) [N,K/2] + scales fp16 [N] -> packed uint8 [N*K/2]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    pos = np.ascontiguousarray(pos, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float16).view(np.uint16)
    N = codes.shape[0]
    if codes.shape != (N, K // 2) or pos.shape != (N, K // 2) or scales.shape != (N,):
        raise ValueError("codes, pos [N,K/2] and scales [N] expected")
    nbytes = sparse_packed_bytes(N, K)
    out = np.empty(max(nbytes, 1), dtype=np.uint8)
    _check("fp6s_prepack", _lib.fp6s_prepack(_host_ptr(codes), _host_ptr(pos), _host_ptr(scales), N, K,
                                             _host_ptr(out), nbytes))
    return out[:nbytes]


def sparse_linear(X, packed, scales, N: int, K: int, out=None, stream=None):
    """Y[M,N] fp16 = X[M,K] . Wdq^T for 2:4-sparse packed FP6 weights."""
    return sparse_linear_plan(X, packed, scales, N, K, 0, 0, out=out, stream=stream)


def sparse_linear_plan(X, packed, scales, N: int, K: int, variant: int = 0, splits: int = 0,
                       out=None, stream=None):
    import torch
    if not isinstance(X, torch.Tensor) or X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be an fp16 [M,K] tensor")
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _check_device_tensors((X, torch.float16, (M, K), "X"),
                          (packed, torch.uint8, sparse_packed_bytes(N, K), _SPARSE_PACKED),
                          (scales, torch.float16, N, "scales"),
                          (out, torch.float16, (M, N), "out"))
    st = _lib.fp6s_linear_plan(_dev_ptr(X), _dev_ptr(packed), _dev_ptr(scales), _dev_ptr(out), M, N, K,
                               variant, splits, _stream_handle(stream))
    _check("fp6s_linear_plan", st)
    return out


def sparse_plan_query(M: int, N: int, K: int):
    """(variant, splits) that fp6s_linear picks for this shape on the current GPU."""
    v, s = ctypes.c_int(0), ctypes.c_int(0)
    _check("fp6s_linear_plan_query",
           _lib.fp6s_linear_plan_query(M, N, K, ctypes.byref(v), ctypes.byref(s)))
    return v.value, s.value


def sparse_dequant(packed, scales, N: int, K: int, out=None, stream=None):
    """Dense Wdq fp16 [N,K] (zeros at pruned positions) from packed 2:4 weights."""
    import torch
    if out is None:
        out = torch.empty((N, K), dtype=torch.float16, device=packed.device)
    _check_device_tensors((packed, torch.uint8, sparse_packed_bytes(N, K), _SPARSE_PACKED),
                          (scales, torch.float16, N, "scales"),
                          (out, torch.float16, (N, K), "out"))
    st = _lib.fp6s_dequant(_dev_ptr(packed), _dev_ptr(scales), _dev_ptr(out), N, K, _stream_handle(stream))
    _check("fp6s_dequant", st)
    return out


def release() -> None:
    _check("fp6_release", _lib.fp6_release())
