"""Python binding of libbnbx, the MI355X (gfx950) NF4 4-bit weight library.

Argument marshalling only: every function here has the name of a C entry
point declared in ``include/bnbx.h`` and forwards to it through ctypes.  All
computation happens in the library's HIP kernels.  Device buffers may be
passed as integers (device addresses) or as objects with ``data_ptr()``
(torch tensors); ``stream`` is a hipStream_t handle (int), a torch stream, or
None for the caller's current torch stream when torch has a GPU, else the
null stream.

If the shared library is missing, importing works but every call raises
``BnbxLibraryMissing``: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "BNBX_OK", "BNBX_E_INVAL", "BNBX_E_ALIGN", "BNBX_E_UNSUPPORTED", "BNBX_E_WORKSPACE",
    "BNBX_E_HIP", "BNBX_E_INTERNAL", "BnbxError", "BnbxLibraryMissing", "Nf4State", "library_path", "lib",
    "bnbx_status_str", "bnbx_nf4_codebook", "bnbx_fp4_codebook", "bnbx_dynamic_map",
    "bnbx_quantize_nf4_workspace_bytes",
    "bnbx_quantize_nf4", "bnbx_quantize_nf4_noalloc", "BNBX_NOALLOC_MAX_WEIGHTS",
    "bnbx_quantize_nf4_grouped_workspace_bytes", "bnbx_quantize_nf4_grouped", "QuantizeItem",
    "BNBX_QUANTIZE_MAX_ITEMS",
    "bnbx_dequantize_nf4", "bnbx_gemv_nf4", "bnbx_gemv_nf4_grouped", "GemvItem",
    "BNBX_GEMV_MAX_ITEMS",
    "bnbx_gemm_nf4_workspace_bytes", "bnbx_gemm_nf4", "bnbx_gemm_nf4_dx", "bnbx_gemm_nf4_lora",
    "bnbx_lora_down", "bnbx_probe_stream_read", "BNBX_PROBE_SINK_WORDS", "EXPORTED_SYMBOLS", "BNBX_QUANT_NF4", "BNBX_QUANT_FP4",
    "BNBX_DTYPE_BF16", "BNBX_DTYPE_F16", "BNBX_DQ_NONE", "BNBX_DQ_LINEAR", "BNBX_DQ_DYNAMIC",
]

BNBX_OK = 0
BNBX_E_INVAL = -1
BNBX_E_ALIGN = -2
BNBX_E_UNSUPPORTED = -3
BNBX_E_WORKSPACE = -4
BNBX_E_HIP = -5
BNBX_E_INTERNAL = -6

BNBX_QUANT_NF4 = 0
BNBX_QUANT_FP4 = 1
BNBX_DTYPE_BF16 = 0
BNBX_DTYPE_F16 = 1
BNBX_DQ_NONE = 0
BNBX_DQ_LINEAR = 1
BNBX_DQ_DYNAMIC = 2

BNBX_NOALLOC_MAX_WEIGHTS = 1 << 28
BNBX_GEMV_MAX_ITEMS = 4
BNBX_QUANTIZE_MAX_ITEMS = 8

EXPORTED_SYMBOLS = (
    "bnbx_status_str", "bnbx_nf4_codebook", "bnbx_fp4_codebook", "bnbx_dynamic_map",
    "bnbx_quantize_nf4_workspace_bytes",
    "bnbx_quantize_nf4", "bnbx_quantize_nf4_noalloc", "bnbx_quantize_nf4_grouped_workspace_bytes",
    "bnbx_quantize_nf4_grouped", "bnbx_dequantize_nf4", "bnbx_gemv_nf4",
    "bnbx_gemv_nf4_grouped",
    "bnbx_gemm_nf4_workspace_bytes", "bnbx_gemm_nf4", "bnbx_gemm_nf4_dx", "bnbx_gemm_nf4_lora",
    "bnbx_lora_down",
    "bnbx_probe_stream_read",          # include/bnbx_probe.h (measurement aid)
)
BNBX_PROBE_SINK_WORDS = 1024

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libbnbx.so")


class BnbxLibraryMissing(RuntimeError):
    pass


class BnbxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {bnbx_status_str(status)} ({status})")


class Nf4State(ctypes.Structure):
    """bnbx_nf4_state: host descriptor holding device pointers."""

    _fields_ = [
        ("n", ctypes.c_int64),
        ("blocksize", ctypes.c_int32),
        ("double_quant", ctypes.c_int32),
        ("quant_type", ctypes.c_int32),
        ("compute_dtype", ctypes.c_int32),
        ("absmax", ctypes.c_void_p),
        ("absmax2", ctypes.c_void_p),
        ("absmax_mean", ctypes.c_void_p),
    ]


class QuantizeItem(ctypes.Structure):
    """bnbx_quantize_item: one tensor of a grouped quantize (device pointers;
    the state pointer is a host address)."""

    _fields_ = [
        ("w", ctypes.c_void_p),
        ("packed", ctypes.c_void_p),
        ("st", ctypes.POINTER(Nf4State)),
    ]


class GemvItem(ctypes.Structure):
    """bnbx_gemv_item: one weight of a grouped GEMV (device pointers; the
    state pointer is a host address)."""

    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("st", ctypes.POINTER(Nf4State)),
        ("N", ctypes.c_int32),
        ("y", ctypes.c_void_p),
        ("ldy", ctypes.c_int64),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbnbx.so (built in-tree by dequant_gemm_nf4_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise BnbxLibraryMissing(
            f"{path} is not built; run `python -m dequant_gemm_nf4_amd.build` (no fallback exists)")
    # Loaded before torch had initialized HIP, the library's launches on
    # torch's memory failed (most likely two HIP runtime instances: torch
    # bundles its own).  Importing torch first avoided it in every run.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover
        pass
    L = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sp = ctypes.POINTER(Nf4State)
    L.bnbx_status_str.argtypes = [i32]
    L.bnbx_status_str.restype = ctypes.c_char_p
    L.bnbx_nf4_codebook.argtypes = [ctypes.POINTER(ctypes.c_float)]
    L.bnbx_nf4_codebook.restype = i32
    L.bnbx_fp4_codebook.argtypes = [ctypes.POINTER(ctypes.c_float)]
    L.bnbx_fp4_codebook.restype = i32
    L.bnbx_dynamic_map.argtypes = [ctypes.POINTER(ctypes.c_float)]
    L.bnbx_dynamic_map.restype = i32
    L.bnbx_quantize_nf4_workspace_bytes.argtypes = [i64, i32, i32]
    L.bnbx_quantize_nf4_workspace_bytes.restype = sz
    L.bnbx_quantize_nf4.argtypes = [vp, vp, sp, vp, sz, vp]
    L.bnbx_quantize_nf4.restype = i32
    L.bnbx_quantize_nf4_noalloc.argtypes = [vp, vp, sp, vp]
    L.bnbx_quantize_nf4_noalloc.restype = i32
    L.bnbx_quantize_nf4_grouped_workspace_bytes.argtypes = [ctypes.POINTER(i64), i32, i32, i32]
    L.bnbx_quantize_nf4_grouped_workspace_bytes.restype = sz
    L.bnbx_quantize_nf4_grouped.argtypes = [ctypes.POINTER(QuantizeItem), i32, vp, sz, vp]
    L.bnbx_quantize_nf4_grouped.restype = i32
    L.bnbx_dequantize_nf4.argtypes = [vp, sp, vp, vp]
    L.bnbx_dequantize_nf4.restype = i32
    L.bnbx_gemv_nf4.argtypes = [vp, i64, vp, sp, i32, i32, i32, vp, i64, vp]
    L.bnbx_gemv_nf4.restype = i32
    L.bnbx_gemv_nf4_grouped.argtypes = [vp, i64, ctypes.POINTER(GemvItem), i32, i32, i32, vp]
    L.bnbx_gemv_nf4_grouped.restype = i32
    L.bnbx_gemm_nf4_workspace_bytes.argtypes = [i32, i32, i32]
    L.bnbx_gemm_nf4_workspace_bytes.restype = sz
    L.bnbx_gemm_nf4.argtypes = [vp, i64, vp, sp, i32, i32, i32, vp, i64, vp, sz, vp]
    L.bnbx_gemm_nf4.restype = i32
    L.bnbx_gemm_nf4_lora.argtypes = [vp, i64, vp, sp, i32, i32, i32, vp, i64, vp, i64, i32, vp,
                                     i64, vp]
    L.bnbx_gemm_nf4_lora.restype = i32
    L.bnbx_gemm_nf4_dx.argtypes = [vp, i64, vp, sp, i32, i32, i32, vp, i64, vp]
    L.bnbx_gemm_nf4_dx.restype = i32
    L.bnbx_lora_down.argtypes = [vp, i64, vp, i64, i32, i32, i32, ctypes.c_float, i32, vp, i64, vp]
    L.bnbx_lora_down.restype = i32
    L.bnbx_probe_stream_read.argtypes = [vp, sz, vp, sz, vp, vp]
    L.bnbx_probe_stream_read.restype = i32
    _lib = L
    return L


def _ptr(a) -> int | None:
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return int(a.data_ptr())


def _stream(stream) -> int | None:
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return int(torch.cuda.current_stream().cuda_stream)
        except ImportError:  # pragma: no cover
            pass
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(status: int, where: str) -> None:
    if status != BNBX_OK:
        raise BnbxError(status, where)


def bnbx_status_str(status: int) -> str:
    return lib().bnbx_status_str(int(status)).decode()


def bnbx_nf4_codebook() -> list[float]:
    buf = (ctypes.c_float * 16)()
    _check(lib().bnbx_nf4_codebook(buf), "bnbx_nf4_codebook")
    return list(buf)


def bnbx_fp4_codebook() -> list[float]:
    buf = (ctypes.c_float * 16)()
    _check(lib().bnbx_fp4_codebook(buf), "bnbx_fp4_codebook")
    return list(buf)


def bnbx_dynamic_map() -> list[float]:
    buf = (ctypes.c_float * 256)()
    _check(lib().bnbx_dynamic_map(buf), "bnbx_dynamic_map")
    return list(buf)


def bnbx_quantize_nf4_workspace_bytes(n: int, blocksize: int = 64, double_quant: int = 1) -> int:
    return int(lib().bnbx_quantize_nf4_workspace_bytes(int(n), int(blocksize), int(double_quant)))


def bnbx_quantize_nf4(w, packed, state: Nf4State, workspace=None, workspace_bytes: int = 0,
                      stream=None) -> None:
    _check(lib().bnbx_quantize_nf4(_ptr(w), _ptr(packed), ctypes.byref(state), _ptr(workspace),
                                   int(workspace_bytes), _stream(stream)), "bnbx_quantize_nf4")


def bnbx_quantize_nf4_noalloc(w, packed, state: Nf4State, stream=None) -> None:
    _check(lib().bnbx_quantize_nf4_noalloc(_ptr(w), _ptr(packed), ctypes.byref(state),
                                           _stream(stream)), "bnbx_quantize_nf4_noalloc")


def bnbx_quantize_nf4_grouped_workspace_bytes(ns, blocksize: int = 64,
                                              double_quant: int = 1) -> int:
    arr = (ctypes.c_int64 * max(len(ns), 1))(*[int(n) for n in ns])
    return int(lib().bnbx_quantize_nf4_grouped_workspace_bytes(arr, len(ns), int(blocksize),
                                                               int(double_quant)))


def bnbx_quantize_nf4_grouped(items, workspace=None, workspace_bytes: int = 0,
                              stream=None) -> None:
    """items: sequence of (w, packed, state)."""
    n = len(items)
    arr = (QuantizeItem * max(n, 1))()
    states = [st for _, _, st in items]    # kept alive for the call
    for i, (w, packed, st) in enumerate(items):
        arr[i] = QuantizeItem(_ptr(w), _ptr(packed), ctypes.pointer(st))
    _check(lib().bnbx_quantize_nf4_grouped(arr, n, _ptr(workspace), int(workspace_bytes),
                                           _stream(stream)), "bnbx_quantize_nf4_grouped")
    del states


def bnbx_dequantize_nf4(packed, state: Nf4State, out, stream=None) -> None:
    _check(lib().bnbx_dequantize_nf4(_ptr(packed), ctypes.byref(state), _ptr(out),
                                     _stream(stream)), "bnbx_dequantize_nf4")


def bnbx_gemv_nf4(x, ldx: int, packed, state: Nf4State, M: int, N: int, K: int, y, ldy: int,
                  stream=None) -> None:
    _check(lib().bnbx_gemv_nf4(_ptr(x), int(ldx), _ptr(packed), ctypes.byref(state), int(M),
                               int(N), int(K), _ptr(y), int(ldy), _stream(stream)),
           "bnbx_gemv_nf4")


def bnbx_gemv_nf4_grouped(x, ldx: int, items, M: int, K: int, stream=None) -> None:
    """items: sequence of (packed, state, N, y, ldy)."""
    n = len(items)
    arr = (GemvItem * max(n, 1))()
    states = [st for _, st, _, _, _ in items]    # kept alive for the call
    for i, (packed, st, N, y, ldy) in enumerate(items):
        arr[i] = GemvItem(_ptr(packed), ctypes.pointer(st), int(N), _ptr(y), int(ldy))
    _check(lib().bnbx_gemv_nf4_grouped(_ptr(x), int(ldx), arr, n, int(M), int(K),
                                       _stream(stream)), "bnbx_gemv_nf4_grouped")
    del states


def bnbx_gemm_nf4_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().bnbx_gemm_nf4_workspace_bytes(int(M), int(N), int(K)))


def bnbx_gemm_nf4(x, ldx: int, packed, state: Nf4State, M: int, N: int, K: int, y, ldy: int,
                  workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    _check(lib().bnbx_gemm_nf4(_ptr(x), int(ldx), _ptr(packed), ctypes.byref(state), int(M),
                               int(N), int(K), _ptr(y), int(ldy), _ptr(workspace),
                               int(workspace_bytes), _stream(stream)), "bnbx_gemm_nf4")


def bnbx_gemm_nf4_lora(x, ldx: int, packed, state: Nf4State, M: int, N: int, K: int, xa,
                       ldxa: int, lora_b, ldb: int, r: int, y, ldy: int, stream=None) -> None:
    _check(lib().bnbx_gemm_nf4_lora(_ptr(x), int(ldx), _ptr(packed), ctypes.byref(state), int(M),
                                    int(N), int(K), _ptr(xa), int(ldxa), _ptr(lora_b), int(ldb),
                                    int(r), _ptr(y), int(ldy), _stream(stream)),
           "bnbx_gemm_nf4_lora")


def bnbx_gemm_nf4_dx(dy, lddy: int, packed, state: Nf4State, M: int, N: int, K: int, dx,
                     lddx: int, stream=None) -> None:
    _check(lib().bnbx_gemm_nf4_dx(_ptr(dy), int(lddy), _ptr(packed), ctypes.byref(state), int(M),
                                  int(N), int(K), _ptr(dx), int(lddx), _stream(stream)),
           "bnbx_gemm_nf4_dx")


def bnbx_lora_down(x, ldx: int, lora_a, lda: int, M: int, K: int, r: int, scale: float,
                   compute_dtype: int, xa, ldxa: int, stream=None) -> None:
    _check(lib().bnbx_lora_down(_ptr(x), int(ldx), _ptr(lora_a), int(lda), int(M), int(K), int(r),
                                float(scale), int(compute_dtype), _ptr(xa), int(ldxa),
                                _stream(stream)), "bnbx_lora_down")


def _nbytes(t) -> int | None:
    return None if t is None or isinstance(t, int) else int(t.numel() * t.element_size())


def bnbx_probe_stream_read(a, a_bytes: int, b, b_bytes: int, sink, stream=None) -> None:
    # The library cannot see buffer sizes: for tensors, a byte count past the
    # end is rejected here rather than read.
    for t, n in ((a, a_bytes), (b, b_bytes), (sink, 4 * BNBX_PROBE_SINK_WORDS)):
        size = _nbytes(t)
        if size is not None and n > size:
            raise BnbxError(BNBX_E_INVAL, "bnbx_probe_stream_read: byte count past the buffer")
    _check(lib().bnbx_probe_stream_read(_ptr(a), int(a_bytes), _ptr(b), int(b_bytes), _ptr(sink),
                                        _stream(stream)), "bnbx_probe_stream_read")
