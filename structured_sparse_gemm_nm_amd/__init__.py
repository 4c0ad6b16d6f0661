"""N:M structured-sparse GEMM for AMD MI355X (gfx950): thin Python binding.

The work happens in libnmsparse.so (hand-written HIP kernels behind a C ABI,
declared in include/nmsparse.h).  This module only marshals arguments: it
checks tensors, allocates outputs with torch, and passes raw device pointers
and the current HIP stream.  There is no CPU fallback: if the library is
missing every call raises.

Function names follow the C ABI: nm_compress, nm_decompress, nm_spmm,
nm_spmm_perm, nm_packed_sizes.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["NM_OK", "NM_F16", "NM_BF16", "NM_F32", "NM_I8", "NM_I32", "NM_FP8", "NMError", "lib", "lib_path",
           "nm_packed_sizes", "nm_compress", "nm_decompress", "nm_spmm", "nm_spmm_perm",
           "nm_check_perm", "nm_set_variant", "PATTERNS"]

NM_OK = 0
NM_F16, NM_BF16, NM_F32, NM_I8, NM_I32, NM_FP8 = 0, 1, 2, 3, 4, 5
PATTERNS = ((2, 4), (1, 4), (1, 8))

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libnmsparse.so")
_lib = None


class NMError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"nmsparse status {status}: {detail}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded C library (loaded once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m structured_sparse_gemm_nm_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.nm_version.restype = i32
    L.nm_version.argtypes = []
    L.nm_status_string.restype = ctypes.c_char_p
    L.nm_status_string.argtypes = [i32]
    L.nm_last_error.restype = ctypes.c_char_p
    L.nm_last_error.argtypes = []
    L.nm_packed_sizes.restype = i32
    L.nm_packed_sizes.argtypes = [i64, i64, i32, i32, i32, ctypes.POINTER(sz), ctypes.POINTER(sz),
                                  ctypes.POINTER(i64)]
    L.nm_compress.restype = i32
    L.nm_compress.argtypes = [vp, i64, i64, i64, i32, i32, i32, vp, vp, vp]
    L.nm_decompress.restype = i32
    L.nm_decompress.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, i64, vp]
    L.nm_spmm.restype = i32
    L.nm_spmm.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, i64, i64, vp, i64, i32, vp]
    L.nm_spmm_perm.restype = i32
    L.nm_spmm_perm.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, i64, i64, vp, vp, i64, i32, vp]
    L.nm_check_perm.restype = i32
    L.nm_check_perm.argtypes = [vp, i64, vp]
    L.nm_set_variant.restype = i32
    L.nm_set_variant.argtypes = [i32]
    _lib = L
    return L


def _check(status: int) -> None:
    if status != NM_OK:
        raise NMError(status, lib().nm_last_error().decode())


# --------------------------------------------------------------------------
# torch marshalling
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return NM_F16
    if t.dtype == torch.bfloat16:
        return NM_BF16
    if t.dtype == torch.int8:
        return NM_I8
    if t.dtype == torch.float8_e4m3fn:
        return NM_FP8
    raise TypeError(f"expected float16, bfloat16, int8 or float8_e4m3fn, got {t.dtype}")


def _torch_dtype(code: int):
    torch = _torch()
    return {NM_F16: torch.float16, NM_BF16: torch.bfloat16, NM_F32: torch.float32,
            NM_I8: torch.int8, NM_I32: torch.int32, NM_FP8: torch.float8_e4m3fn}[code]


def _stream_ptr(device) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(device).cuda_stream)


def _require_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a HIP device (no CPU path)")


def _row_major(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit stride along its rows")


def nm_packed_sizes(R: int, K: int, n: int, m: int, dtype: int = NM_F16):
    """(values_bytes, idx_bytes, idx_row_words) of the packed format."""
    vb, ib, w = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64()
    _check(lib().nm_packed_sizes(R, K, n, m, dtype, ctypes.byref(vb), ctypes.byref(ib),
                                 ctypes.byref(w)))
    return vb.value, ib.value, w.value


def nm_compress(W, n: int = 2, m: int = 4, values=None, idx=None):
    """Prune W [R, K] (fp16/bf16, or int8 / float8_e4m3fn for 2:4; device) to n:m and pack.
    Returns (values [R, S], idx [R, words])."""
    torch = _torch()
    _require_cuda(W)
    _row_major(W, "W")
    R, K = W.shape
    dt = _dtype_code(W)
    _, _, words = nm_packed_sizes(R, K, n, m, dt)
    S = K // m * n
    if values is None:
        values = torch.empty((R, S), dtype=W.dtype, device=W.device)
    if idx is None:
        idx = torch.empty((R, words), dtype=torch.int32, device=W.device)
    _check(lib().nm_compress(W.data_ptr(), R, K, W.stride(0), dt, n, m, values.data_ptr(),
                             idx.data_ptr(), _stream_ptr(W.device)))
    return values, idx


def nm_decompress(values, idx, K: int, n: int = 2, m: int = 4, out=None):
    """Dense W_nm [R, K] from the packed pair."""
    torch = _torch()
    _require_cuda(values, idx)
    R = values.shape[0]
    dt = _dtype_code(values)
    if out is None:
        out = torch.empty((R, K), dtype=values.dtype, device=values.device)
    _check(lib().nm_decompress(values.data_ptr(), idx.data_ptr(), R, K, n, m, dt, out.data_ptr(),
                               out.stride(0), _stream_ptr(values.device)))
    return out


def nm_spmm(values, idx, act, K: int, n: int = 2, m: int = 4, out_dtype=None, out=None):
    """Y^T [T, R] = act [T, K] . W_nm^T, i.e. Y = W_nm X with X = act^T."""
    return _spmm(values, idx, act, K, n, m, None, out_dtype, out)


def nm_spmm_perm(values, idx, act, perm, K: int, n: int = 2, m: int = 4, out_dtype=None, out=None):
    """Y^T[t, r] = sum_k W_nm[r, k] act[t, perm[k]]  (y = (W Pi) x)."""
    return _spmm(values, idx, act, K, n, m, perm, out_dtype, out)


def _spmm(values, idx, act, K, n, m, perm, out_dtype, out):
    torch = _torch()
    _require_cuda(values, idx, act)
    _row_major(act, "act")
    R = values.shape[0]
    T = act.shape[0]
    dt = _dtype_code(values)
    if act.dtype != values.dtype:
        raise TypeError("act and values must share a dtype")
    if dt == NM_I8:  # the exact integer product
        if out_dtype not in (None, torch.int32):
            raise TypeError("int8 weights give an int32 output")
        od = NM_I32
    elif dt == NM_FP8:  # fp32 sums of the E4M3 products
        if out_dtype not in (None, torch.float32):
            raise TypeError("float8_e4m3fn weights give a float32 output")
        od = NM_F32
    else:
        od = NM_F32 if (out_dtype is None or out_dtype == torch.float32) else _dtype_code(
            torch.empty(0, dtype=out_dtype))
    if out is None:
        out = torch.empty((T, R), dtype=_torch_dtype(od), device=act.device)
    else:
        _require_cuda(out)
        _row_major(out, "out")
        if out.dtype != _torch_dtype(od):
            raise TypeError(f"out is {out.dtype}, the output dtype is {_torch_dtype(od)}")
        if out.shape[0] < T or out.shape[1] < R or out.device != act.device:
            raise ValueError(f"out must be a [{T}, {R}] tensor on {act.device}")
    stream = _stream_ptr(act.device)
    if perm is None:
        st = lib().nm_spmm(values.data_ptr(), idx.data_ptr(), R, K, n, m, dt, act.data_ptr(), T,
                           act.stride(0), out.data_ptr(), out.stride(0), od, stream)
    else:
        _require_cuda(perm)
        if perm.dtype != torch.int32 or perm.numel() != K:
            raise TypeError("perm must be an int32 tensor of K entries")
        st = lib().nm_spmm_perm(values.data_ptr(), idx.data_ptr(), R, K, n, m, dt, act.data_ptr(),
                                T, act.stride(0), perm.data_ptr(), out.data_ptr(), out.stride(0),
                                od, stream)
    _check(st)
    return out


def nm_check_perm(perm) -> None:
    _require_cuda(perm)
    _check(lib().nm_check_perm(perm.data_ptr(), perm.numel(), _stream_ptr(perm.device)))


def nm_set_variant(variant: int) -> None:
    _check(lib().nm_set_variant(variant))
