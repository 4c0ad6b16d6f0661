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
           "nm_spmm_perm_workspace_size", "nm_spmm_perm_static", "nm_check_perm", "nm_spmm_dx", "nm_spmm_dw",
           "nm_hybrid_layout", "nm_hybrid_compress", "nm_hybrid_spmm", "nm_block_structure", "nm_block_compress",
           "nm_block_spmm", "nm_diag_compress", "nm_diag_spmm", "PATTERNS"]

NM_OK = 0
NM_F16, NM_BF16, NM_F32, NM_I8, NM_I32, NM_FP8 = 0, 1, 2, 3, 4, 5
PATTERNS = ((2, 4), (1, 4), (1, 8))

_HERE = os.path.dirname(os.path.abspath(__file__))
# NMSPARSE_LIB selects another build of the same library (the host-sanitized
# one that `build --sanitize` writes, for instance)
_LIB_PATH = os.environ.get("NMSPARSE_LIB") or os.path.join(_HERE, "libnmsparse.so")
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
    L.nm_spmm_perm.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, i64, i64, vp, vp, i64, i32, vp, sz, vp]
    L.nm_spmm_perm_static.restype = i32
    L.nm_spmm_perm_static.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, i64, i64, vp, vp, i64, i32, vp]
    L.nm_spmm_perm_workspace_size.restype = i32
    L.nm_spmm_perm_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(sz)]
    L.nm_check_perm.restype = i32
    L.nm_check_perm.argtypes = [vp, i64, vp]
    L.nm_spmm_variant.restype = i32
    L.nm_spmm_variant.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, i64, i64, vp, vp, i64, i32, vp, sz, i32, vp]
    L.nm_spmm_dx.restype = i32
    L.nm_spmm_dx.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, i64, i64, vp, i64, i32, vp]
    L.nm_spmm_dw.restype = i32
    L.nm_spmm_dw.argtypes = [vp, i64, i64, i32, i32, i32, vp, i64, i64, vp, i64, vp, i32, vp]
    L.nm_hybrid_layout.restype = i32
    L.nm_hybrid_layout.argtypes = [i64, i64, i64, i64, vp, vp, vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.nm_hybrid_compress.restype = i32
    L.nm_hybrid_compress.argtypes = [vp, i64, i64, i64, i32, i64, i64, vp, vp, i64, i64, vp, vp, vp]
    L.nm_hybrid_spmm.restype = i32
    L.nm_hybrid_spmm.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, vp, i64, i64, vp, i64, i32, vp]
    L.nm_block_structure.restype = i32
    L.nm_block_structure.argtypes = [i64, i64, vp, vp, vp, ctypes.POINTER(i64)]
    L.nm_block_compress.restype = i32
    L.nm_block_compress.argtypes = [vp, i64, i64, i64, i32, vp, vp, i64, vp, vp]
    L.nm_block_spmm.restype = i32
    L.nm_block_spmm.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp, i64, i64, vp, vp, i64, i32, vp]
    L.nm_diag_compress.restype = i32
    L.nm_diag_compress.argtypes = [vp, i64, i64, i64, i32, vp, i64, vp, vp]
    L.nm_diag_spmm.restype = i32
    L.nm_diag_spmm.argtypes = [vp, vp, i64, i64, i64, i32, vp, i64, i64, vp, vp, i64, i32, vp]
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


def _check_packed(values, idx, R, K, n, m, dt, name_v="values", name_i="idx"):
    """values must be a contiguous [R, K*n/m] tensor of the weight dtype and idx a
    contiguous int32 [R, idx_row_words] tensor, both on one device: the C ABI
    takes bare pointers, so a wrong size here would become an out-of-bounds access."""
    torch = _torch()
    _, _, words = nm_packed_sizes(R, K, n, m, dt)
    S = K // m * n
    if tuple(values.shape) != (R, S) or not values.is_contiguous():
        raise ValueError(f"{name_v} must be a contiguous [{R}, {S}] tensor, got {tuple(values.shape)}")
    if idx.dtype != torch.int32 or tuple(idx.shape) != (R, words) or not idx.is_contiguous():
        raise ValueError(f"{name_i} must be a contiguous int32 [{R}, {words}] tensor, got "
                         f"{idx.dtype} {tuple(idx.shape)}")
    if idx.device != values.device:
        raise ValueError(f"{name_v} and {name_i} must be on one device")


def nm_compress(W, n: int = 2, m: int = 4, values=None, idx=None):
    """Prune W [R, K] (fp16/bf16, or int8 / float8_e4m3fn for 2:4; device) to n:m and pack.
    Returns (values [R, S], idx [R, words])."""
    torch = _torch()
    _row_major(W, "W")
    R, K = W.shape
    dt = _dtype_code(W)
    _, _, words = nm_packed_sizes(R, K, n, m, dt)
    S = K // m * n
    if values is not None or idx is not None:  # caller-provided outputs: check before the device
        _check_packed(values if values is not None else W.new_empty((R, S)),
                      idx if idx is not None else W.new_empty((R, words), dtype=torch.int32), R, K, n, m, dt)
    _require_cuda(W)
    if values is None:
        values = torch.empty((R, S), dtype=W.dtype, device=W.device)
    elif values.dtype != W.dtype:
        raise TypeError(f"values is {values.dtype}, W is {W.dtype}")
    if idx is None:
        idx = torch.empty((R, words), dtype=torch.int32, device=W.device)
    _check_packed(values, idx, R, K, n, m, dt)
    if values.device != W.device:
        raise ValueError("values, idx and W must be on one device")
    _check(lib().nm_compress(W.data_ptr(), R, K, W.stride(0), dt, n, m, values.data_ptr(),
                             idx.data_ptr(), _stream_ptr(W.device)))
    return values, idx


def nm_decompress(values, idx, K: int, n: int = 2, m: int = 4, out=None):
    """Dense W_nm [R, K] from the packed pair."""
    torch = _torch()
    R = values.shape[0]
    dt = _dtype_code(values)
    _check_packed(values, idx, R, K, n, m, dt)
    if out is not None:
        _row_major(out, "out")
        if out.dtype != values.dtype or tuple(out.shape) != (R, K) or out.device != values.device:
            raise ValueError(f"out must be a {values.dtype} [{R}, {K}] tensor on {values.device}")
    _require_cuda(values, idx)
    if out is None:
        out = torch.empty((R, K), dtype=values.dtype, device=values.device)
    _check(lib().nm_decompress(values.data_ptr(), idx.data_ptr(), R, K, n, m, dt, out.data_ptr(),
                               out.stride(0), _stream_ptr(values.device)))
    return out


def nm_spmm(values, idx, act, K: int, n: int = 2, m: int = 4, out_dtype=None, out=None, variant: int = 0):
    """Y^T [T, R] = act [T, K] . W_nm^T, i.e. Y = W_nm X with X = act^T.
    variant != 0 names the kernel family (tests, ablations; see nm_spmm_variant)."""
    return _spmm(values, idx, act, K, n, m, None, out_dtype, out, variant, None)


def nm_spmm_perm_workspace_size(R: int, K: int, T: int, n: int = 2, m: int = 4, dtype: int = NM_F16) -> int:
    """Bytes of caller workspace nm_spmm_perm uses for its gather pass (0: none)."""
    b = ctypes.c_size_t()
    _check(lib().nm_spmm_perm_workspace_size(R, K, T, n, m, dtype, ctypes.byref(b)))
    return b.value


def nm_spmm_perm(values, idx, act, perm, K: int, n: int = 2, m: int = 4, out_dtype=None, out=None,
                 variant: int = 0, workspace="auto"):
    """Y^T[t, r] = sum_k W_nm[r, k] act[t, perm[k]]  (y = (W Pi) x).
    workspace: "auto" (a torch tensor of nm_spmm_perm_workspace_size bytes, when the
    shape takes the gather pass), None (the kernel applies the map as it reads act),
    or a caller-owned device tensor."""
    return _spmm(values, idx, act, K, n, m, perm, out_dtype, out, variant, workspace)


def nm_spmm_perm_static(values, idx, act, perm, K: int, n: int = 2, m: int = 4, out_dtype=None, out=None):
    """nm_spmm_perm with the library's static per-GPU workspace (no allocation in
    the library; calls that overlap in time on one GPU race)."""
    return _spmm(values, idx, act, K, n, m, perm, out_dtype, out, 0, "static")


def _train_out_dtype(torch, dt, out_dtype):
    if dt not in (NM_F16, NM_BF16):
        raise TypeError("the training products take float16 or bfloat16 weights")
    if out_dtype is None or out_dtype == torch.float32:
        return NM_F32
    od = _dtype_code(torch.empty(0, dtype=out_dtype))
    if od != dt:
        raise TypeError("out_dtype must be float32 or the weights' dtype")
    return od


def nm_spmm_dx(values, idx, G, K: int, n: int = 2, m: int = 4, out_dtype=None, out=None):
    """dX [T, K] = G [T, R] @ W_nm: the gradient of the activations of Yt = act @ W_nm^T."""
    torch = _torch()
    _row_major(G, "G")
    R = values.shape[0]
    T = G.shape[0]
    dt = _dtype_code(values)
    od = _train_out_dtype(torch, dt, out_dtype)
    _check_packed(values, idx, R, K, n, m, dt)
    if G.dtype != values.dtype or G.shape[1] != R or G.device != values.device:
        raise ValueError(f"G must be a [T, {R}] {values.dtype} tensor on {values.device}")
    if out is not None:
        _row_major(out, "out")
        if out.dtype != _torch_dtype(od) or tuple(out.shape) != (T, K) or out.device != G.device:
            raise ValueError(f"out must be a [{T}, {K}] {_torch_dtype(od)} tensor on {G.device}")
    _require_cuda(values, idx, G, *(t for t in (out,) if t is not None))
    if out is None:
        out = torch.empty((T, K), dtype=_torch_dtype(od), device=G.device)
    _check(lib().nm_spmm_dx(values.data_ptr(), idx.data_ptr(), R, K, n, m, dt, G.data_ptr(), T, G.stride(0),
                            out.data_ptr(), out.stride(0), od, _stream_ptr(G.device)))
    return out


def nm_spmm_dw(idx, G, act, K: int, n: int = 2, m: int = 4, out_dtype=None, out=None):
    """dW [R, S]: the gradient of each stored survivor, sum_t G[t, r] act[t, k(r, s)]."""
    torch = _torch()
    _row_major(G, "G")
    _row_major(act, "act")
    R = idx.shape[0]
    T = G.shape[0]
    dt = _dtype_code(act)
    od = _train_out_dtype(torch, dt, out_dtype)
    S = K * n // m
    if G.dtype != act.dtype or G.shape[1] != R or act.shape != (T, K) or G.device != act.device:
        raise ValueError(f"G must be [T, {R}] and act [T, {K}], one dtype, on one device")
    _, _, words = nm_packed_sizes(R, K, n, m, dt)
    if idx.dtype != torch.int32 or tuple(idx.shape) != (R, words) or not idx.is_contiguous():
        raise ValueError(f"idx must be a contiguous int32 [{R}, {words}] tensor")
    if out is not None:
        if out.dtype != _torch_dtype(od) or tuple(out.shape) != (R, S) or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous [{R}, {S}] {_torch_dtype(od)} tensor")
    _require_cuda(idx, G, act, *(t for t in (out,) if t is not None))
    if out is None:
        out = torch.empty((R, S), dtype=_torch_dtype(od), device=G.device)
    _check(lib().nm_spmm_dw(idx.data_ptr(), R, K, n, m, dt, G.data_ptr(), T, G.stride(0), act.data_ptr(),
                            act.stride(0), out.data_ptr(), od, _stream_ptr(G.device)))
    return out


def _spmm(values, idx, act, K, n, m, perm, out_dtype, out, variant, workspace):
    torch = _torch()
    _row_major(act, "act")
    R = values.shape[0]
    T = act.shape[0]
    dt = _dtype_code(values)
    if act.dtype != values.dtype:
        raise TypeError("act and values must share a dtype")
    _check_packed(values, idx, R, K, n, m, dt)
    if act.shape[1] != K or act.device != values.device:
        raise ValueError(f"act must be a [T, {K}] tensor on {values.device}")
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
    if out is not None:
        _row_major(out, "out")
        if out.dtype != _torch_dtype(od):
            raise TypeError(f"out is {out.dtype}, the output dtype is {_torch_dtype(od)}")
        if tuple(out.shape) != (T, R) or out.device != act.device:
            raise ValueError(f"out must be a [{T}, {R}] tensor on {act.device}")
    if perm is not None:
        if perm.dtype != torch.int32 or perm.numel() != K or not perm.is_contiguous():
            raise TypeError("perm must be a contiguous int32 tensor of K entries")
        if perm.device != act.device:
            raise ValueError("perm must be on the device of act")
    ws = None
    if perm is not None and isinstance(workspace, str):
        if workspace not in ("auto", "static"):
            raise ValueError('workspace must be "auto", None or a device tensor')
        if workspace == "auto":
            need = nm_spmm_perm_workspace_size(R, K, T, n, m, dt)
            ws = torch.empty(need, dtype=torch.uint8, device=act.device) if need else None
    elif perm is not None and workspace is not None:
        ws = workspace
        if not ws.is_contiguous() or ws.device != act.device:
            raise ValueError("workspace must be a contiguous tensor on the device of act")
    _require_cuda(values, idx, act, *(t for t in (out, perm, ws) if t is not None))
    if out is None:
        out = torch.empty((T, R), dtype=_torch_dtype(od), device=act.device)
    stream = _stream_ptr(act.device)
    L = lib()
    ws_ptr = None if ws is None else ws.data_ptr()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    if perm is not None and workspace == "static":
        st = L.nm_spmm_perm_static(values.data_ptr(), idx.data_ptr(), R, K, n, m, dt, act.data_ptr(), T,
                                   act.stride(0), perm.data_ptr(), out.data_ptr(), out.stride(0), od, stream)
    elif variant:
        st = L.nm_spmm_variant(values.data_ptr(), idx.data_ptr(), R, K, n, m, dt, act.data_ptr(), T,
                               act.stride(0), None if perm is None else perm.data_ptr(), out.data_ptr(),
                               out.stride(0), od, ws_ptr, ws_bytes, variant, stream)
    elif perm is None:
        st = L.nm_spmm(values.data_ptr(), idx.data_ptr(), R, K, n, m, dt, act.data_ptr(), T,
                       act.stride(0), out.data_ptr(), out.stride(0), od, stream)
    else:
        st = L.nm_spmm_perm(values.data_ptr(), idx.data_ptr(), R, K, n, m, dt, act.data_ptr(),
                            T, act.stride(0), perm.data_ptr(), out.data_ptr(), out.stride(0),
                            od, ws_ptr, ws_bytes, stream)
    _check(st)
    return out


def nm_check_perm(perm) -> None:
    _require_cuda(perm)
    _check(lib().nm_check_perm(perm.data_ptr(), perm.numel(), _stream_ptr(perm.device)))


# --------------------------------------------------------------------------
# hybrid dense / 2:4 tiles
# --------------------------------------------------------------------------

class HybridLayout:
    """Layout of a weight cut into tile_rows x tile_cols tiles, each dense (flag 1)
    or 2:4 (flag 0), as nm_hybrid_layout computes it (host tables, plus their
    device copies made on first use per device)."""

    def __init__(self, R, K, tile_rows, tile_cols, flags, tile_meta, row_meta, values_count, idx_bytes):
        self.R, self.K, self.tile_rows, self.tile_cols = R, K, tile_rows, tile_cols
        self.flags, self.tile_meta, self.row_meta = flags, tile_meta, row_meta
        self.values_count, self.idx_bytes = values_count, idx_bytes
        self._dev = {}

    def device_tables(self, device):
        torch = _torch()
        key = str(device)
        if key not in self._dev:
            self._dev[key] = (torch.from_numpy(self.tile_meta).to(device),
                              torch.from_numpy(self.row_meta).to(device))
        return self._dev[key]


def nm_hybrid_layout(R: int, K: int, tile_rows: int, tile_cols: int, flags) -> HybridLayout:
    """Layout tables for the tile flags (uint8 [ceil(R/tile_rows), K/tile_cols]: 1 dense, 0 2:4)."""
    import numpy as np
    RB, KB = -(-R // tile_rows) if tile_rows > 0 else 0, K // tile_cols if tile_cols > 0 else 0
    f = np.ascontiguousarray(np.asarray(flags, dtype=np.uint8))
    if f.shape != (RB, KB):
        raise ValueError(f"flags must have shape ({RB}, {KB})")
    tm = np.zeros((RB, KB, 2), dtype=np.int64)
    rm = np.zeros((RB, 4), dtype=np.int64)
    nv, ni = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().nm_hybrid_layout(R, K, tile_rows, tile_cols, f.ctypes.data, tm.ctypes.data, rm.ctypes.data,
                                  ctypes.byref(nv), ctypes.byref(ni)))
    return HybridLayout(R, K, tile_rows, tile_cols, f, tm, rm, nv.value, ni.value)


def nm_hybrid_compress(W, layout: HybridLayout, values=None, idx=None):
    """Pack W [R, K] (fp16/bf16, device) by the layout: (values [values_count], idx uint8 [idx_bytes])."""
    torch = _torch()
    _row_major(W, "W")
    R, K = W.shape
    if (R, K) != (layout.R, layout.K):
        raise ValueError(f"W is [{R}, {K}], the layout is for [{layout.R}, {layout.K}]")
    dt = _dtype_code(W)
    if values is None:
        values = torch.empty(layout.values_count, dtype=W.dtype, device=W.device)
    if idx is None:
        idx = torch.zeros(max(layout.idx_bytes, 16), dtype=torch.uint8, device=W.device)
    if values.dtype != W.dtype or values.numel() < layout.values_count or not values.is_contiguous():
        raise ValueError(f"values must be a contiguous {W.dtype} tensor of {layout.values_count} elements")
    if idx.dtype != torch.uint8 or idx.numel() < layout.idx_bytes or not idx.is_contiguous():
        raise ValueError(f"idx must be a contiguous uint8 tensor of {layout.idx_bytes} bytes")
    _require_cuda(W, values, idx)
    tm, rm = layout.device_tables(W.device)
    _check(lib().nm_hybrid_compress(W.data_ptr(), R, K, W.stride(0), dt, layout.tile_rows, layout.tile_cols,
                                    tm.data_ptr(), rm.data_ptr(), layout.values_count, layout.idx_bytes,
                                    values.data_ptr(), idx.data_ptr(), _stream_ptr(W.device)))
    return values, idx


def nm_hybrid_spmm(values, idx, layout: HybridLayout, act, out_dtype=None, out=None):
    """Y^T [T, R] = act [T, K] . W_hat^T for a hybrid-tile packed weight."""
    torch = _torch()
    _row_major(act, "act")
    T, K = act.shape
    R = layout.R
    dt = _dtype_code(values)
    if act.dtype != values.dtype or K != layout.K:
        raise ValueError(f"act must be [T, {layout.K}] of the dtype of values")
    if values.numel() < layout.values_count or idx.numel() < layout.idx_bytes:
        raise ValueError("values / idx smaller than the layout's packed sizes")
    od = NM_F32 if (out_dtype is None or out_dtype == torch.float32) else dt
    if out is not None:
        _row_major(out, "out")
        if out.dtype != _torch_dtype(od) or tuple(out.shape) != (T, R):
            raise ValueError(f"out must be a {_torch_dtype(od)} [{T}, {R}] tensor")
    _require_cuda(values, idx, act, *(t for t in (out,) if t is not None))
    if out is None:
        out = torch.empty((T, R), dtype=_torch_dtype(od), device=act.device)
    tm, rm = layout.device_tables(act.device)
    _check(lib().nm_hybrid_spmm(values.data_ptr(), idx.data_ptr(), tm.data_ptr(), rm.data_ptr(), R, K,
                                layout.tile_rows, layout.tile_cols, layout.values_count, layout.idx_bytes, dt,
                                act.data_ptr(), T, act.stride(0), out.data_ptr(), out.stride(0), od,
                                _stream_ptr(act.device)))
    return out


# ---------------------------------------------------------------------------
# The column permutation on block-sparse and diagonal-sparse weights
# ---------------------------------------------------------------------------

def _out16(torch, dt, out_dtype, what):
    if dt not in (NM_F16, NM_BF16):
        raise TypeError(f"{what} take float16 or bfloat16 weights")
    if out_dtype is None or out_dtype == torch.float32:
        return NM_F32
    od = _dtype_code(torch.empty(0, dtype=out_dtype))
    if od != dt:
        raise TypeError("out_dtype must be float32 or the weights' dtype")
    return od


def _int32_vector(t, n, name, device):
    torch = _torch()
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or (n is not None and t.numel() != n) \
            or t.device != device:
        size = f"[{n}] " if n is not None else ""
        raise ValueError(f"{name} must be a contiguous int32 {size}tensor on {device}")


def _product_out(torch, out, T, R, od, device):
    if out is not None:
        _row_major(out, "out")
        if out.dtype != _torch_dtype(od) or tuple(out.shape) != (T, R) or out.device != device:
            raise ValueError(f"out must be a [{T}, {R}] {_torch_dtype(od)} tensor on {device}")
        return out
    return torch.empty((T, R), dtype=_torch_dtype(od), device=device)


def nm_block_structure(R: int, K: int, mask):
    """(row_ptr int32 [R/32 + 1], col int32 [nnzb]) as numpy arrays, from a host
    mask over the 32 x 32 block grid ([R/32, K/32], 1 keeps a block)."""
    import numpy as np
    m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8).reshape(-1))
    if R % 32 == 0 and K % 32 == 0 and m.size != (R // 32) * (K // 32):
        raise ValueError(f"mask must have {(R // 32) * (K // 32)} entries")
    n = ctypes.c_int64()
    _check(lib().nm_block_structure(R, K, m.ctypes.data if m.size else None, None, None, ctypes.byref(n)))
    row_ptr = np.zeros(R // 32 + 1, dtype=np.int32)
    col = np.zeros(max(n.value, 1), dtype=np.int32)
    _check(lib().nm_block_structure(R, K, m.ctypes.data if m.size else None, row_ptr.ctypes.data,
                                    col.ctypes.data, None))
    return row_ptr, col[:n.value]


def nm_block_compress(W, row_ptr, col, values=None):
    """values [nnzb, 32, 32]: the kept blocks of W (row_ptr, col: int32 device
    tensors); a caller tensor `values` of that shape is filled in place."""
    torch = _torch()
    _row_major(W, "W")
    R, K = W.shape
    dt = _dtype_code(W)
    _int32_vector(row_ptr, R // 32 + 1, "row_ptr", W.device)
    _int32_vector(col, None, "col", W.device)
    _require_cuda(W, row_ptr, col)
    nnzb = col.numel()
    if values is None:
        values = torch.empty((nnzb, 32, 32), dtype=W.dtype, device=W.device)
    elif values.dtype != W.dtype or tuple(values.shape) != (nnzb, 32, 32) or not values.is_contiguous() \
            or values.device != W.device:
        raise ValueError(f"values must be a contiguous [{nnzb}, 32, 32] {W.dtype} tensor on {W.device}")
    _check(lib().nm_block_compress(W.data_ptr(), R, K, W.stride(0), dt, row_ptr.data_ptr(),
                                   col.data_ptr() or None, nnzb, values.data_ptr() or None, _stream_ptr(W.device)))
    return values


def nm_block_spmm(values, row_ptr, col, act, perm=None, out_dtype=None, out=None):
    """Y [T, R] = act read through perm times the block-sparse W^T (R = 32 * (row_ptr.numel() - 1))."""
    torch = _torch()
    _row_major(act, "act")
    T, K = act.shape
    R = 32 * (row_ptr.numel() - 1)
    dt = _dtype_code(act)
    od = _out16(torch, dt, out_dtype, "block products")
    nnzb = col.numel()
    if values.dtype != act.dtype or tuple(values.shape) != (nnzb, 32, 32) or not values.is_contiguous() \
            or values.device != act.device:
        raise ValueError(f"values must be a contiguous [{nnzb}, 32, 32] {act.dtype} tensor on {act.device}")
    _int32_vector(row_ptr, None, "row_ptr", act.device)
    _int32_vector(col, None, "col", act.device)
    if perm is not None:
        _int32_vector(perm, K, "perm", act.device)
    out = _product_out(torch, out, T, R, od, act.device)
    _require_cuda(values, row_ptr, col, act, out, *(t for t in (perm,) if t is not None))
    _check(lib().nm_block_spmm(values.data_ptr() or None, row_ptr.data_ptr(), col.data_ptr() or None, nnzb, R, K,
                               dt, act.data_ptr(), T, act.stride(0),
                               perm.data_ptr() if perm is not None else None, out.data_ptr(), out.stride(0), od,
                               _stream_ptr(act.device)))
    return out


def nm_diag_compress(W, offsets, values=None):
    """values [D, R]: values[d, r] = W[r, (r + offsets[d]) mod K] (offsets: int32
    device tensor); a caller tensor `values` of that shape is filled in place."""
    torch = _torch()
    _row_major(W, "W")
    R, K = W.shape
    dt = _dtype_code(W)
    _int32_vector(offsets, None, "offsets", W.device)
    _require_cuda(W, offsets)
    D = offsets.numel()
    if values is None:
        values = torch.empty((D, R), dtype=W.dtype, device=W.device)
    elif values.dtype != W.dtype or tuple(values.shape) != (D, R) or not values.is_contiguous() \
            or values.device != W.device:
        raise ValueError(f"values must be a contiguous [{D}, {R}] {W.dtype} tensor on {W.device}")
    _check(lib().nm_diag_compress(W.data_ptr(), R, K, W.stride(0), dt, offsets.data_ptr() or None, D,
                                  values.data_ptr() or None, _stream_ptr(W.device)))
    return values


def nm_diag_spmm(values, offsets, act, perm=None, out_dtype=None, out=None):
    """Y [T, R] = act read through perm times the diagonal-sparse W^T (R = values.shape[1])."""
    torch = _torch()
    _row_major(act, "act")
    T, K = act.shape
    D, R = values.shape
    dt = _dtype_code(act)
    od = _out16(torch, dt, out_dtype, "diagonal products")
    if values.dtype != act.dtype or not values.is_contiguous() or values.device != act.device:
        raise ValueError(f"values must be a contiguous [D, R] {act.dtype} tensor on {act.device}")
    _int32_vector(offsets, D, "offsets", act.device)
    if perm is not None:
        _int32_vector(perm, K, "perm", act.device)
    out = _product_out(torch, out, T, R, od, act.device)
    _require_cuda(values, offsets, act, out, *(t for t in (perm,) if t is not None))
    _check(lib().nm_diag_spmm(values.data_ptr() or None, offsets.data_ptr() or None, D, R, K, dt, act.data_ptr(),
                              T, act.stride(0), perm.data_ptr() if perm is not None else None, out.data_ptr(),
                              out.stride(0), od, _stream_ptr(act.device)))
    return out
