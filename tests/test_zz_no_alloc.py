"""The allocation-free permuted GEMM (nm_spmm_perm_static), called through the
C ABI: its gather pass uses the library's static per-GPU workspace instead of
one the caller provides.  Two calls in a row, the second on a smaller input,
each equal bit for bit to nm_spmm_perm with a caller workspace (the same
gather and GEMM kernels) and within the fp32 summation bound of the oracle."""
import ctypes

import numpy as np
import pytest

import nm_inputs
import structured_sparse_gemm_nm_amd as nm
from oracle import nm_oracle as O
from gpu_util import assert_close, error_bound, log, to_dev, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def call_static(vals, idx, A, P, K, od):
    """nm_spmm_perm_static through ctypes, on the current stream."""
    L = nm.lib()
    T, R = A.shape[0], vals.shape[0]
    Y = torch.empty((T, R), dtype=od, device="cuda")
    dt = nm.NM_F16 if vals.dtype == torch.float16 else nm.NM_BF16
    odc = nm.NM_F32 if od == torch.float32 else dt
    st = L.nm_spmm_perm_static(ctypes.c_void_p(vals.data_ptr()), ctypes.c_void_p(idx.data_ptr()), R, K, 2, 4,
                               dt, ctypes.c_void_p(A.data_ptr()), T, A.stride(0), ctypes.c_void_p(P.data_ptr()),
                               ctypes.c_void_p(Y.data_ptr()), Y.stride(0), odc,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.nm_last_error().decode()
    return Y


# (R, K, T, dtype, output): the second input is smaller than the first, so the
# array still holds the first call's larger X' when the second runs
CASES = [(3072, 768, 2000, "f16", "f32"), (700, 512, 300, "bf16", "half")]


def test_static_workspace_two_calls():
    outs = []
    for R, K, T, dt, out in CASES:
        log(f"static workspace R={R} K={K} T={T} {dt} out={out}")
        w = nm_inputs.normal_half((R, K), 0.02, dt, 80, 0, R + K + T)
        act = nm_inputs.normal_half((T, K), 1.0, dt, 80, 1, R + K + T)
        perm = nm_inputs.random_permutation(K, 80, R + T)
        vals, idx = nm.nm_compress(to_dev(w, dt), 2, 4)
        A = to_dev(act, dt)
        P = torch.from_numpy(perm).cuda()
        od = torch_dtype(dt) if out == "half" else torch.float32
        assert 0 < nm.nm_spmm_perm_workspace_size(R, K, T, 2, 4, nm.NM_F16) <= 32 << 20
        y_static = call_static(vals, idx, A, P, K, od)
        y_ws = nm.nm_spmm_perm(vals, idx, A, P, K, 2, 4, out_dtype=od)   # caller workspace
        torch.cuda.synchronize()
        assert torch.equal(y_static, y_ws)
        ref_vals, ref_idx = O.prune_pack(w, 2, 4)
        yref = O.spmm_ref(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm)
        assert_close(y_static, yref, error_bound(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm),
                     **({"out_half": dt} if out == "half" else {}))
        outs.append(y_static)
    # the binding's name for it gives the same result
    y_again = nm.nm_spmm_perm_static(vals, idx, A, P, K, 2, 4, out_dtype=od)
    torch.cuda.synchronize()
    assert torch.equal(y_again, outs[-1])


def test_static_workspace_few_tokens():
    # T <= 16 gathers inside the kernel: no workspace is touched
    R, K, T, dt = 600, 1024, 9, "f16"
    log("static workspace few tokens")
    w = nm_inputs.normal_half((R, K), 0.02, dt, 81, 0, 1)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 81, 1, 1)
    perm = nm_inputs.random_permutation(K, 81, 1)
    vals, idx = nm.nm_compress(to_dev(w, dt), 2, 4)
    A = to_dev(act, dt)
    P = torch.from_numpy(perm).cuda()
    y = call_static(vals, idx, A, P, K, torch.float32)
    torch.cuda.synchronize()
    ref_vals, ref_idx = O.prune_pack(w, 2, 4)
    yref = O.spmm_ref(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm)
    assert_close(y, yref, error_bound(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm))
