"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library through its binding, compare with the oracle."""
import functools
import sys

import numpy as np

import nm_inputs
from oracle import nm_oracle as O


def log(msg):
    """Name the case on the real stderr before each GPU step (bypasses capture)."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def torch_dtype(dt):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16}[dt]


def to_dev(bits, dt):
    """uint16 bit patterns -> fp16/bf16 device tensor with the same bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dt)).cuda()


def bits_of(t):
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def words_of(t):
    return t.detach().cpu().numpy().view(np.uint32)


@functools.lru_cache(maxsize=8)
def oracle_pack(wid, n, m):
    w = nm_inputs.WORKLOADS[wid].weights()
    vals, idx = O.prune_pack(w, n, m)
    return w, vals, idx


def error_bound(values, idx, K, n, m, act_bits, dt, perm=None, out_half=None):
    """Elementwise bound on |Y - Yref| for fp32 accumulation in any order.

    Products of two 16-bit floats are exact in fp32; a sum of S such terms in
    any order with rounding unit u = 2^-23 (allowing round-toward-zero) is off
    by at most S*u*sum|w x|.  Half outputs add one rounding of |y|.
    """
    wd = np.abs(O.half_bits_to_f64(O.decompress(values, idx, K, n, m), dt))
    x = np.abs(O.half_bits_to_f64(act_bits, dt)).T
    if perm is not None:
        x = x[np.asarray(perm, dtype=np.int64), :]
    S = K // m * n
    bound = (S * 2.0 ** -23) * (wd @ x) + 1e-30
    return bound


def assert_close(y_gpu_tr, yref, bound=None, out_half=None, tol=1e-2):
    """y_gpu_tr is the device output [T, R]; yref is [R, T] float64."""
    y = y_gpu_tr.float().cpu().numpy().astype(np.float64).T
    assert y.shape == yref.shape
    assert np.all(np.isfinite(y))
    max_rel, norm_rel = O.relative_error(y, yref)
    assert max_rel <= tol, f"max relative error {max_rel:.3e} > {tol}"
    if bound is not None:
        b = bound
        if out_half == "f16":
            b = b + np.abs(yref) * 2.0 ** -10 + 2.0 ** -24
        elif out_half == "bf16":
            b = b + np.abs(yref) * 2.0 ** -7 + 1e-38
        err = np.abs(y - yref)
        worst = np.max(err / b)
        assert worst <= 1.0, f"error exceeds the fp32 summation bound by {worst:.3f}x"
    return max_rel, norm_rel
