"""The column permutation on block-sparse and diagonal-sparse weights on
MI355X (nm_block_*, nm_diag_*) against the oracle (oracle/nm_hosts.py).

Packing bit-exact; products element by element within 1e-2 max floored
relative error and the fp32 summation bound (a sum of n products of two
16-bit floats, each exact in fp32, in any order: n * 2^-23 * sum |terms|),
with and without the permutation, fp16 / bf16, fp32 and half outputs; exact
on small integers; the map read inside the kernel equals the product on an
explicitly permuted copy bit for bit; empty structures, every block / every
diagonal kept, ragged tokens; sampled rows of the 3072 x 768 x 12608 layers
the benchmark times.
"""
import numpy as np
import pytest

import nm_inputs
import structured_sparse_gemm_nm_amd as nm
from oracle import nm_hosts as H
from oracle import nm_oracle as O
from gpu_util import assert_close, bits_of, log, to_dev, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

U = 2.0 ** -23


def bound(w_dense_bits, act_bits, dt, perm, n_terms):
    wd = np.abs(O.half_bits_to_f64(w_dense_bits, dt))
    x = np.abs(O.half_bits_to_f64(act_bits, dt))
    if perm is not None:
        x = x[:, np.asarray(perm, dtype=np.int64)]
    return (n_terms * U) * (wd @ x.T) + 1e-30                # [R, T]


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


# ---------------------------------------------------------------- block

def block_case(R, K, T, keep, dt, seed):
    w = nm_inputs.normal_half((R, K), 1.0, dt, 82, 0, seed)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 82, 1, seed)
    mask = nm_inputs.block_mask((R // 32, K // 32), keep, 82, seed)
    perm = nm_inputs.random_permutation(K, 82, seed)
    return w, act, mask, perm


# K <= 2048 runs the staged kernel (a token tile staged once in LDS), larger K
# the direct one
BLOCK_SHAPES = [(64, 96, 5, 0.5), (256, 768, 300, 0.1), (160, 224, 257, 0.4), (32, 32, 1, 1.0),
                (96, 512, 513, 1.0), (128, 256, 64, 0.0), (64, 2048, 45, 0.3), (96, 2112, 270, 0.2)]


@pytest.mark.parametrize("R,K,T,keep", BLOCK_SHAPES)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("use_perm", [False, True])
def test_block_against_oracle(R, K, T, keep, dt, use_perm):
    log(f"block R={R} K={K} T={T} keep={keep} {dt} perm={use_perm}")
    w, act, mask, perm = block_case(R, K, T, keep, dt, R + K + T)
    p = perm if use_perm else None
    row_ptr, col = nm.nm_block_structure(R, K, mask)
    rp, cl = dev_i32(row_ptr), dev_i32(col)
    vals = nm.nm_block_compress(to_dev(w, dt), rp, cl)
    ref_vals = H.block_pack(w, row_ptr, col)
    assert np.array_equal(bits_of(vals).reshape(ref_vals.shape), ref_vals)
    A = to_dev(act, dt)
    pd = dev_i32(perm) if use_perm else None
    y = nm.nm_block_spmm(vals, rp, cl, A, perm=pd)
    yh = nm.nm_block_spmm(vals, rp, cl, A, perm=pd, out_dtype=torch_dtype(dt))
    torch.cuda.synchronize()
    ref = H.block_spmm_ref(ref_vals, row_ptr, col, R, K, act, dt, perm=p)
    b = bound(H.block_dense(ref_vals, row_ptr, col, R, K), act, dt, p, K)
    if not mask.any():
        assert not y.any().item() and not yh.any().item()
        return
    assert_close(y, ref, b)
    assert_close(yh, ref, b, out_half=dt)


def test_block_map_equals_explicit_permutation():
    # the map read inside the kernel gives the same bits as the product of the
    # unmapped kernel on a copy of act permuted beforehand
    R, K, T, dt = 128, 256, 200, "bf16"
    w, act, mask, perm = block_case(R, K, T, 0.3, dt, 7)
    row_ptr, col = nm.nm_block_structure(R, K, mask)
    rp, cl = dev_i32(row_ptr), dev_i32(col)
    vals = nm.nm_block_compress(to_dev(w, dt), rp, cl)
    A = to_dev(act, dt)
    y_map = nm.nm_block_spmm(vals, rp, cl, A, perm=dev_i32(perm))
    y_copy = nm.nm_block_spmm(vals, rp, cl, A[:, torch.from_numpy(perm.astype(np.int64)).cuda()].contiguous())
    y_id = nm.nm_block_spmm(vals, rp, cl, A, perm=dev_i32(np.arange(K)))
    y_plain = nm.nm_block_spmm(vals, rp, cl, A)
    torch.cuda.synchronize()
    assert torch.equal(y_map, y_copy)
    assert torch.equal(y_id, y_plain)


def test_block_exact_on_integers():
    R, K, T = 96, 320, 77
    w = nm_inputs.integer_half((R, K), -6, 6, "f16", 83, 0)
    act = nm_inputs.integer_half((T, K), -5, 5, "f16", 83, 1)
    mask = nm_inputs.block_mask((R // 32, K // 32), 0.5, 83)
    perm = nm_inputs.random_permutation(K, 83)
    row_ptr, col = nm.nm_block_structure(R, K, mask)
    rp, cl = dev_i32(row_ptr), dev_i32(col)
    vals = nm.nm_block_compress(to_dev(w, "f16"), rp, cl)
    y = nm.nm_block_spmm(vals, rp, cl, to_dev(act, "f16"), perm=dev_i32(perm))
    torch.cuda.synchronize()
    ref = H.block_spmm_ref(H.block_pack(w, row_ptr, col), row_ptr, col, R, K, act, "f16", perm=perm)
    assert np.array_equal(y.cpu().numpy().astype(np.float64).T, ref)


def test_block_nan_padding_never_read():
    # act inside a wider buffer whose extra columns hold NaN
    R, K, T, dt = 64, 128, 40, "bf16"
    w, act, mask, perm = block_case(R, K, T, 0.5, dt, 11)
    mask[0, 3] = 1
    ap = np.full((T, K + 32), 0x7FC0, dtype=np.uint16)
    ap[:, :K] = act
    A = to_dev(ap, dt)[:, :K]
    row_ptr, col = nm.nm_block_structure(R, K, mask)
    rp, cl = dev_i32(row_ptr), dev_i32(col)
    vals = nm.nm_block_compress(to_dev(w, dt), rp, cl)
    for p in (None, perm):
        y = nm.nm_block_spmm(vals, rp, cl, A, perm=dev_i32(p) if p is not None else None)
        torch.cuda.synchronize()
        rv = H.block_pack(w, row_ptr, col)
        assert_close(y, H.block_spmm_ref(rv, row_ptr, col, R, K, act, dt, perm=p),
                     bound(H.block_dense(rv, row_ptr, col, R, K), act, dt, p, K))


def test_block_workload_sampled():
    wl = nm_inputs.WORKLOADS[10]
    log("block workload 10 sampled")
    R, K, T = wl.R, wl.K, wl.Ts[0]
    w, act, mask, perm = wl.weights(), wl.activations(T), wl.block_mask(), wl.permutation()
    row_ptr, col = nm.nm_block_structure(R, K, mask)
    rp, cl = dev_i32(row_ptr), dev_i32(col)
    vals = nm.nm_block_compress(to_dev(w, wl.dtype), rp, cl)
    y = nm.nm_block_spmm(vals, rp, cl, to_dev(act, wl.dtype), perm=dev_i32(perm)).cpu().numpy()
    rv = H.block_pack(w, row_ptr, col)
    assert np.array_equal(bits_of(vals).reshape(rv.shape), rv)
    toks = np.array([0, 1, 255, 256, 6000, T - 1])
    ref = H.block_spmm_ref(rv, row_ptr, col, R, K, act[toks], wl.dtype, perm=perm)
    err, _ = O.relative_error(y[toks].astype(np.float64).T, ref)
    assert err <= 1e-2


# ---------------------------------------------------------------- diagonal

def diag_case(R, K, T, D, dt, seed):
    w = nm_inputs.normal_half((R, K), 1.0, dt, 84, 0, seed)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 84, 1, seed)
    offs = nm_inputs.diag_offsets(K, D, 84, seed)
    perm = nm_inputs.random_permutation(K, 84, seed)
    return w, act, offs, perm


# R >= 4K and R >= 2K group 4 / 2 rows that share their columns (rows past R
# in the last group: 700 x 160, 500 x 128, 300 x 96; R a multiple of 4K: 512 x 128)
DIAG_SHAPES = [(100, 64, 5, 8), (1000, 768, 300, 77), (257, 1792, 33, 300), (64, 64, 1, 64), (40, 128, 70, 1),
               (300, 96, 31, 0), (700, 160, 45, 33), (500, 128, 40, 17), (512, 128, 64, 9), (256, 128, 3, 2)]


@pytest.mark.parametrize("R,K,T,D", DIAG_SHAPES)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("use_perm", [False, True])
def test_diag_against_oracle(R, K, T, D, dt, use_perm):
    log(f"diag R={R} K={K} T={T} D={D} {dt} perm={use_perm}")
    w, act, offs, perm = diag_case(R, K, T, D, dt, R + K + T + D)
    p = perm if use_perm else None
    od = dev_i32(offs)
    vals = nm.nm_diag_compress(to_dev(w, dt), od)
    ref_vals = H.diag_pack(w, offs)
    assert np.array_equal(bits_of(vals).reshape(ref_vals.shape), ref_vals)
    A = to_dev(act, dt)
    pd = dev_i32(perm) if use_perm else None
    y = nm.nm_diag_spmm(vals, od, A, perm=pd)
    yh = nm.nm_diag_spmm(vals, od, A, perm=pd, out_dtype=torch_dtype(dt))
    torch.cuda.synchronize()
    if D == 0:
        assert not y.any().item() and not yh.any().item()
        return
    ref = H.diag_spmm_ref(ref_vals, offs, R, K, act, dt, perm=p)
    b = bound(H.diag_dense(ref_vals, offs, R, K), act, dt, p, D)
    assert_close(y, ref, b)
    assert_close(yh, ref, b, out_half=dt)


@pytest.mark.parametrize("R,K", [(500, 256), (1000, 240)])
def test_diag_map_equals_explicit_permutation(R, K):
    T, dt = 90, "f16"
    w, act, offs, perm = diag_case(R, K, T, 40, dt, 5)
    od = dev_i32(offs)
    vals = nm.nm_diag_compress(to_dev(w, dt), od)
    A = to_dev(act, dt)
    y_map = nm.nm_diag_spmm(vals, od, A, perm=dev_i32(perm))
    y_copy = nm.nm_diag_spmm(vals, od, A[:, torch.from_numpy(perm.astype(np.int64)).cuda()].contiguous())
    y_id = nm.nm_diag_spmm(vals, od, A, perm=dev_i32(np.arange(K)))
    y_plain = nm.nm_diag_spmm(vals, od, A)
    torch.cuda.synchronize()
    assert torch.equal(y_map, y_copy)
    assert torch.equal(y_id, y_plain)


@pytest.mark.parametrize("R,K,D", [(300, 512, 60), (900, 200, 61), (450, 200, 7)])
def test_diag_exact_on_integers(R, K, D):
    T = 45
    w = nm_inputs.integer_half((R, K), -6, 6, "bf16", 85, 0)
    act = nm_inputs.integer_half((T, K), -5, 5, "bf16", 85, 1)
    offs = nm_inputs.diag_offsets(K, D, 85)
    perm = nm_inputs.random_permutation(K, 85)
    od = dev_i32(offs)
    vals = nm.nm_diag_compress(to_dev(w, "bf16"), od)
    y = nm.nm_diag_spmm(vals, od, to_dev(act, "bf16"), perm=dev_i32(perm))
    torch.cuda.synchronize()
    ref = H.diag_spmm_ref(H.diag_pack(w, offs), offs, R, K, act, "bf16", perm=perm)
    assert np.array_equal(y.cpu().numpy().astype(np.float64).T, ref)


def test_diag_workload_sampled():
    wl = nm_inputs.WORKLOADS[11]
    log("diag workload 11 sampled")
    R, K, T = wl.R, wl.K, wl.Ts[0]
    w, act, offs, perm = wl.weights(), wl.activations(T), wl.diag_offsets(), wl.permutation()
    od = dev_i32(offs)
    vals = nm.nm_diag_compress(to_dev(w, wl.dtype), od)
    y = nm.nm_diag_spmm(vals, od, to_dev(act, wl.dtype), perm=dev_i32(perm)).cpu().numpy()
    rv = H.diag_pack(w, offs)
    assert np.array_equal(bits_of(vals).reshape(rv.shape), rv)
    toks = np.array([0, 1, 31, 32, 6000, T - 1])
    ref = H.diag_spmm_ref(rv, offs, R, K, act[toks], wl.dtype, perm=perm)
    err, _ = O.relative_error(y[toks].astype(np.float64).T, ref)
    assert err <= 1e-2
