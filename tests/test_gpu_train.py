"""Training-side products on MI355X (nm_spmm_dx, nm_spmm_dw) against the oracle.

dX = G W_nm and the packed dW, through the C ABI, element by element against
the fp64 oracle (oracle/nm_train.py): max floored relative error <= 1e-2 and
every element within the fp32 summation bound (sum of n products of two
16-bit floats, each exact in fp32, in any order: n * 2^-23 * sum |terms|);
exact on small integers; ragged R, K and T and NaN in the padding of G and act
(which must not reach a valid output); sampled rows
at the 4096 x 4096 x 2048 size the benchmark times.
"""
import numpy as np
import pytest

import nm_inputs
import structured_sparse_gemm_nm_amd as nm
from oracle import nm_oracle as O
from oracle import nm_train as TR
from gpu_util import assert_close, log, to_dev, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

U = 2.0 ** -23


def dx_bound(vals, idx, K, n, m, g, dt):
    wd = np.abs(O.half_bits_to_f64(O.decompress(vals, idx, K, n, m), dt))
    ga = np.abs(O.half_bits_to_f64(g, dt))
    return (g.shape[1] * U) * (ga @ wd) + 1e-30            # [T, K]


def dw_bound(idx, K, n, m, g, act, dt):
    ga = np.abs(O.half_bits_to_f64(g, dt))
    xa = np.abs(O.half_bits_to_f64(act, dt))
    full = (g.shape[0] * U) * (ga.T @ xa) + 1e-30           # [R, K]
    return np.take_along_axis(full, TR.stored_columns(idx, K, n, m), axis=1)


def case(R, K, T, dt, seed, sw=1.0):
    w = nm_inputs.normal_half((R, K), sw, dt, 70, 0, seed)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 70, 1, seed)
    g = nm_inputs.normal_half((T, R), 1.0, dt, 70, 4, seed)
    return w, act, g


# R % 8 == 0 and K % 32 == 0 (the products' shape rule); R below, at and past
# a multiple of the 64-row chunk, K tiles of 128 with and without a partial
# last one, ragged T, T = 1
SHAPES = [(256, 256, 128), (304, 512, 200), (136, 416, 77), (64, 128, 1), (1000, 1056, 333), (72, 4096, 64)]


@pytest.mark.parametrize("R,K,T", SHAPES)
@pytest.mark.parametrize("n,m", nm.PATTERNS)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_dx_against_oracle(R, K, T, n, m, dt):
    log(f"dx R={R} K={K} T={T} {n}:{m} {dt}")
    w, _, g = case(R, K, T, dt, R + K + T + n * m)
    vals, idx = O.prune_pack(w, n, m)
    dv, di = to_dev(vals, dt), torch.from_numpy(idx.view(np.int32)).cuda()
    dx = nm.nm_spmm_dx(dv, di, to_dev(g, dt), K, n, m)
    dxh = nm.nm_spmm_dx(dv, di, to_dev(g, dt), K, n, m, out_dtype=torch_dtype(dt))
    torch.cuda.synchronize()
    ref = TR.spmm_dx_ref(vals, idx, K, n, m, g, dt)
    b = dx_bound(vals, idx, K, n, m, g, dt)
    assert_close(dx, ref.T, b.T)
    assert_close(dxh, ref.T, b.T, out_half=dt)


@pytest.mark.parametrize("R,K,T", SHAPES)
@pytest.mark.parametrize("n,m", nm.PATTERNS)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_dw_against_oracle(R, K, T, n, m, dt):
    log(f"dw R={R} K={K} T={T} {n}:{m} {dt}")
    w, act, g = case(R, K, T, dt, R * 3 + K + T + n * m)
    _, idx = O.prune_pack(w, n, m)
    di = torch.from_numpy(idx.view(np.int32)).cuda()
    dw = nm.nm_spmm_dw(di, to_dev(g, dt), to_dev(act, dt), K, n, m)
    dwh = nm.nm_spmm_dw(di, to_dev(g, dt), to_dev(act, dt), K, n, m, out_dtype=torch_dtype(dt))
    torch.cuda.synchronize()
    ref = TR.spmm_dw_ref(idx, K, n, m, g, act, dt)
    b = dw_bound(idx, K, n, m, g, act, dt)
    assert_close(dw.t(), ref, b)
    assert_close(dwh.t(), ref, b, out_half=dt)


@pytest.mark.parametrize("n,m", nm.PATTERNS)
def test_exact_on_integers(n, m):
    # integer inputs small enough that every sum is exact in fp32
    log(f"dx/dw integers {n}:{m}")
    R, K, T = 200, 256, 150
    w = nm_inputs.integer_half((R, K), -6, 6, "f16", 71, 0, n * m)
    act = nm_inputs.integer_half((T, K), -5, 5, "f16", 71, 1, n * m)
    g = nm_inputs.integer_half((T, R), -4, 4, "f16", 71, 4, n * m)
    vals, idx = O.prune_pack(w, n, m)
    di = torch.from_numpy(idx.view(np.int32)).cuda()
    dx = nm.nm_spmm_dx(to_dev(vals, "f16"), di, to_dev(g, "f16"), K, n, m)
    dw = nm.nm_spmm_dw(di, to_dev(g, "f16"), to_dev(act, "f16"), K, n, m)
    torch.cuda.synchronize()
    assert np.array_equal(dx.cpu().numpy().astype(np.float64), TR.spmm_dx_ref(vals, idx, K, n, m, g, "f16"))
    assert np.array_equal(dw.cpu().numpy().astype(np.float64), TR.spmm_dw_ref(idx, K, n, m, g, act, "f16"))


@pytest.mark.parametrize("R,K,T", [(136, 256, 100), (256, 416, 70)])
def test_nan_padding_never_reaches_outputs(R, K, T):
    # G and act live inside wider buffers whose extra columns hold NaN
    log(f"dx/dw NaN padding R={R} K={K} T={T}")
    dt = "bf16"
    w, act, g = case(R, K, T, dt, 5 + R)
    vals, idx = O.prune_pack(w, 2, 4)
    nan = 0x7FC0
    gp = np.full((T, R + 24), nan, dtype=np.uint16)
    gp[:, :R] = g
    ap = np.full((T, K + 16), nan, dtype=np.uint16)
    ap[:, :K] = act
    G = to_dev(gp, dt)[:, :R]
    A = to_dev(ap, dt)[:, :K]
    di = torch.from_numpy(idx.view(np.int32)).cuda()
    dx = nm.nm_spmm_dx(to_dev(vals, dt), di, G, K, 2, 4)
    dw = nm.nm_spmm_dw(di, G, A, K, 2, 4)
    torch.cuda.synchronize()
    assert_close(dx, TR.spmm_dx_ref(vals, idx, K, 2, 4, g, dt).T, dx_bound(vals, idx, K, 2, 4, g, dt).T)
    assert_close(dw.t(), TR.spmm_dw_ref(idx, K, 2, 4, g, act, dt), dw_bound(idx, K, 2, 4, g, act, dt))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_rows_past_R_contribute_nothing(dt):
    # R = 72 leaves 56 rows of the last 64-row chunk past R.  Row 0 starts
    # with survivors 1.0 and 2.0, whose bit patterns OR'ed together are +Inf
    # in both 16-bit types: a row past R that picked up row 0's values instead
    # of zeros would put Inf (and, times a zero gradient row, NaN) into dX
    log(f"dx rows past R {dt}")
    R, K, T = 72, 256, 96
    w, _, g = case(R, K, T, dt, 12)
    w[0, :4] = nm_inputs.to_half_bits(np.array([1.0, 2.0, 0.0, 0.0], dtype=np.float32), dt)
    vals, idx = O.prune_pack(w, 2, 4)
    dx = nm.nm_spmm_dx(to_dev(vals, dt), torch.from_numpy(idx.view(np.int32)).cuda(), to_dev(g, dt), K, 2, 4)
    torch.cuda.synchronize()
    assert_close(dx, TR.spmm_dx_ref(vals, idx, K, 2, 4, g, dt).T, dx_bound(vals, idx, K, 2, 4, g, dt).T)


def test_caller_outputs_filled_in_place():
    log("dx/dw caller outputs")
    R, K, T, dt = 128, 256, 64, "f16"
    w, act, g = case(R, K, T, dt, 9)
    vals, idx = O.prune_pack(w, 1, 4)
    di = torch.from_numpy(idx.view(np.int32)).cuda()
    out_x = torch.full((T, K), 7.0, dtype=torch.float32, device="cuda")
    out_w = torch.full((R, K // 4), 7.0, dtype=torch.float32, device="cuda")
    assert nm.nm_spmm_dx(to_dev(vals, dt), di, to_dev(g, dt), K, 1, 4, out=out_x) is out_x
    assert nm.nm_spmm_dw(di, to_dev(g, dt), to_dev(act, dt), K, 1, 4, out=out_w) is out_w
    torch.cuda.synchronize()
    assert_close(out_x, TR.spmm_dx_ref(vals, idx, K, 1, 4, g, dt).T)
    assert_close(out_w.t(), TR.spmm_dw_ref(idx, K, 1, 4, g, act, dt))


def test_workload_size_sampled():
    # the benchmark's 4096 x 4096 x 2048 bf16 2:4 layer: sampled rows of dX
    # (tokens) and of dW (weight rows) against the oracle on those rows only
    log("dx/dw 4096x4096x2048 sampled")
    R, K, T, dt = 4096, 4096, 2048, "bf16"
    w = nm_inputs.normal_half((R, K), 0.02, dt, 72, 0)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 72, 1)
    g = nm_inputs.normal_half((T, R), 1.0, dt, 72, 4)
    vals, idx = O.prune_pack(w, 2, 4)
    di = torch.from_numpy(idx.view(np.int32)).cuda()
    dx = nm.nm_spmm_dx(to_dev(vals, dt), di, to_dev(g, dt), K, 2, 4).cpu().numpy()
    dw = nm.nm_spmm_dw(di, to_dev(g, dt), to_dev(act, dt), K, 2, 4).cpu().numpy()
    wd = O.half_bits_to_f64(O.decompress(vals, idx, K, 2, 4), dt)
    gf = O.half_bits_to_f64(g, dt)
    af = O.half_bits_to_f64(act, dt)
    cols = TR.stored_columns(idx, K, 2, 4)
    for t in (0, 1, 127, 128, 1000, 2047):
        ref = gf[t] @ wd
        err, _ = O.relative_error(dx[t].astype(np.float64)[None], ref[None])
        assert err <= 1e-2, ("dx", t, err)
    for r in (0, 63, 64, 2049, 4095):
        ref = (gf[:, r] @ af)[cols[r]]
        err, _ = O.relative_error(dw[r].astype(np.float64)[None], ref[None])
        assert err <= 1e-2, ("dw", r, err)


def test_empty_reductions_write_zeros():
    # R == 0: dX = G W_nm over no rows is all zeros; T == 0: dW over no tokens
    # is all zeros (both outputs are overwritten, never left as they were)
    log("dx R=0 / dw T=0")
    K, T, dt = 256, 40, torch.bfloat16
    vals = torch.empty((0, K // 2), dtype=dt, device="cuda")
    idx = torch.empty((0, K // 32), dtype=torch.int32, device="cuda")
    G = torch.zeros((T, 8), dtype=dt, device="cuda")[:, :0]          # [T, 0] with a row stride of 8
    out = torch.full((T, K), 5.0, dtype=torch.float32, device="cuda")
    assert nm.nm_spmm_dx(vals, idx, G, K, 2, 4, out=out) is out
    R = 64
    _, ridx = O.prune_pack(nm_inputs.normal_half((R, K), 1.0, "bf16", 73, 0), 2, 4)
    di = torch.from_numpy(ridx.view(np.int32)).cuda()
    G0 = torch.empty((0, R), dtype=dt, device="cuda")
    A0 = torch.empty((0, K), dtype=dt, device="cuda")
    outw = torch.full((R, K // 2), 5.0, dtype=torch.float32, device="cuda")
    assert nm.nm_spmm_dw(di, G0, A0, K, 2, 4, out=outw) is outw
    torch.cuda.synchronize()
    assert not out.any().item()
    assert not outw.any().item()
