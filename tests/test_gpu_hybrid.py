"""Hybrid dense / 2:4 tiles on MI355X: the HIP pack and product against the oracle.

Pack: values and index bytes bit-exact (the padding after the last index byte
is not part of the data).  Product: max floored relative error <= 1e-2 against
the fp64 oracle and every element inside the fp32 summation bound; all-dense
tiles exact on integers; all-2:4 tiles bit-identical to the 2:4 pipelined
kernel (same sparse MFMAs in the same K order); a sampled check at the
4096 x 4096 x 2048 size the benchmark times.
"""
import numpy as np
import pytest

import nm_inputs
import structured_sparse_gemm_nm_amd as nm
from oracle import nm_hybrid as H
from oracle import nm_oracle as O
from gpu_util import assert_close, bits_of, log, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def data_bytes(layout):
    rows = np.array([H.rows_of(b, layout.R, layout.tile_rows) for b in range(layout.row_meta.shape[0])])
    return int(np.sum(rows * layout.row_meta[:, 1]))


def hybrid_bound(vals, idx, R, K, tr, tc, flags, act, dt):
    wd = np.abs(O.half_bits_to_f64(H.hybrid_decompress(vals, idx, R, K, tr, tc, flags), dt))
    x = np.abs(O.half_bits_to_f64(act, dt)).T
    return (K * 2.0 ** -23) * (wd @ x) + 1e-30


def case(R, K, tr, tc, frac, dt, seed):
    flags = nm_inputs.tile_flags(H.tile_grid(R, K, tr, tc), frac, 60, seed)
    w = nm_inputs.normal_half((R, K), 0.02, dt, 60, 0, seed)
    return flags, w


@pytest.mark.parametrize("R,K,tr,tc,frac,dt", [(256, 256, 64, 64, 0.5, "f16"), (300, 512, 64, 128, 0.3, "bf16"),
                                               (1000, 1024, 128, 64, 0.7, "f16"), (64, 64, 64, 64, 1.0, "bf16"),
                                               (130, 512, 64, 256, 0.0, "f16")])
def test_hybrid_pack_bit_exact(R, K, tr, tc, frac, dt):
    log(f"hybrid pack R={R} K={K} tiles {tr}x{tc} dense {frac} {dt}")
    flags, w = case(R, K, tr, tc, frac, dt, R + K)
    L = nm.nm_hybrid_layout(R, K, tr, tc, flags)
    vals, idx = nm.nm_hybrid_compress(to_dev(w, dt), L)
    torch.cuda.synchronize()
    ref_v, ref_i = H.hybrid_pack(w, tr, tc, flags)
    assert np.array_equal(bits_of(vals), ref_v)
    nb = data_bytes(L)
    assert np.array_equal(idx.cpu().numpy()[:nb], ref_i[:nb])


@pytest.mark.parametrize("R,K,T,tr,tc,frac,dt,out", [(256, 512, 100, 64, 64, 0.5, "f16", "f32"),
                                                     (300, 1024, 257, 64, 128, 0.4, "bf16", "half"),
                                                     (1000, 768, 64, 128, 64, 0.6, "f16", "f32"),
                                                     (2048, 512, 640, 64, 64, 0.5, "bf16", "f32"),
                                                     (4100, 256, 1000, 64, 128, 0.25, "f16", "half"),
                                                     (4096, 768, 1024, 64, 64, 0.5, "bf16", "f32")])
def test_hybrid_spmm_against_oracle(R, K, T, tr, tc, frac, dt, out):
    # 64-wide tile-columns give tile-rows an odd number of 8-byte index runs,
    # so rows start at either half of a 16-byte index block
    log(f"hybrid spmm R={R} K={K} T={T} tiles {tr}x{tc} dense {frac} {dt} out={out}")
    flags, w = case(R, K, tr, tc, frac, dt, R + K + T)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 61, 1, R + K + T)
    L = nm.nm_hybrid_layout(R, K, tr, tc, flags)
    vals, idx = nm.nm_hybrid_compress(to_dev(w, dt), L)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    y = nm.nm_hybrid_spmm(vals, idx, L, to_dev(act, dt), out_dtype=tdt if out == "half" else None)
    torch.cuda.synchronize()
    ref_v, ref_i = H.hybrid_pack(w, tr, tc, flags)
    yref = H.hybrid_spmm_ref(ref_v, ref_i, R, K, tr, tc, flags, act, dt)
    assert_close(y, yref, hybrid_bound(ref_v, ref_i, R, K, tr, tc, flags, act, dt),
                 **({"out_half": dt} if out == "half" else {}))


@pytest.mark.parametrize("R,K,T,tr,tc", [(512, 256, 200, 64, 64), (4096, 256, 1024, 128, 128)])
def test_hybrid_all_dense_exact_integers(R, K, T, tr, tc):
    # the second shape takes the 256 x 64 tiles, the first the 128 x 64 ones
    log(f"hybrid all-dense integers R={R} K={K} T={T}")
    flags = np.ones(H.tile_grid(R, K, tr, tc), dtype=np.uint8)
    w = nm_inputs.integer_half((R, K), -8, 8, "f16", 62, 0, R)
    act = nm_inputs.integer_half((T, K), -8, 8, "f16", 62, 1, R)
    L = nm.nm_hybrid_layout(R, K, tr, tc, flags)
    vals, idx = nm.nm_hybrid_compress(to_dev(w, "f16"), L)
    y = nm.nm_hybrid_spmm(vals, idx, L, to_dev(act, "f16"))
    torch.cuda.synchronize()
    wi = w.view(np.float16).astype(np.int64)
    ai = act.view(np.float16).astype(np.int64)
    assert np.array_equal(y.cpu().numpy().astype(np.int64), ai @ wi.T)


@pytest.mark.parametrize("R,K,T,dt", [(512, 512, 256, "f16"), (4096, 512, 1024, "bf16")])
def test_hybrid_all_sparse_matches_2of4_kernel(R, K, T, dt):
    log(f"hybrid all-2:4 vs pipelined 2:4 kernel R={R} K={K} T={T} {dt}")
    tr, tc = 64, 64
    flags = np.zeros(H.tile_grid(R, K, tr, tc), dtype=np.uint8)
    w = nm_inputs.normal_half((R, K), 0.02, dt, 63, 0, R)
    act = to_dev(nm_inputs.normal_half((T, K), 1.0, dt, 63, 1, R), dt)
    L = nm.nm_hybrid_layout(R, K, tr, tc, flags)
    Wd = to_dev(w, dt)
    hv, hi = nm.nm_hybrid_compress(Wd, L)
    y = nm.nm_hybrid_spmm(hv, hi, L, act)
    v, i = nm.nm_compress(Wd, 2, 4)
    y24 = nm.nm_spmm(v, i, act, K, 2, 4, variant=2)
    torch.cuda.synchronize()
    assert torch.equal(hv.view(R, K // 2), v)
    assert torch.equal(y, y24)


def test_hybrid_workload_sampled():
    # the benchmark's shape: 4096 x 4096 bf16, 128 x 128 tiles, half of them
    # dense, 2048 tokens; the product on sampled rows
    log("hybrid 4096x4096x2048 sampled")
    R, K, T, tr, tc = 4096, 4096, 2048, 128, 128
    flags = nm_inputs.tile_flags(H.tile_grid(R, K, tr, tc), 0.5, 64, 0)
    w = nm_inputs.normal_half((R, K), 0.02, "bf16", 64, 0)
    act = nm_inputs.normal_half((T, K), 1.0, "bf16", 64, 1)
    L = nm.nm_hybrid_layout(R, K, tr, tc, flags)
    vals, idx = nm.nm_hybrid_compress(to_dev(w, "bf16"), L)
    y = nm.nm_hybrid_spmm(vals, idx, L, to_dev(act, "bf16"))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 1000, 2047, 2048, 3071, 4000, 4095])
    # the oracle on the sampled rows' tile-rows only (each a weight of its own)
    yv = y.cpu().numpy()
    for r in rows:
        b = r // tr
        sub_w = w[b * tr:(b + 1) * tr]
        sv, si = H.hybrid_pack(sub_w, tr, tc, flags[b:b + 1])
        yref = H.hybrid_spmm_ref(sv, si, tr, K, tr, tc, flags[b:b + 1], act, "bf16")[r - b * tr]
        err, _ = O.relative_error(yv[:, r].astype(np.float64), yref)
        assert err <= 1e-2, (r, err)
