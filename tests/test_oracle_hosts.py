"""Pins of the block / diagonal host-structure oracle (oracle/nm_hosts.py), CPU.

Each check ties the oracle to something other than its own formulas: explicit
permutation matrices, brute-force loops, structures that reduce to a dense
matrix (every block kept, all K diagonals) or to a diagonal / cyclic-shift
matrix, and hand-worked layouts.  A few plausible mistakes are planted to show
the pins catch them.
"""
import numpy as np
import pytest

import nm_inputs
from oracle import nm_hosts as H
from oracle import nm_oracle as O


def f64(bits, dt="f16"):
    return O.half_bits_to_f64(np.asarray(bits), dt)


def ints(shape, lo, hi, seed, dt="f16"):
    rng = np.random.default_rng(seed)
    return nm_inputs.to_half_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32), dt)


def perm_matrix(perm):
    """Pi with Pi[k, perm[k]] = 1, so (W Pi x)[r] = sum_k W[r, k] x[perm[k]]."""
    K = len(perm)
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0
    return P


# ---------------------------------------------------------------- block

def test_block_worked_layout():
    # 64 x 96 weight, blocks (0, 2) and (1, 0), (1, 1) kept
    mask = np.array([[0, 0, 1], [1, 1, 0]])
    row_ptr, col = H.block_structure(mask)
    assert row_ptr.tolist() == [0, 1, 3]
    assert col.tolist() == [2, 0, 1]
    w = ints((64, 96), -3, 3, 1)
    vals = H.block_pack(w, row_ptr, col)
    assert vals.shape == (3, 32, 32)
    assert np.array_equal(vals[0], w[0:32, 64:96])
    assert np.array_equal(vals[1], w[32:64, 0:32])
    assert np.array_equal(vals[2], w[32:64, 32:64])
    dense = H.block_dense(vals, row_ptr, col, 64, 96)
    keep = np.kron(mask, np.ones((32, 32))).astype(bool)
    assert np.array_equal(dense[keep], w[keep]) and not dense[~keep].any()


def test_block_all_kept_is_the_dense_product():
    R, K, T = 64, 128, 9
    w = nm_inputs.normal_half((R, K), 1.0, "bf16", 80, 0)
    act = nm_inputs.normal_half((T, K), 1.0, "bf16", 80, 1)
    row_ptr, col = H.block_structure(np.ones((2, 4)))
    vals = H.block_pack(w, row_ptr, col)
    y = H.block_spmm_ref(vals, row_ptr, col, R, K, act, "bf16")
    assert np.allclose(y, np.matmul(f64(w, "bf16"), f64(act, "bf16").T), rtol=1e-13, atol=1e-13)


def test_block_none_kept_is_zero():
    row_ptr, col = H.block_structure(np.zeros((2, 3)))
    vals = H.block_pack(np.zeros((64, 96), dtype=np.uint16), row_ptr, col)
    act = ints((5, 96), -3, 3, 2)
    assert not H.block_spmm_ref(vals, row_ptr, col, 64, 96, act, "f16").any()


def test_block_brute_force_with_perm():
    # pure-Python loops over the kept blocks against the oracle, and against
    # the explicit Pi matrix: Y = W_dense Pi act^T
    R, K, T = 64, 96, 3
    rng = np.random.default_rng(5)
    mask = rng.random((2, 3)) < 0.5
    mask[0, 1] = True
    row_ptr, col = H.block_structure(mask)
    w = ints((R, K), -4, 4, 6)
    act = ints((T, K), -3, 3, 7)
    perm = rng.permutation(K)
    vals = H.block_pack(w, row_ptr, col)
    y = H.block_spmm_ref(vals, row_ptr, col, R, K, act, "f16", perm=perm)
    wf, xf = f64(w), f64(act)
    ref = np.zeros((R, T))
    for b in range(2):
        for c in range(3):
            if not mask[b, c]:
                continue
            for i in range(32):
                for t in range(T):
                    s = 0.0
                    for j in range(32):
                        s += wf[32 * b + i, 32 * c + j] * xf[t, perm[32 * c + j]]
                    ref[32 * b + i, t] += s
    assert np.array_equal(y, ref)
    dense = f64(H.block_dense(vals, row_ptr, col, R, K))
    assert np.array_equal(y, dense @ perm_matrix(perm) @ xf.T)


def test_block_identity_perm_equals_no_perm():
    R, K, T = 64, 64, 4
    row_ptr, col = H.block_structure(np.array([[1, 0], [1, 1]]))
    w = ints((R, K), -4, 4, 8)
    act = ints((T, K), -3, 3, 9)
    vals = H.block_pack(w, row_ptr, col)
    assert np.array_equal(H.block_spmm_ref(vals, row_ptr, col, R, K, act, "f16"),
                          H.block_spmm_ref(vals, row_ptr, col, R, K, act, "f16", perm=np.arange(K)))


# ---------------------------------------------------------------- diagonal

def test_diag_worked_shift():
    # R = K = 4, one diagonal at offset 1: W is the cyclic shift with values v
    v = np.array([[1.0, 2.0, 3.0, 4.0]], dtype=np.float32)
    vals = nm_inputs.to_half_bits(v, "f16")
    dense = f64(H.diag_dense(vals, [1], 4, 4))
    assert dense.tolist() == [[0, 1, 0, 0], [0, 0, 2, 0], [0, 0, 0, 3], [4, 0, 0, 0]]
    act = nm_inputs.to_half_bits(np.array([[10.0, 20.0, 30.0, 40.0]], dtype=np.float32), "f16")
    # y[r] = v[r] * x[(r + 1) mod 4]
    assert H.diag_spmm_ref(vals, [1], 4, 4, act, "f16")[:, 0].tolist() == [20.0, 60.0, 120.0, 40.0]
    # through perm = [3, 2, 1, 0]: y[r] = v[r] * x[perm[(r + 1) mod 4]]
    # = 1 * x[2], 2 * x[1], 3 * x[0], 4 * x[3]
    assert H.diag_spmm_ref(vals, [1], 4, 4, act, "f16", perm=[3, 2, 1, 0])[:, 0].tolist() == \
        [30.0, 40.0, 30.0, 160.0]


def test_diag_wraps_rows_past_K():
    # R = 6 > K = 4: row r of the offset-0 diagonal sits at column r mod 4
    cols = H.diag_columns([0, 3], 6, 4)
    assert cols.tolist() == [[0, 1, 2, 3, 0, 1], [3, 0, 1, 2, 3, 0]]


def test_diag_all_offsets_is_the_dense_product():
    # every entry of W lies on exactly one of the K diagonals
    R, K, T = 12, 8, 5
    w = nm_inputs.normal_half((R, K), 1.0, "f16", 81, 0)
    act = nm_inputs.normal_half((T, K), 1.0, "f16", 81, 1)
    offs = np.random.default_rng(3).permutation(K)
    vals = H.diag_pack(w, offs)
    assert np.array_equal(H.diag_dense(vals, offs, R, K), w)
    assert np.allclose(H.diag_spmm_ref(vals, offs, R, K, act, "f16"), f64(w) @ f64(act).T, rtol=1e-13, atol=1e-13)


def test_diag_main_diagonal_closed_form():
    # R = K, offset 0: Y^T[t, r] = v[r] * act[t, perm[r]]
    K, T = 16, 3
    v = ints((1, K), -5, 5, 10)
    act = ints((T, K), -5, 5, 11)
    perm = np.random.default_rng(12).permutation(K)
    y = H.diag_spmm_ref(v, [0], K, K, act, "f16", perm=perm)
    assert np.array_equal(y, (f64(v)[0][:, None] * f64(act)[:, perm].T))


def test_diag_brute_force_with_perm():
    R, K, T = 10, 8, 3
    offs = [0, 3, 5]
    w = ints((R, K), -4, 4, 13)
    act = ints((T, K), -3, 3, 14)
    perm = np.random.default_rng(15).permutation(K)
    vals = H.diag_pack(w, offs)
    y = H.diag_spmm_ref(vals, offs, R, K, act, "f16", perm=perm)
    wf, xf = f64(w), f64(act)
    ref = np.zeros((R, T))
    for r in range(R):
        for t in range(T):
            for o in offs:
                k = (r + o) % K
                ref[r, t] += wf[r, k] * xf[t, perm[k]]
    assert np.array_equal(y, ref)
    assert np.array_equal(y, f64(H.diag_dense(vals, offs, R, K)) @ perm_matrix(perm) @ xf.T)


# ---------------------------------------------------------------- planted mistakes

@pytest.mark.parametrize("mistake", ["offset_sign", "perm_inverse", "block_transposed"])
def test_planted_mistakes_fail_a_pin(monkeypatch, mistake):
    if mistake == "offset_sign":
        monkeypatch.setattr(H, "diag_columns", lambda o, R, K: (np.arange(R)[None, :] - np.asarray(o)[:, None]) % K)
        with pytest.raises(AssertionError):
            test_diag_worked_shift()
    elif mistake == "perm_inverse":
        monkeypatch.setattr(H, "permuted", lambda x, p: x if p is None else x[:, np.argsort(np.asarray(p))])
        with pytest.raises(AssertionError):
            test_block_brute_force_with_perm()
    else:
        orig = H.block_pack

        def transposed(w, row_ptr, col):
            return np.ascontiguousarray(np.swapaxes(orig(w, row_ptr, col), 1, 2))
        monkeypatch.setattr(H, "block_pack", transposed)
        with pytest.raises(AssertionError):
            test_block_worked_layout()
