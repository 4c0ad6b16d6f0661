"""Pins of the training-side oracle (oracle/nm_train.py), on the CPU.

Each check ties dX and dW to something other than their own formulas:
  * exact finite differences through the forward oracle: with integer inputs
    the loss L = sum G * Yt is exact in fp64 and linear in each input, so
    adding 1 to one activation (or one stored value) changes L by exactly that
    input's gradient;
  * the bilinear identities sum G*Yt = sum dX*act = sum dW*values on random
    inputs (every term of the loss is counted once in each);
  * a hand-worked example on the pages' worked row.
"""
import numpy as np
import pytest

import nm_inputs
from oracle import nm_oracle as O
from oracle import nm_train as TR


def ints(shape, lo, hi, seed, dt="f16"):
    rng = np.random.default_rng(seed)
    return nm_inputs.to_half_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32), dt)


def loss(values, idx, K, n, m, act, g, dt):
    """L = sum_{t, r} G[t, r] Yt[t, r], with Yt from the forward oracle."""
    yt = O.spmm_ref(values, idx, K, n, m, act, dt).T          # [T, R]
    return float(np.sum(O.half_bits_to_f64(g, dt) * yt))


def bump(bits, index, dt):
    """The same array with one element increased by 1 (exact for small integers)."""
    out = bits.copy()
    v = O.half_bits_to_f64(out[index:index + 1] if out.ndim == 1 else out[index][None], dt)[0] + 1.0
    out[index] = nm_inputs.to_half_bits(np.array([v], dtype=np.float32), dt)[0]
    return out


@pytest.mark.parametrize("n,m,R,K,T", [(2, 4, 5, 16, 4), (1, 4, 3, 32, 3), (1, 8, 4, 32, 3)])
def test_finite_differences_exact(n, m, R, K, T):
    dt = "f16"
    w = ints((R, K), -6, 6, R * K + n)
    act = ints((T, K), -5, 5, 7 + T)
    g = ints((T, R), -4, 4, 11 + R)
    values, idx = O.prune_pack(w, n, m)
    base = loss(values, idx, K, n, m, act, g, dt)
    dx = TR.spmm_dx_ref(values, idx, K, n, m, g, dt)
    for t in range(T):
        for k in range(K):
            a2 = act.copy()
            a2[t] = bump(act[t], k, dt)
            assert loss(values, idx, K, n, m, a2, g, dt) - base == dx[t, k]
    dw = TR.spmm_dw_ref(idx, K, n, m, g, act, dt)
    S = values.shape[1]
    for r in range(R):
        for s in range(S):
            v2 = values.copy()
            v2[r] = bump(values[r], s, dt)
            assert loss(v2, idx, K, n, m, act, g, dt) - base == dw[r, s]


@pytest.mark.parametrize("n,m,dt", [(2, 4, "bf16"), (1, 4, "f16"), (1, 8, "bf16")])
def test_bilinear_identities(n, m, dt):
    R, K, T = 48, 128, 20
    w = nm_inputs.normal_half((R, K), 1.0, dt, 90, 0, n * m)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 90, 1, n * m)
    g = nm_inputs.normal_half((T, R), 1.0, dt, 90, 4, n * m)
    values, idx = O.prune_pack(w, n, m)
    L = loss(values, idx, K, n, m, act, g, dt)
    dx = TR.spmm_dx_ref(values, idx, K, n, m, g, dt)
    dw = TR.spmm_dw_ref(idx, K, n, m, g, act, dt)
    assert np.sum(dx * O.half_bits_to_f64(act, dt)) == pytest.approx(L, rel=1e-12)
    assert np.sum(dw * O.half_bits_to_f64(values, dt)) == pytest.approx(L, rel=1e-12)


def test_worked_row():
    # the worked row keeps positions [[0, 3], [1, 2]]: columns 0, 3, 5, 6
    row = np.array([[0.5, 0.0, 0.0, -2.0, 0.0, 3.0, -1.0, 0.0]], dtype=np.float32)
    w = nm_inputs.to_half_bits(row, "f16")
    values, idx = O.prune_pack(w, 2, 4)
    assert TR.stored_columns(idx, 8, 2, 4).tolist() == [[0, 3, 5, 6]]
    g = nm_inputs.to_half_bits(np.array([[2.0]], dtype=np.float32), "f16")            # [T=1, R=1]
    act = nm_inputs.to_half_bits(np.arange(1, 9, dtype=np.float32)[None], "f16")       # [1, 8]
    assert TR.spmm_dx_ref(values, idx, 8, 2, 4, g, "f16").tolist() == [[1, 0, 0, -4, 0, 6, -2, 0]]
    assert TR.spmm_dw_ref(idx, 8, 2, 4, g, act, "f16").tolist() == [[2, 8, 12, 14]]


def test_zero_survivor_gets_its_gradient():
    # T2: a group with one non-zero still stores two slots; the zero slot's
    # gradient is G times the activation at its column
    row = np.array([[0.0, 0.0, 5.0, 0.0]], dtype=np.float32)
    w = nm_inputs.to_half_bits(row, "f16")
    values, idx = O.prune_pack(w, 2, 4)
    cols = TR.stored_columns(idx, 4, 2, 4)
    assert cols.tolist() == [[0, 2]]      # ties among the zeros go to the lowest position
    g = nm_inputs.to_half_bits(np.array([[3.0]], dtype=np.float32), "f16")
    act = nm_inputs.to_half_bits(np.array([[1.0, 2.0, 4.0, 8.0]], dtype=np.float32), "f16")
    assert TR.spmm_dw_ref(idx, 4, 2, 4, g, act, "f16").tolist() == [[3.0, 12.0]]
