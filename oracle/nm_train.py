"""CPU oracle for the training-side products of an N:M layer.

TEST INFRASTRUCTURE ONLY.  Like nm_oracle, this module exists to check the GPU
library; only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it, and it shares no code with the HIP path.

Sources: COE-592 lecture 04-2, "M:N sparsity on NVIDIA tensor cores", section
"The recipe", step 3: after the one-shot prune the network is retrained with
the zeros held fixed, so the pattern survives; thelatestinai.com "Structured
Sparsity" cards, the RNM-TD3 abstract: row-wise N:M sparsity is enforced
throughout training.  Training an N:M layer through its packed form needs two
products besides the forward one, and both are plain calculus on the forward
product of nm_oracle (Yt[t, r] = sum_k W_nm[r, k] act[t, k], readings R1-R7):
with G = dL/dYt ([T, R], the layout of Yt),

  dX   dL/dact[t, k]   = sum_r G[t, r] W_nm[r, k]        (G @ W_nm, [T, K]);
  dW   dL/dvalue[r, s] = sum_t G[t, r] act[t, k(r, s)]   ([R, S], the packed
       layout), where k(r, s) = M*(s div N) + p(r, s) is the column survivor s
       of row r came from.  Dropped weights are held at zero, so they have no
       gradient and none is formed: the gradient lives in the packed layout,
       one value per stored survivor, the shape an optimizer step on the
       packed values takes.

Readings taken where the pages are silent (T1-T2):
  T1  the gradient of the output arrives as G[T, R], the layout of the
      forward output, in the weights' 16-bit type; dX is written [T, K] like
      act and dW [R, S] like values; both are fp32 by default;
  T2  a stored survivor that holds a zero (R1) is a weight like any other:
      it gets its gradient.

Both are computed as their definitions: a dense fp64 product of the
decompressed weight, and a dense fp64 product G^T act sampled at the stored
positions.  Pinned by tests/test_oracle_train.py against the forward oracle
(exact finite differences on integer inputs, the adjoint identity), brute-force
loops and hand-worked values; no function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from . import nm_oracle as O


def stored_columns(idx: np.ndarray, K: int, n: int, m: int) -> np.ndarray:
    """k(r, s): the column of W each stored survivor came from, [R, S] int64."""
    S = O.survivors_per_row(K, n, m)
    positions = O.unpack_indices(np.asarray(idx), S, m)          # [R, S] in-group positions
    group = np.arange(S, dtype=np.int64) // n                    # survivor s lies in group s div N
    return group[None, :] * m + positions.astype(np.int64)


def spmm_dx_ref(values, idx, K: int, n: int, m: int, g_bits, dtype: str) -> np.ndarray:
    """dX = G @ W_nm in float64, [T, K] (G given as 16-bit bits [T, R])."""
    wd = O.half_bits_to_f64(O.decompress(values, idx, K, n, m), dtype)   # [R, K]
    g = O.half_bits_to_f64(np.asarray(g_bits, dtype=np.uint16), dtype)    # [T, R]
    return g @ wd


def spmm_dw_ref(idx, K: int, n: int, m: int, g_bits, act_bits, dtype: str) -> np.ndarray:
    """dW[r, s] = sum_t G[t, r] act[t, k(r, s)] in float64, [R, S]."""
    g = O.half_bits_to_f64(np.asarray(g_bits, dtype=np.uint16), dtype)    # [T, R]
    x = O.half_bits_to_f64(np.asarray(act_bits, dtype=np.uint16), dtype)  # [T, K]
    full = g.T @ x                                                         # [R, K]: every weight's gradient
    cols = stored_columns(idx, K, n, m)
    return np.take_along_axis(full, cols, axis=1)
