"""CPU oracle for the permutation primitive on two other host structures:
block-sparse and diagonal-sparse weights.

TEST INFRASTRUCTURE ONLY.  Like nm_oracle, this module exists to check the GPU
library; only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it, and it shares no code with the HIP path.

Sources: searcharxiv.com author page, the SHUFFLESPARSE abstract (one learned
permutation, applied the same way to block, N:M and diagonal structures) and
the DynaDiag abstract (weights kept on a diagonal pattern); gist.science
"Technische Samenvatting: SHUFFLESPARSE", section "2. Methodologie" (the layer
computes y = (W Pi) x with W following a fixed structured pattern S) and the
item "Efficiëntie bij Inferentie" of "Belangrijke Technische Componenten" (the
hardened Pi is a precomputed index map through which the structured kernel
reads its input; no separate permutation pass).  The permutation convention
is nm_oracle's R7: Y^T[t, r] = sum_k W[r, k] act[t, perm[k]].

The pages name the two structures and nothing of their geometry or storage;
the readings taken (B1-B3, D1-D3):
  B1  block structure: W [R, K] is cut into 32 x 32 blocks on a regular grid
      (R and K multiples of 32); a block is kept whole or dropped.  Which
      blocks are kept is an input, a mask over the block grid (choosing it is
      training, out of scope);
  B2  block storage: block-sparse rows.  row_ptr[RB + 1] (int32): the kept
      blocks of block-row b are entries row_ptr[b] .. row_ptr[b + 1] - 1;
      col[nnzb] (int32): their block-columns, ascending within a block-row;
      values[nnzb, 32, 32]: each kept block row-major, the weights' bits
      unchanged;
  B3  block product: Y^T[t, r] = sum over kept blocks (r div 32, c) of
      sum_j values[blk, r mod 32, j] * act[t, perm[32 c + j]];
  D1  diagonal structure: W [R, K] is non-zero only on D wrap-around
      diagonals given by distinct offsets o_d in [0, K): row r of diagonal d
      sits at column (r + o_d) mod K (for R > K a diagonal wraps round K more
      than once, so every row holds exactly D weights);
  D2  diagonal storage: offsets[D] (int32, as given, any order) and
      values[D, R] with values[d, r] = W[r, (r + o_d) mod K];
  D3  diagonal product: Y^T[t, r] = sum_d values[d, r] * act[t, perm[(r + o_d) mod K]].

Every product below is its definition: the dense fp64 matrix the structure
stores, multiplied by the activations read through perm.  Pinned by
tests/test_oracle_hosts.py (explicit Pi matrices, brute-force loops, the
structures that reduce to a dense matrix or to a diagonal matrix, worked
examples); no function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from . import nm_oracle as O

BLOCK = 32  # B1: block edge


# ---------------------------------------------------------------------------
# block-sparse (B1-B3)
# ---------------------------------------------------------------------------

def block_structure(mask: np.ndarray):
    """B2: (row_ptr [RB + 1], col [nnzb]) from a kept-block mask [RB, KB]."""
    mask = np.asarray(mask).astype(bool)
    row_ptr = np.zeros(mask.shape[0] + 1, dtype=np.int32)
    cols = []
    for b in range(mask.shape[0]):
        kept = np.nonzero(mask[b])[0]             # ascending block-columns
        cols.extend(int(c) for c in kept)
        row_ptr[b + 1] = row_ptr[b] + len(kept)
    return row_ptr, np.array(cols, dtype=np.int32)


def block_pack(w_bits: np.ndarray, row_ptr, col) -> np.ndarray:
    """B2: the kept blocks of W (bits [R, K]) as values [nnzb, 32, 32]."""
    w = np.asarray(w_bits)
    values = np.zeros((len(col), BLOCK, BLOCK), dtype=w.dtype)
    for b in range(len(row_ptr) - 1):
        for blk in range(row_ptr[b], row_ptr[b + 1]):
            c = int(col[blk])
            values[blk] = w[BLOCK * b:BLOCK * (b + 1), BLOCK * c:BLOCK * (c + 1)]
    return values


def block_dense(values, row_ptr, col, R: int, K: int) -> np.ndarray:
    """The dense matrix a block-sparse W stores (bits; dropped blocks zero)."""
    values = np.asarray(values)
    w = np.zeros((R, K), dtype=values.dtype)
    for b in range(len(row_ptr) - 1):
        for blk in range(row_ptr[b], row_ptr[b + 1]):
            c = int(col[blk])
            w[BLOCK * b:BLOCK * (b + 1), BLOCK * c:BLOCK * (c + 1)] = values[blk]
    return w


def permuted(act_f64: np.ndarray, perm) -> np.ndarray:
    """act read through the index map: X'[t, k] = act[t, perm[k]] (R7)."""
    return act_f64 if perm is None else act_f64[:, np.asarray(perm, dtype=np.int64)]


def block_spmm_ref(values, row_ptr, col, R: int, K: int, act_bits, dtype: str, perm=None) -> np.ndarray:
    """B3 in float64, returned as Y [R, T] (Y^T transposed, like nm_oracle.spmm_ref)."""
    w = O.half_bits_to_f64(block_dense(values, row_ptr, col, R, K), dtype)
    x = permuted(O.half_bits_to_f64(np.asarray(act_bits, dtype=np.uint16), dtype), perm)
    return w @ x.T


# ---------------------------------------------------------------------------
# diagonal-sparse (D1-D3)
# ---------------------------------------------------------------------------

def diag_columns(offsets, R: int, K: int) -> np.ndarray:
    """D1: the column of row r on diagonal d, [D, R]."""
    o = np.asarray(offsets, dtype=np.int64)
    return (np.arange(R, dtype=np.int64)[None, :] + o[:, None]) % K


def diag_pack(w_bits: np.ndarray, offsets) -> np.ndarray:
    """D2: values[d, r] = W[r, (r + o_d) mod K]."""
    w = np.asarray(w_bits)
    R, K = w.shape
    cols = diag_columns(offsets, R, K)
    return w[np.arange(R)[None, :], cols]


def diag_dense(values, offsets, R: int, K: int) -> np.ndarray:
    """The dense matrix a diagonal-sparse W stores (bits; off the diagonals zero)."""
    values = np.asarray(values)
    w = np.zeros((R, K), dtype=values.dtype)
    cols = diag_columns(offsets, R, K)
    for d in range(cols.shape[0]):
        w[np.arange(R), cols[d]] = values[d]
    return w


def diag_spmm_ref(values, offsets, R: int, K: int, act_bits, dtype: str, perm=None) -> np.ndarray:
    """D3 in float64, returned as Y [R, T]."""
    w = O.half_bits_to_f64(diag_dense(values, offsets, R, K), dtype)
    x = permuted(O.half_bits_to_f64(np.asarray(act_bits, dtype=np.uint16), dtype), perm)
    return w @ x.T
