"""CPU oracle for N:M structured weight sparsity: prune, pack, decompress, GEMM.

TEST INFRASTRUCTURE ONLY.  This module exists to check the GPU library; only
the test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it.  The library itself never calls into it and there is no CPU
fallback through it.  It shares no code with the HIP path.

Plain NumPy, written for a reader to check against the pages by eye:

* Definition (COE-592 lecture 04-2, "M:N sparsity on NVIDIA tensor cores",
  opening section): along each row of W, every group of M consecutive weights
  keeps N of them; the worked row has survivor positions [[0, 3], [1, 2]];
  a pattern is written survivors:block-size.  The groups run along the row of
  W, which is the reduction axis of the GEMM.
* Pruning rule (same page, section "The recipe", step 2): in each group keep
  the weights with the largest absolute value, zero the others.
* Storage (same page, section "Where this sits among the three case
  studies"): survivors of a row are pushed left into a contiguous block of
  values; a small index per survivor records which slot of its group it came
  from (2 bits for groups of four).
* GEMM (same section): sparse weight matrix times dense matrix gives a dense
  matrix; only the weight operand is compressed.
* Permuted layer (SHUFFLESPARSE technical summary, section 2 "Methodologie"
  and the "Efficiency at inference" item of "Belangrijke Technische
  Componenten"): y = (W Pi) x, where the hardened permutation is applied as a
  precomputed index map on the input reads.

Readings taken where the pages are silent:
  R1  exactly N slots are stored per group (a slot may hold a zero);
  R2  magnitude is compared on the stored 16-bit value: key = bits & 0x7FFF,
      the sign bit dropped; equal keys go to the lower position;
  R3  positions inside a group are stored in ascending order;
  R4  index width b = ceil(log2 M) bits (2 for M = 4, 3 for M = 8);
  R5  each row's indices form an LSB-first bitstream: survivor s occupies bits
      [s*b, s*b + b); the row is zero-padded to whole little-endian uint32
      words;
  R6  activations arrive as act[T, K] (K-contiguous) and X = act^T;
  R7  with a permutation, y[r, t] = sum_k W[r, k] * act[t, perm[k]].

Parity pins: every function here is pinned by tests under tests/ (worked
row, 36-bit group cost, brute-force top-N, exhaustive ties, worked K = 8
product, identity and integer GEMMs, dense N = M case, explicit-matrix
permutation route; for int8: the 20-bit group cost, brute-force top-N by |w|
with -128 and ties, big-integer products; for E4M3: the decode against the
library's float8_e4m3fn and printed field values, brute-force top-N by |w|,
exact small-integer products).  No function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

F16 = "f16"
BF16 = "bf16"


# --------------------------------------------------------------------------
# 16-bit storage types
# --------------------------------------------------------------------------

def half_bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of fp16 / bf16 bit patterns (uint16)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def magnitude_keys(bits: np.ndarray) -> np.ndarray:
    """Reading R2: |w| as an integer key.

    fp16 and bf16 keep the sign in bit 15; for non-negative IEEE values the
    unsigned bit order is the magnitude order, so dropping the sign bit gives
    a key whose order is the order of |w| (+0 and -0 share key 0).
    """
    return (np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)).astype(np.int32)


# --------------------------------------------------------------------------
# Format arithmetic
# --------------------------------------------------------------------------

def index_bits(m: int) -> int:
    """Reading R4: bits needed to name one of M slots."""
    return max(1, int(m - 1).bit_length())


def survivors_per_row(K: int, n: int, m: int) -> int:
    return K // m * n


def idx_words_per_row(K: int, n: int, m: int) -> int:
    """uint32 words holding one row's index bitstream (reading R5)."""
    nbits = survivors_per_row(K, n, m) * index_bits(m)
    return (nbits + 31) // 32


# --------------------------------------------------------------------------
# Prune: choose the survivors of every group
# --------------------------------------------------------------------------

def select_survivors(w_bits: np.ndarray, n: int, m: int) -> np.ndarray:
    """Positions (0..m-1) of the n kept weights of each group, ascending.

    Returns int64 [R, K/m, n].  Within a group the weights are ranked by key
    (largest first); a stable sort of the negated keys leaves equal keys in
    position order, so ties go to the lower position (R2).  The first n of
    that ranking are kept and then put back in ascending order (R3).
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    R, K = w_bits.shape
    if K % m:
        raise ValueError("K must be a multiple of m")
    keys = magnitude_keys(w_bits).reshape(R, K // m, m)
    ranking = np.argsort(-keys, axis=-1, kind="stable")
    kept = np.sort(ranking[..., :n], axis=-1)
    return kept.astype(np.int64)


# --------------------------------------------------------------------------
# Pack: values pushed left, indices into a per-row bitstream
# --------------------------------------------------------------------------

def pack_values(w_bits: np.ndarray, positions: np.ndarray, m: int) -> np.ndarray:
    """values[r, g*n + j] = bits of W[r, g*m + positions[r, g, j]] (no arithmetic)."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    R, K = w_bits.shape
    G, n = positions.shape[1], positions.shape[2]
    groups = w_bits.reshape(R, G, m)
    vals = np.take_along_axis(groups, positions, axis=-1)
    return vals.reshape(R, G * n).copy()


def pack_indices(positions: np.ndarray, m: int) -> np.ndarray:
    """Reading R5: row bitstream, survivor s at bits [s*b, s*b+b), LSB first.

    Built as an explicit bit array: bit j of survivor s's position goes to
    stream bit s*b + j; the stream is zero-padded to 32-bit words and word w
    collects stream bits [32w, 32w + 32) with stream bit 32w + i at weight 2^i.
    """
    R = positions.shape[0]
    pos = positions.reshape(R, -1).astype(np.int64)
    S = pos.shape[1]
    b = index_bits(m)
    nwords = (S * b + 31) // 32
    stream = np.zeros((R, nwords * 32), dtype=np.uint64)
    for j in range(b):
        stream[:, j:S * b:b] = (pos >> j) & 1
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    words = (stream.reshape(R, nwords, 32) * weights).sum(axis=-1)
    return words.astype(np.uint32)


def prune_pack(w_bits: np.ndarray, n: int, m: int):
    """Magnitude top-n-of-m prune, then pack.  Returns (values uint16 [R, S], idx uint32 [R, W])."""
    positions = select_survivors(w_bits, n, m)
    return pack_values(w_bits, positions, m), pack_indices(positions, m)


# --------------------------------------------------------------------------
# Unpack / decompress
# --------------------------------------------------------------------------

def unpack_indices(idx: np.ndarray, S: int, m: int) -> np.ndarray:
    """Inverse of pack_indices: positions [R, S] read back from the bitstream."""
    idx = np.asarray(idx, dtype=np.uint32)
    R = idx.shape[0]
    b = index_bits(m)
    start = np.arange(S, dtype=np.int64) * b
    pos = np.zeros((R, S), dtype=np.int64)
    for j in range(b):
        bit = start + j
        word = idx[:, bit // 32].astype(np.int64)
        pos |= ((word >> (bit % 32)) & 1) << j
    return pos


def decompress(values: np.ndarray, idx: np.ndarray, K: int, n: int, m: int) -> np.ndarray:
    """Dense bit patterns [R, K]: each stored value back at g*m + position, zeros elsewhere."""
    values = np.asarray(values, dtype=np.uint16)
    R, S = values.shape
    if S != survivors_per_row(K, n, m):
        raise ValueError("values width does not match K*n/m")
    pos = unpack_indices(idx, S, m)
    group = np.arange(S, dtype=np.int64) // n
    cols = group[None, :] * m + pos
    dense = np.zeros((R, K), dtype=np.uint16)
    rows = np.broadcast_to(np.arange(R)[:, None], (R, S))
    dense[rows, cols] = values
    return dense


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------

def spmm_ref(values, idx, K: int, n: int, m: int, act_bits, dtype: str, perm=None) -> np.ndarray:
    """Y = W_nm X in float64, returned as [R, T].

    W_nm is the decompressed weight; X = act^T (R6).  With a permutation the
    input rows are read through the index map, X_perm[k, :] = X[perm[k], :]
    (R7), which is (W Pi) x for Pi[k, perm[k]] = 1.
    """
    wd = half_bits_to_f64(decompress(values, idx, K, n, m), dtype)
    x = half_bits_to_f64(np.asarray(act_bits, dtype=np.uint16), dtype).T  # [K, T]
    if perm is not None:
        x = x[np.asarray(perm, dtype=np.int64), :]
    return wd @ x


def spmm_rows_ref(values, idx, K: int, n: int, m: int, act_bits, dtype: str, rows, cols,
                  perm=None) -> np.ndarray:
    """Y[rows[i], cols[i]] one at a time, for sampled checks at full size."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    wd = half_bits_to_f64(decompress(values[np.unique(rows)], idx[np.unique(rows)], K, n, m), dtype)
    where = {r: i for i, r in enumerate(np.unique(rows))}
    out = np.empty(len(rows), dtype=np.float64)
    act = np.asarray(act_bits, dtype=np.uint16)
    p = None if perm is None else np.asarray(perm, dtype=np.int64)
    for i, (r, t) in enumerate(zip(rows, cols)):
        xt = half_bits_to_f64(act[t], dtype)
        if p is not None:
            xt = xt[p]
        out[i] = float(np.dot(wd[where[int(r)]], xt))
    return out


# --------------------------------------------------------------------------
# 8-bit integer weights and activations
# --------------------------------------------------------------------------
# The 2:4 pattern is also taken for INT8 weights (COE-592 lecture 04-2, "M:N
# sparsity on NVIDIA tensor cores", opening section).  The index stays 2 bits
# per stored value, so a group costs 2 x 8 value bits + 2 x 2 index bits = 20
# of the dense 32 (25% index overhead, a 37.5% saving; same page, section
# "Where this sits among the three case studies"), and the reduction length
# must be a multiple of 32 for INT8 (same section).  Readings:
#   R8  the magnitude of an int8 weight is |w| as an integer, so -128 ranks
#       above 127; equal magnitudes go to the lower position (as R2);
#   R9  the product accumulates in 32-bit integers; with |w|, |x| <= 128 and
#       K <= 2^16 survivors per row it is exact, so the reference is the exact
#       integer result.

I8 = "i8"


def magnitude_keys_i8(w: np.ndarray) -> np.ndarray:
    """|w| of int8 weights as int32 (0..128)."""
    return np.abs(np.asarray(w, dtype=np.int8).astype(np.int32))


def select_survivors_i8(w: np.ndarray, n: int, m: int) -> np.ndarray:
    """As select_survivors, ranking int8 weights by |w| (R8)."""
    w = np.asarray(w, dtype=np.int8)
    R, K = w.shape
    if K % m:
        raise ValueError("K must be a multiple of m")
    keys = magnitude_keys_i8(w).reshape(R, K // m, m)
    ranking = np.argsort(-keys, axis=-1, kind="stable")
    return np.sort(ranking[..., :n], axis=-1).astype(np.int64)


def prune_pack_i8(w: np.ndarray, n: int, m: int):
    """Magnitude top-n-of-m prune of int8 W, then pack.

    Returns (values int8 [R, S], idx uint32 [R, W]); the index stream is the
    same as for 16-bit weights (pack_indices).
    """
    w = np.asarray(w, dtype=np.int8)
    positions = select_survivors_i8(w, n, m)
    R, K = w.shape
    vals = np.take_along_axis(w.reshape(R, K // m, m), positions, axis=-1).reshape(R, -1).copy()
    return vals, pack_indices(positions, m)


def decompress_i8(values: np.ndarray, idx: np.ndarray, K: int, n: int, m: int) -> np.ndarray:
    """Dense int8 [R, K]: each stored value back at g*m + position, zeros elsewhere."""
    values = np.asarray(values, dtype=np.int8)
    R, S = values.shape
    if S != survivors_per_row(K, n, m):
        raise ValueError("values width does not match K*n/m")
    pos = unpack_indices(idx, S, m)
    cols = (np.arange(S, dtype=np.int64) // n)[None, :] * m + pos
    dense = np.zeros((R, K), dtype=np.int8)
    dense[np.broadcast_to(np.arange(R)[:, None], (R, S)), cols] = values
    return dense


def spmm_ref_i8(values, idx, K: int, n: int, m: int, act, perm=None) -> np.ndarray:
    """Y = W_nm X exactly, int64 [R, T], for int8 W_nm and act[T, K] (R6, R7, R9)."""
    wd = decompress_i8(values, idx, K, n, m).astype(np.int64)
    x = np.asarray(act, dtype=np.int8).astype(np.int64).T  # [K, T]
    if perm is not None:
        x = x[np.asarray(perm, dtype=np.int64), :]
    return wd @ x


# --------------------------------------------------------------------------
# 8-bit floating-point weights and activations (OCP E4M3)
# --------------------------------------------------------------------------
# The pages name 16-bit and INT8 2:4 types; an 8-bit float takes the same
# one-byte packed layout, group cost and K % 32 rule as INT8 (reading R10).
# Readings:
#   R10 the format is OCP FP8 E4M3 (sign, 4 exponent bits with bias 7, 3
#       mantissa bits; exponent 0 subnormal; S.1111.111 is NaN; no inf), the
#       one the 8-bit sparse MFMA of this hardware takes;
#   R11 magnitude is compared on bits & 0x7F (the sign bit dropped), which
#       orders finite values by |w| as for 16-bit floats; equal keys go to the
#       lower position;
#   R12 the reference product is exact (fp64 of the decoded values).

F8 = "f8e4m3"


def fp8_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of OCP E4M3 bit patterns (uint8), from the field definition."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((b & 0x7F) == 0x7F, np.nan, out)


def select_survivors_fp8(w_bits: np.ndarray, n: int, m: int) -> np.ndarray:
    """As select_survivors, with keys bits & 0x7F of the 8-bit patterns (R11)."""
    w = np.asarray(w_bits, dtype=np.uint8)
    R, K = w.shape
    if K % m:
        raise ValueError("K must be a multiple of m")
    keys = (w & np.uint8(0x7F)).astype(np.int32).reshape(R, K // m, m)
    ranking = np.argsort(-keys, axis=-1, kind="stable")
    return np.sort(ranking[..., :n], axis=-1).astype(np.int64)


def prune_pack_fp8(w_bits: np.ndarray, n: int, m: int):
    """Returns (values uint8 [R, S] bit patterns, idx uint32 [R, W])."""
    w = np.asarray(w_bits, dtype=np.uint8)
    positions = select_survivors_fp8(w, n, m)
    R, K = w.shape
    vals = np.take_along_axis(w.reshape(R, K // m, m), positions, axis=-1).reshape(R, -1).copy()
    return vals, pack_indices(positions, m)


def decompress_fp8(values: np.ndarray, idx: np.ndarray, K: int, n: int, m: int) -> np.ndarray:
    """Dense uint8 bit patterns [R, K] (zeros elsewhere)."""
    return decompress_i8(np.asarray(values, dtype=np.uint8).view(np.int8), idx, K, n, m).view(np.uint8)


def spmm_ref_fp8(values, idx, K: int, n: int, m: int, act_bits, perm=None) -> np.ndarray:
    """Y = W_nm X in float64, [R, T], for E4M3 W_nm and act[T, K] (R6, R7, R12)."""
    wd = fp8_to_f64(decompress_fp8(values, idx, K, n, m))
    x = fp8_to_f64(np.asarray(act_bits, dtype=np.uint8)).T  # [K, T]
    if perm is not None:
        x = x[np.asarray(perm, dtype=np.int64), :]
    return wd @ x


def relative_error(y: np.ndarray, yref: np.ndarray):
    """(max floored relative error, normwise relative error).

    Element error is |y - yref| / max(|yref|, rms(yref)); the floor keeps the
    ratio bounded where yref is near zero.
    """
    y = np.asarray(y, dtype=np.float64)
    yref = np.asarray(yref, dtype=np.float64)
    if yref.size == 0:
        return 0.0, 0.0
    rms = float(np.sqrt(np.mean(yref * yref)))
    floor = np.maximum(np.abs(yref), rms if rms > 0 else 1.0)
    max_rel = float(np.max(np.abs(y - yref) / floor))
    den = float(np.linalg.norm(yref))
    norm_rel = float(np.linalg.norm(y - yref) / den) if den > 0 else float(np.linalg.norm(y - yref))
    return max_rel, norm_rel
