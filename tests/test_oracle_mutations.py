"""Planted mistakes in the CPU oracle must each fail at least one pin.

Every mutation is applied to the oracle module on the CPU (monkeypatch undoes
it after the test); nothing here touches the GPU path.
"""
import numpy as np
import pytest

from oracle import nm_oracle as O
import test_oracle_pins as pins


def _fails_some_pin(oracle):
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(oracle)
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    return failed


_orig_select = O.select_survivors
_orig_pack_indices = O.pack_indices
_orig_decompress = O.decompress
_orig_spmm = O.spmm_ref


def tie_to_higher_position(w_bits, n, m):
    R, K = w_bits.shape
    keys = O.magnitude_keys(w_bits).reshape(R, K // m, m)
    ranking = np.argsort(-keys[..., ::-1], axis=-1, kind="stable")
    ranking = (m - 1) - ranking
    return np.sort(ranking[..., :n], axis=-1).astype(np.int64)


def keep_smallest(w_bits, n, m):
    R, K = w_bits.shape
    keys = O.magnitude_keys(w_bits).reshape(R, K // m, m)
    ranking = np.argsort(keys, axis=-1, kind="stable")
    return np.sort(ranking[..., :n], axis=-1).astype(np.int64)


def signed_keys(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.int16).astype(np.int32)


def unsorted_positions(w_bits, n, m):
    R, K = w_bits.shape
    keys = O.magnitude_keys(w_bits).reshape(R, K // m, m)
    ranking = np.argsort(-keys, axis=-1, kind="stable")
    return ranking[..., :n].astype(np.int64)


def msb_first_indices(positions, m):
    R = positions.shape[0]
    pos = positions.reshape(R, -1).astype(np.int64)
    S = pos.shape[1]
    b = O.index_bits(m)
    nwords = (S * b + 31) // 32
    stream = np.zeros((R, nwords * 32), dtype=np.uint64)
    for j in range(b):
        stream[:, j:S * b:b] = (pos >> (b - 1 - j)) & 1
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    return (stream.reshape(R, nwords, 32) * weights).sum(axis=-1).astype(np.uint32)


def drop_last_group(values, idx, K, n, m):
    d = _orig_decompress(values, idx, K, n, m)
    d[:, K - m:] = 0
    return d


def transposed_activation(values, idx, K, n, m, act_bits, dtype, perm=None):
    wd = O.half_bits_to_f64(_orig_decompress(values, idx, K, n, m), dtype)
    x = O.half_bits_to_f64(np.asarray(act_bits, dtype=np.uint16), dtype)  # forgot the transpose
    if x.shape[0] != K:
        x = x.T
    if perm is not None:
        x = x[np.asarray(perm, dtype=np.int64), :]
    return wd @ x


def inverse_permutation(values, idx, K, n, m, act_bits, dtype, perm=None):
    if perm is not None:
        perm = np.argsort(np.asarray(perm))
    return _orig_spmm(values, idx, K, n, m, act_bits, dtype, perm=perm)


_orig_decompress_i8 = O.decompress_i8
_orig_spmm_i8 = O.spmm_ref_i8


def i8_keys_wrap_at_128(w):
    # |w| computed in int8 arithmetic: abs(-128) wraps back to -128
    return np.abs(np.asarray(w, dtype=np.int8)).astype(np.int32)


def i8_signed_keys(w):
    return np.asarray(w, dtype=np.int8).astype(np.int32)


def i8_drop_last_group(values, idx, K, n, m):
    d = _orig_decompress_i8(values, idx, K, n, m)
    d[:, K - m:] = 0
    return d


def i8_inverse_permutation(values, idx, K, n, m, act, perm=None):
    if perm is not None:
        perm = np.argsort(np.asarray(perm))
    return _orig_spmm_i8(values, idx, K, n, m, act, perm=perm)


def i8_product_wraps_int32(values, idx, K, n, m, act, perm=None):
    # accumulating in int16 by mistake
    return _orig_spmm_i8(values, idx, K, n, m, act, perm=perm).astype(np.int16).astype(np.int64)


_orig_fp8_decode = O.fp8_to_f64


def fp8_bias_8(bits):
    # exponent bias 8 instead of 7
    return _orig_fp8_decode(bits) / 2.0


def fp8_signed_keys(w_bits, n, m):
    w = np.asarray(w_bits, dtype=np.uint8)
    R, K = w.shape
    keys = w.view(np.int8).astype(np.int32).reshape(R, K // m, m)
    ranking = np.argsort(-keys, axis=-1, kind="stable")
    return np.sort(ranking[..., :n], axis=-1).astype(np.int64)


MUTATIONS = {
    "fp8_bias_8": ("fp8_to_f64", fp8_bias_8),
    "fp8_signed_keys": ("select_survivors_fp8", fp8_signed_keys),
    "i8_keys_wrap_at_128": ("magnitude_keys_i8", i8_keys_wrap_at_128),
    "i8_signed_keys": ("magnitude_keys_i8", i8_signed_keys),
    "i8_drop_last_group": ("decompress_i8", i8_drop_last_group),
    "i8_inverse_permutation": ("spmm_ref_i8", i8_inverse_permutation),
    "i8_product_wraps": ("spmm_ref_i8", i8_product_wraps_int32),
    "tie_to_higher_position": ("select_survivors", tie_to_higher_position),
    "keep_smallest": ("select_survivors", keep_smallest),
    "unsorted_positions": ("select_survivors", unsorted_positions),
    "signed_keys": ("magnitude_keys", signed_keys),
    "msb_first_indices": ("pack_indices", msb_first_indices),
    "drop_last_group": ("decompress", drop_last_group),
    "transposed_activation": ("spmm_ref", transposed_activation),
    "inverse_permutation": ("spmm_ref", inverse_permutation),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = _fails_some_pin(O)
    assert failed, f"mutation {name} passed every pin"
