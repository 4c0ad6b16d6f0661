"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each check_* function raises AssertionError when the oracle is wrong.  The
tests below run them on the oracle as written; test_oracle_mutations.py plants
plausible mistakes in the oracle and shows that some check fails for each.
"""
import itertools
import os

import numpy as np
import pytest

import nm_inputs
from oracle import nm_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.strip()
    return out


def f16_bits(vals):
    return np.asarray(vals, dtype=np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# Independent brute force: the kept set from the definition, by enumeration
# ---------------------------------------------------------------------------

def brute_force_kept(w_f64_groups, n):
    """For each group (rows of a [G, m] float64 array), the unique n-subset T with
    |w_i| > |w_j|, or |w_i| == |w_j| and i < j, for every i in T and j not in T.
    Returns a bool mask [G, m] and asserts exactly one subset qualifies."""
    G, m = w_f64_groups.shape
    a = np.abs(w_f64_groups)
    mask = np.zeros((G, m), dtype=bool)
    found = np.zeros(G, dtype=np.int64)
    for subset in itertools.combinations(range(m), n):
        inside = list(subset)
        outside = [j for j in range(m) if j not in subset]
        ok = np.ones(G, dtype=bool)
        for i in inside:
            for j in outside:
                ok &= (a[:, i] > a[:, j]) | ((a[:, i] == a[:, j]) & (i < j))
        found += ok
        sel = np.zeros(m, dtype=bool)
        sel[inside] = True
        mask[ok] = sel
    assert np.all(found == 1), "the definition must single out exactly one subset"
    return mask


def oracle_mask(oracle, w_bits, n, m):
    pos = oracle.select_survivors(w_bits, n, m)
    R, K = w_bits.shape
    mask = np.zeros((R, K // m, m), dtype=bool)
    np.put_along_axis(mask, pos, True, axis=-1)
    return mask.reshape(R, K)


# ---------------------------------------------------------------------------
# Checks
# ---------------------------------------------------------------------------

def check_worked_row(oracle):
    g = read_golden("worked_row_2of4.txt")
    pattern = g["pattern"].split()
    want = [int(t) for t in g["positions"].replace("|", " ").split()]
    for values in ([0.5, -1.25, 3.0, -2.0], [1, 1, 1, 1], [-7.0, 0.75, -0.75, 6.5]):
        it = iter(values)
        row = [next(it) if c == "v" else 0.0 for c in pattern]
        # second row: same survivors, pruned slots hold small nonzeros
        it = iter(values)
        row2 = [next(it) if c == "v" else 1e-3 for c in pattern]
        w = f16_bits([row, row2])
        pos = oracle.select_survivors(w, 2, 4)
        assert pos[0].tolist() == [want[0:2], want[2:4]]
        assert pos[1].tolist() == [want[0:2], want[2:4]]
        vals, idx = oracle.prune_pack(w, 2, 4)
        assert vals[0].tolist() == f16_bits(values).tolist()
        assert idx.shape == (2, 1)
        assert int(idx[0, 0]) & 0xFF == int(g["idx_byte"], 16)
        assert int(idx[0, 0]) >> 8 == 0  # padding bits are zero


def check_group_cost(oracle):
    g = read_golden("group_cost_fp16.txt")
    dense_bits, packed_bits = int(g["dense_bits_per_group"]), int(g["packed_bits_per_group"])
    for R, K in ((256, 256), (7, 64), (3, 4096)):
        w = nm_inputs.normal_half((R, K), 1.0, "f16", 99, 0)
        vals, idx = oracle.prune_pack(w, 2, 4)
        total_bits = vals.nbytes * 8 + idx.nbytes * 8
        assert total_bits == R * (K // 4) * packed_bits
        assert R * K * 16 == R * (K // 4) * dense_bits
    # rows whose index bits do not fill a word are padded to one: K = 16 -> 16 bits -> 32
    vals, idx = oracle.prune_pack(nm_inputs.normal_half((7, 16), 1.0, "f16", 99, 0), 2, 4)
    assert vals.nbytes == 7 * 8 * 2 and idx.nbytes == 7 * 4
    assert round(100 * (1 - packed_bits / dense_bits)) == int(g["saving_percent_approx"])
    assert 100 * 2 / 16 == float(g["index_overhead_fp16_percent"])
    assert 100 * 2 / 8 == float(g["index_overhead_int8_percent"])
    # INT8 group: 2x8 value bits + 2x2 index bits out of 32
    assert 100 * (1 - (2 * 8 + 2 * 2) / 32) == float(g["int8_saving_percent"])
    # the small workload: 256 x 256 fp16 -> 65,536 B values + 8,192 B indices
    w = nm_inputs.WORKLOADS[1].weights()
    vals, idx = oracle.prune_pack(w, 2, 4)
    assert vals.nbytes == 65536 and idx.nbytes == 8192


def check_exactly_n_ascending(oracle):
    for (n, m) in ((2, 4), (1, 4), (1, 8), (3, 4), (2, 8), (1, 2)):
        w = nm_inputs.normal_half((5, 8 * m), 1.0, "bf16", 98, n * 10 + m)
        pos = oracle.select_survivors(w, n, m)
        assert pos.shape == (5, 8, n)
        assert pos.min() >= 0 and pos.max() < m
        assert np.all(np.diff(pos, axis=-1) > 0)


def check_brute_force(oracle):
    cases = []
    # random values with many ties: small integers times random signs
    rng = np.random.default_rng(12345)
    for dtype in ("f16", "bf16"):
        for (n, m) in ((2, 4), (1, 4), (1, 8), (3, 4), (2, 8), (3, 8)):
            x = rng.integers(0, 4, size=(6, 4 * m)).astype(np.float32)
            x *= rng.choice([-1.0, 1.0], size=x.shape).astype(np.float32)
            cases.append((nm_inputs.to_half_bits(x, dtype), dtype, n, m))
            y = rng.standard_normal((6, 4 * m)).astype(np.float32)
            cases.append((nm_inputs.to_half_bits(y, dtype), dtype, n, m))
    for w, dtype, n, m in cases:
        wf = O.half_bits_to_f64(w, dtype)  # plain decode, no keys
        want = brute_force_kept(wf.reshape(-1, m), n).reshape(w.shape)
        got = oracle_mask(oracle, w, n, m)
        assert np.array_equal(got, want)


def check_exhaustive_ties(oracle):
    mags = np.array([0.0, 0.5, 1.0, 2.0])
    rng = np.random.default_rng(7)
    for m, ns in ((4, (1, 2, 3)), (8, (1,))):
        keys = np.array(list(itertools.product(range(4), repeat=m)))  # every tie pattern
        signs = rng.choice([-1.0, 1.0], size=keys.shape)
        x = (mags[keys] * signs).astype(np.float32)
        for dtype in ("f16", "bf16"):
            w = nm_inputs.to_half_bits(x.reshape(-1, m), dtype).reshape(-1, m)
            wf = O.half_bits_to_f64(w, dtype)
            for n in ns:
                want = brute_force_kept(wf, n)
                got = oracle_mask(oracle, w, n, m)
                assert np.array_equal(got, want), (m, n, dtype)


def check_round_trip(oracle):
    for (n, m) in ((2, 4), (1, 4), (1, 8)):
        for dtype in ("f16", "bf16"):
            w = nm_inputs.normal_half((9, 16 * m), 0.02, dtype, 97, m + n)
            vals, idx = oracle.prune_pack(w, n, m)
            back = oracle.decompress(vals, idx, w.shape[1], n, m)
            mask = brute_force_kept(O.half_bits_to_f64(w, dtype).reshape(-1, m), n).reshape(w.shape)
            assert np.array_equal(back, np.where(mask, w, np.uint16(0)))
            # an already-N:M matrix is a fixed point of prune -> decompress
            vals2, idx2 = oracle.prune_pack(back, n, m)
            assert np.array_equal(oracle.decompress(vals2, idx2, w.shape[1], n, m), back)
            # the kept set has the largest sum of |w| over all n-subsets
            wf = np.abs(O.half_bits_to_f64(w, dtype)).reshape(-1, m)
            kept_sum = (wf * mask.reshape(-1, m)).sum(axis=1)
            best = np.max([wf[:, list(s)].sum(axis=1) for s in itertools.combinations(range(m), n)],
                          axis=0)
            assert np.array_equal(kept_sum, best)


def check_bitstream(oracle):
    # Big-integer reading of the LSB-first stream, independent of numpy bit tricks.
    rng = np.random.default_rng(5)
    for (n, m) in ((2, 4), (1, 4), (1, 8), (3, 8)):
        b = (m - 1).bit_length()
        for K in (16 * m, 8 * m, 40 * m):
            G = K // m
            pos = np.sort(np.array([[rng.choice(m, size=n, replace=False) for _ in range(G)]
                                    for _ in range(3)]), axis=-1)
            words = oracle.pack_indices(pos, m)
            S = G * n
            assert words.shape == (3, (S * b + 31) // 32)
            for r in range(3):
                big = 0
                for s, p in enumerate(pos[r].reshape(-1)):
                    big |= int(p) << (s * b)
                got = 0
                for w_i, word in enumerate(words[r]):
                    got |= int(word) << (32 * w_i)
                assert got == big
            assert np.array_equal(oracle.unpack_indices(words, S, m), pos.reshape(3, -1))


def check_k8_walkthrough(oracle):
    g = read_golden("k8_walkthrough.txt")
    w_row = [float(v) for v in g["w_row"].split()]
    b_col = [float(v) for v in g["b_col"].split()]
    w = f16_bits([w_row])
    vals, idx = oracle.prune_pack(w, 2, 4)
    assert vals.shape == (1, 4)
    assert O.half_bits_to_f64(vals, "f16")[0].tolist() == [float(v) for v in g["stored_values"].split()]
    assert oracle.unpack_indices(idx, 4, 4)[0].tolist() == [int(v) for v in g["positions"].split()]
    act = f16_bits([b_col])  # T = 1: the dense column as one activation row
    y = oracle.spmm_ref(vals, idx, 8, 2, 4, act, "f16")
    assert y.shape == (1, 1) and y[0, 0] == float(g["y"])
    assert int(g["multiplies"]) == vals.shape[1]


def check_identity_gemm(oracle):
    # X = I: Y is the pruned weight matrix itself, exactly.
    for (n, m), dtype in (((2, 4), "bf16"), ((1, 8), "f16"), ((1, 4), "bf16")):
        K = 8 * m
        w = nm_inputs.normal_half((6, K), 1.0, dtype, 96, m)
        vals, idx = oracle.prune_pack(w, n, m)
        eye = nm_inputs.to_half_bits(np.eye(K, dtype=np.float32), dtype)
        y = oracle.spmm_ref(vals, idx, K, n, m, eye, dtype)
        mask = brute_force_kept(O.half_bits_to_f64(w, dtype).reshape(-1, m), n).reshape(w.shape)
        assert np.array_equal(y, np.where(mask, O.half_bits_to_f64(w, dtype), 0.0))


def check_integer_gemm_brute_force(oracle):
    # Pure-Python triple loop over the original W with the brute-force mask.
    for (n, m), dtype, (R, K, T) in (((2, 4), "f16", (5, 16, 5)), ((1, 8), "bf16", (3, 32, 4)),
                                     ((1, 4), "f16", (4, 16, 16))):
        w = nm_inputs.integer_half((R, K), -3, 3, dtype, 95, 0, m)
        act = nm_inputs.integer_half((T, K), -2, 2, dtype, 95, 1, m)
        wf = O.half_bits_to_f64(w, dtype)
        xf = O.half_bits_to_f64(act, dtype)
        mask = brute_force_kept(wf.reshape(-1, m), n).reshape(R, K)
        want = [[sum(wf[r][k] * xf[t][k] for k in range(K) if mask[r][k]) for t in range(T)]
                for r in range(R)]
        vals, idx = oracle.prune_pack(w, n, m)
        got = oracle.spmm_ref(vals, idx, K, n, m, act, dtype)
        assert got.tolist() == want


def check_dense_case(oracle):
    # n = m keeps everything: the product reduces to a plain matmul.
    for m, dtype in ((4, "f16"), (8, "bf16")):
        w = nm_inputs.normal_half((7, 4 * m), 1.0, dtype, 94, m)
        act = nm_inputs.normal_half((3, 4 * m), 1.0, dtype, 94, 1, m)
        vals, idx = oracle.prune_pack(w, m, m)
        y = oracle.spmm_ref(vals, idx, 4 * m, m, m, act, dtype)
        ref = np.matmul(O.half_bits_to_f64(w, dtype), O.half_bits_to_f64(act, dtype).T)
        assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)


def check_permutation(oracle):
    K, R, T = 32, 6, 5
    w = nm_inputs.normal_half((R, K), 1.0, "f16", 93, 0)
    act = nm_inputs.normal_half((T, K), 1.0, "f16", 93, 1)
    perm = nm_inputs.random_permutation(K, 93)
    vals, idx = oracle.prune_pack(w, 2, 4)
    wd = O.half_bits_to_f64(oracle.decompress(vals, idx, K, 2, 4), "f16")
    x = O.half_bits_to_f64(act, "f16").T
    # Pi as an explicit matrix, Pi[k, perm[k]] = 1, then y = (W Pi) x
    pi = np.zeros((K, K))
    pi[np.arange(K), perm] = 1.0
    dense_route = (wd @ pi) @ x
    y = oracle.spmm_ref(vals, idx, K, 2, 4, act, "f16", perm=perm)
    assert np.allclose(y, dense_route, rtol=1e-12, atol=1e-12)
    # identity permutation is the plain product
    y_id = oracle.spmm_ref(vals, idx, K, 2, 4, act, "f16", perm=np.arange(K, dtype=np.int32))
    assert np.array_equal(y_id, oracle.spmm_ref(vals, idx, K, 2, 4, act, "f16"))
    # sampled one-at-a-time route agrees
    rows, cols = np.array([0, 5, 3, 3]), np.array([4, 0, 2, 1])
    pts = oracle.spmm_rows_ref(vals, idx, K, 2, 4, act, "f16", rows, cols, perm=perm)
    assert np.allclose(pts, y[rows, cols], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# int8 weights (COE-592 lecture 04-2, "M:N sparsity on NVIDIA tensor cores":
# INT8 is a 2:4 weight type, opening section; 2 index bits per stored value,
# 25% overhead and a 37.5% saving, section "Where this sits among the three
# case studies")
# ---------------------------------------------------------------------------

def check_i8_worked_row(oracle):
    # the worked row's pattern "value, zero, zero, value / zero, value, value, zero"
    w = np.array([[5, 0, 0, -7, 0, 3, -2, 0]], dtype=np.int8)
    pos = oracle.select_survivors_i8(w, 2, 4)
    assert pos.tolist() == [[[0, 3], [1, 2]]]
    vals, idx = oracle.prune_pack_i8(w, 2, 4)
    assert vals.tolist() == [[5, -7, 3, -2]]
    assert int(idx[0, 0]) & 0xFF == 0x9C


def check_i8_group_cost(oracle):
    # 2 x 8 value bits + 2 x 2 index bits = 20 of 32 bits per group of four
    R, K = 64, 4096
    w = np.random.default_rng(3).integers(-128, 128, (R, K)).astype(np.int8)
    vals, idx = oracle.prune_pack_i8(w, 2, 4)
    assert vals.nbytes + idx.nbytes == R * (K // 4) * 20 // 8
    assert 1 - (vals.nbytes + idx.nbytes) / w.nbytes == 0.375
    assert idx.nbytes / vals.nbytes == 0.25


def check_i8_brute_force(oracle):
    rng = np.random.default_rng(11)
    # many ties, both extremes, zeros
    pool = np.array([-128, -127, -2, -1, 0, 1, 2, 127], dtype=np.int8)
    for n, m in ((2, 4), (1, 4), (1, 8)):
        w = rng.choice(pool, size=(40, 8 * m))
        mask = oracle.select_survivors_i8(w, n, m)
        got = np.zeros((40, 8, m), dtype=bool)
        np.put_along_axis(got, mask, True, axis=-1)
        want = brute_force_kept(w.astype(np.float64).reshape(-1, m), n).reshape(40, 8, m)
        assert np.array_equal(got, want), (n, m)
    # -128 has the largest magnitude
    assert oracle.select_survivors_i8(np.array([[127, -128, 0, 0]], np.int8), 1, 4).tolist() == [[[1]]]


def check_i8_round_trip_and_gemm(oracle):
    rng = np.random.default_rng(12)
    R, K, T = 6, 64, 5
    w = rng.integers(-128, 128, (R, K)).astype(np.int8)
    act = rng.integers(-128, 128, (T, K)).astype(np.int8)
    vals, idx = oracle.prune_pack_i8(w, 2, 4)
    dense = oracle.decompress_i8(vals, idx, K, 2, 4)
    mask = brute_force_kept(w.astype(np.float64).reshape(-1, 4), 2).reshape(R, K)
    assert np.array_equal(dense, np.where(mask, w, 0).astype(np.int8))
    y = oracle.spmm_ref_i8(vals, idx, K, 2, 4, act)
    # Python integers, one product at a time
    for r in range(R):
        for t in range(T):
            ref = sum(int(w[r, k]) * int(act[t, k]) for k in range(K) if mask[r, k])
            assert int(y[r, t]) == ref
    # the extreme product: every weight and activation -128, every group full
    wx = np.full((1, 128), -128, np.int8)
    v2, i2 = oracle.prune_pack_i8(wx, 2, 4)
    assert int(oracle.spmm_ref_i8(v2, i2, 128, 2, 4, np.full((1, 128), -128, np.int8))[0, 0]) == 64 * 128 * 128


def check_i8_permutation(oracle):
    rng = np.random.default_rng(13)
    R, K, T = 5, 32, 4
    w = rng.integers(-128, 128, (R, K)).astype(np.int8)
    act = rng.integers(-128, 128, (T, K)).astype(np.int8)
    perm = rng.permutation(K)
    vals, idx = oracle.prune_pack_i8(w, 2, 4)
    wd = oracle.decompress_i8(vals, idx, K, 2, 4).astype(np.int64)
    Pi = np.zeros((K, K), np.int64)
    Pi[np.arange(K), perm] = 1
    y = oracle.spmm_ref_i8(vals, idx, K, 2, 4, act, perm=perm)
    assert np.array_equal(y, (wd @ Pi) @ act.astype(np.int64).T)


# ---------------------------------------------------------------------------
# OCP FP8 E4M3 weights (same packed layout and group cost as INT8)
# ---------------------------------------------------------------------------

def check_fp8_decode(oracle):
    import torch
    b = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_to_f64(b)
    lib = torch.from_numpy(b).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)])
    # field values: 1.0, the largest finite 448, the smallest subnormal 2^-9,
    # the smallest normal 2^-6, and the sign
    assert oracle.fp8_to_f64(np.array([0x38, 0x7E, 0x01, 0x08, 0xB8], np.uint8)).tolist() == \
        [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -1.0]


def _fp8_bits(vals):
    import torch
    return torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def check_fp8_worked_row_and_brute_force(oracle):
    w = _fp8_bits([[5, 0, 0, -7, 0, 3, -2, 0]])
    assert oracle.select_survivors_fp8(w, 2, 4).tolist() == [[[0, 3], [1, 2]]]
    vals, idx = oracle.prune_pack_fp8(w, 2, 4)
    assert oracle.fp8_to_f64(vals).tolist() == [[5.0, -7.0, 3.0, -2.0]]
    assert int(idx[0, 0]) & 0xFF == 0x9C
    rng = np.random.default_rng(21)
    pool = _fp8_bits([-448, -2, -1, -0.0, 0.0, 1, 2, 448, 2.0 ** -9, -(2.0 ** -9)])
    w = rng.choice(pool, size=(30, 32))
    got = np.zeros((30, 8, 4), dtype=bool)
    np.put_along_axis(got, oracle.select_survivors_fp8(w, 2, 4), True, axis=-1)
    want = brute_force_kept(oracle.fp8_to_f64(w).reshape(-1, 4), 2).reshape(30, 8, 4)
    assert np.array_equal(got, want)


def check_fp8_integer_gemm(oracle):
    # small integers are exact in E4M3, so is their product
    rng = np.random.default_rng(22)
    R, K, T = 5, 64, 4
    wi = rng.integers(-8, 9, (R, K)); xi = rng.integers(-8, 9, (T, K))
    w, x = _fp8_bits(wi.astype(float)), _fp8_bits(xi.astype(float))
    vals, idx = oracle.prune_pack_fp8(w, 2, 4)
    mask = brute_force_kept(wi.astype(np.float64).reshape(-1, 4), 2).reshape(R, K)
    y = oracle.spmm_ref_fp8(vals, idx, K, 2, 4, x)
    for r in range(R):
        for t in range(T):
            assert y[r, t] == sum(int(wi[r, k]) * int(xi[t, k]) for k in range(K) if mask[r, k])
    perm = rng.permutation(K)
    yp = oracle.spmm_ref_fp8(vals, idx, K, 2, 4, x, perm=perm)
    assert np.array_equal(yp, oracle.spmm_ref_fp8(vals, idx, K, 2, 4, x[:, perm]))


ALL_CHECKS = [check_worked_row, check_group_cost, check_exactly_n_ascending, check_brute_force,
              check_exhaustive_ties, check_round_trip, check_bitstream, check_k8_walkthrough,
              check_identity_gemm, check_integer_gemm_brute_force, check_dense_case,
              check_permutation, check_i8_worked_row, check_i8_group_cost, check_i8_brute_force,
              check_i8_round_trip_and_gemm, check_i8_permutation, check_fp8_decode,
              check_fp8_worked_row_and_brute_force, check_fp8_integer_gemm]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(O)


def test_relative_error_definition():
    yref = np.array([[1.0, -2.0], [0.0, 4.0]])
    rms = np.sqrt(np.mean(yref ** 2))
    y = yref + np.array([[0.01, 0.0], [0.1, 0.0]])
    mx, nr = O.relative_error(y, yref)
    assert mx == pytest.approx(max(0.01 / max(1.0, rms), 0.1 / rms))
    assert nr == pytest.approx(np.linalg.norm(y - yref) / np.linalg.norm(yref))


def test_bf16_rounding_of_generator():
    # generator's bf16 rounding is round-to-nearest-even on exact halfway cases
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1.5], dtype=np.float32)
    bits = nm_inputs.f32_to_bf16_bits(x)
    back = O.half_bits_to_f64(bits, "bf16")
    assert back.tolist() == [1.0, 1.0 + 2 ** -6, -1.0, 1.5]
