"""Pins of the hybrid dense / 2:4 tile oracle (oracle/nm_hybrid.py), on the CPU.

Each check ties the oracle to something other than itself:
  * a layout worked out by hand for a 2 x 32 matrix (tables, the stored
    order of a dense block, survivors and index bytes, and back);
  * all tiles dense: the packed values hold the matrix's values block by
    block, decompress to the matrix itself, and the product is the exact
    integer matrix product;
  * all tiles 2:4: the packing and the product are the row-wise 2:4 ones of
    nm_oracle (pinned by its own tests);
  * a random mix, ragged tile-rows included: the weight matrix it stands for
    equals one built tile by tile with a brute-force mask (for each group of
    four, the pair of positions with the largest key sum, the lexicographically
    first pair on ties: the same as the two largest keys with ties to the lower
    position), and the product is exact on integers;
  * sizes and the zero fraction in closed form (zero fraction = half the share
    of 2:4 tile area, for weights without zeros).
"""
import itertools

import numpy as np
import pytest

import nm_inputs
from oracle import nm_hybrid as H
from oracle import nm_oracle as O


def int_bits(shape, lo, hi, seed, dt="f16", nonzero=False):
    rng = np.random.default_rng(seed)
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    if nonzero:
        v[v == 0] = 1.0
    return nm_inputs.to_half_bits(v, dt)


def test_layout_worked_example():
    # 2 x 32 weights, 16-wide tiles, one row per tile-row.  Row 0: a dense tile
    # (16 values) then a 2:4 tile (8 survivors, 2 index bytes); row 1: a 2:4
    # tile then a dense one.
    flags = np.array([[1, 0], [0, 1]])
    tm, rm, nv, ni = H.hybrid_layout(2, 32, 1, 16, flags)
    assert tm.tolist() == [[[0, -1], [16, 0]], [[24, 2], [32, -1]]]
    assert rm.tolist() == [[24, 2, 0, 0], [24, 2, 24, 2]]
    assert (nv, ni) == (48, 16)   # 4 index bytes, zero-padded to one 16-byte block
    w = np.arange(1, 65, dtype=np.float32).reshape(2, 32)
    w[0, 16:32] = [5, -7, 1, 2, 0, 3, -3, 1, 4, 4, -9, 2, -1, 0, 0, 6]   # 2:4 tile of row 0
    w[1, 0:16] = [1, 1, 1, 1, -4, 0, 2, 9, 7, -7, 0, 0, 0, 0, 0, -2]     # 2:4 tile of row 1
    bits = nm_inputs.to_half_bits(w, "f16")
    vals, idx = H.hybrid_pack(bits, 1, 16, flags)
    f = vals.view(np.float16).astype(np.float32)
    # dense block of 16: positions 0, 1 of each group of four, then 2, 3
    assert f[0:16].tolist() == [1, 2, 5, 6, 9, 10, 13, 14, 3, 4, 7, 8, 11, 12, 15, 16]
    # groups (5,-7,1,2) -> positions 0,1; (0,3,-3,1) -> 1,2 (tie kept whole);
    # (4,4,-9,2) -> 0,2 (tie to the lower position); (-1,0,0,6) -> 0,3
    assert f[16:24].tolist() == [5, -7, 3, -3, 4, -9, -1, 6]
    assert idx[0] == (0 | 1 << 2 | 1 << 4 | 2 << 6) == 0x94
    assert idx[1] == (0 | 2 << 2 | 0 << 4 | 3 << 6) == 0xC8
    # (1,1,1,1) -> 0,1; (-4,0,2,9) -> 0,3; (7,-7,0,0) -> 0,1; (0,0,0,-2) -> 0,3
    assert f[24:32].tolist() == [1, 1, -4, 9, 7, -7, 0, -2]
    assert idx[2] == idx[3] == (0 | 1 << 2 | 0 << 4 | 3 << 6) == 0xC4
    assert not idx[4:].any()
    assert f[32:48].tolist() == [49, 50, 53, 54, 57, 58, 61, 62, 51, 52, 55, 56, 59, 60, 63, 64]
    # and back: the weight matrix the packed form stands for
    dec = H.hybrid_decompress(vals, idx, 2, 32, 1, 16, flags).view(np.float16).astype(np.float32)
    expect = w.copy()
    expect[0, 16:32] = [5, -7, 0, 0, 0, 3, -3, 0, 4, 0, -9, 0, -1, 0, 0, 6]
    expect[1, 0:16] = [1, 1, 0, 0, -4, 0, 0, 9, 7, -7, 0, 0, 0, 0, 0, -2]
    assert np.array_equal(dec, expect)


@pytest.mark.parametrize("R,K,tr,tc", [(48, 128, 16, 64), (37, 192, 16, 64), (8, 64, 3, 16)])
def test_all_dense_is_the_matrix(R, K, tr, tc):
    flags = np.ones(H.tile_grid(R, K, tr, tc), dtype=np.uint8)
    w = int_bits((R, K), -8, 8, 1)
    act = int_bits((24, K), -8, 8, 2)
    vals, idx = H.hybrid_pack(w, tr, tc, flags)
    assert vals.size == R * K and idx.size == 0
    # every block of 16 holds the same values as the matrix's (storage order
    # aside), and the packed form stands for the matrix itself
    assert np.array_equal(np.sort(vals.reshape(-1, 16), axis=1), np.sort(w.reshape(-1, 16), axis=1))
    assert np.array_equal(H.hybrid_decompress(vals, idx, R, K, tr, tc, flags), w)
    y = H.hybrid_spmm_ref(vals, idx, R, K, tr, tc, flags, act, "f16")
    wi = w.view(np.float16).astype(np.int64)
    ai = act.view(np.float16).astype(np.int64)
    assert np.array_equal(y, (wi @ ai.T).astype(np.float64))


@pytest.mark.parametrize("R,K,tr,tc,dt", [(48, 128, 16, 64, "f16"), (37, 256, 16, 128, "bf16"),
                                          (5, 64, 2, 16, "f16")])
def test_all_sparse_is_row_wise_2of4(R, K, tr, tc, dt):
    flags = np.zeros(H.tile_grid(R, K, tr, tc), dtype=np.uint8)
    w = nm_inputs.normal_half((R, K), 1.0, dt, 80, 0, R + K)
    act = nm_inputs.normal_half((16, K), 1.0, dt, 80, 1, R + K)
    vals, idx = H.hybrid_pack(w, tr, tc, flags)
    ref_vals, ref_idx = O.prune_pack(w, 2, 4)
    assert np.array_equal(vals.reshape(R, K // 2), ref_vals)
    ref_bytes = ref_idx.astype("<u4").view(np.uint8).reshape(R, -1)[:, :K // 8]
    assert np.array_equal(idx[:R * K // 8].reshape(R, K // 8), ref_bytes)
    assert idx.size == -(-R * K // 8 // 16) * 16 and not idx[R * K // 8:].any()
    y = H.hybrid_spmm_ref(vals, idx, R, K, tr, tc, flags, act, dt)
    assert np.array_equal(y, O.spmm_ref(ref_vals, ref_idx, K, 2, 4, act, dt))


def brute_force_mask(w_bits):
    """For every group of four: the pair with the largest key sum, first pair on ties."""
    keys = (w_bits & 0x7FFF).astype(np.int64)
    R, K = keys.shape
    mask = np.zeros((R, K), dtype=bool)
    pairs = list(itertools.combinations(range(4), 2))  # lexicographic order
    for r in range(R):
        for g in range(K // 4):
            kk = keys[r, 4 * g:4 * g + 4]
            best = max(pairs, key=lambda p: (kk[p[0]] + kk[p[1]], [-x for x in p]))
            mask[r, 4 * g + best[0]] = mask[r, 4 * g + best[1]] = True
    return mask


@pytest.mark.parametrize("R,K,tr,tc,frac", [(40, 128, 16, 32, 0.5), (33, 192, 16, 64, 0.3),
                                            (64, 256, 32, 64, 0.8)])
def test_random_mix_against_tile_masks(R, K, tr, tc, frac):
    grid = H.tile_grid(R, K, tr, tc)
    flags = nm_inputs.tile_flags(grid, frac, 81, R + K)
    w = int_bits((R, K), -3, 3, R * K)          # many ties and zeros
    act = int_bits((20, K), -5, 5, R + K)
    vals, idx = H.hybrid_pack(w, tr, tc, flags)
    # the weight matrix built tile by tile: dense tiles as they are, 2:4 tiles
    # through the brute-force mask
    expect = w.copy()
    mask = brute_force_mask(w)
    for b in range(grid[0]):
        for j in range(grid[1]):
            if not flags[b, j]:
                rs = slice(b * tr, min(R, (b + 1) * tr))
                cs = slice(j * tc, (j + 1) * tc)
                expect[rs, cs] = np.where(mask[rs, cs], w[rs, cs], 0)
    got = H.hybrid_decompress(vals, idx, R, K, tr, tc, flags)
    # dropped weights are +0; a kept -0 stays -0 (compare values, then bits of
    # the kept ones)
    assert np.array_equal(got.view(np.float16).astype(np.float32), expect.view(np.float16).astype(np.float32))
    y = H.hybrid_spmm_ref(vals, idx, R, K, tr, tc, flags, act, "f16")
    ei = expect.view(np.float16).astype(np.int64)
    ai = act.view(np.float16).astype(np.int64)
    assert np.array_equal(y, (ei @ ai.T).astype(np.float64))


@pytest.mark.parametrize("R,K,tr,tc,frac", [(100, 512, 16, 64, 0.25), (64, 1024, 64, 128, 0.6)])
def test_sizes_and_zero_fraction(R, K, tr, tc, frac):
    grid = H.tile_grid(R, K, tr, tc)
    flags = nm_inputs.tile_flags(grid, frac, 82, R)
    _, _, nv, ni = H.hybrid_layout(R, K, tr, tc, flags)
    rows = np.array([H.rows_of(b, R, tr) for b in range(grid[0])])
    nd = flags.sum(axis=1)
    ns = grid[1] - nd
    assert nv == int(np.sum(rows * (nd * tc + ns * tc // 2)))
    assert ni == -(-int(np.sum(rows * ns * tc // 8)) // 16) * 16
    w = int_bits((R, K), -4, 4, 9, nonzero=True)
    vals, idx = H.hybrid_pack(w, tr, tc, flags)
    dec = H.hybrid_decompress(vals, idx, R, K, tr, tc, flags)
    sparse_area = float(np.sum(rows[:, None] * (1 - flags) * tc)) / (R * K)
    assert np.mean(dec == 0) == pytest.approx(0.5 * sparse_area, abs=0)
