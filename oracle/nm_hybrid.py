"""CPU oracle for hybrid dense / 2:4 weight tiles.

TEST INFRASTRUCTURE ONLY.  Like nm_oracle, this module exists to check the GPU
library; only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it, and it shares no code with the HIP path.

Source: thelatestinai.com "Structured Sparsity" topic cards, the PATCH
abstract: a weight matrix is cut into tiles and every tile is either kept
dense or made 2:4 sparse (the choice comes from a learned mask), so the
fraction of zeros can sit anywhere between 0 and 50%.  The pruning inside a
2:4 tile is the one of nm_oracle (largest magnitudes per group of four, same
readings R1-R5); a dense tile keeps its weights unchanged.

Readings taken where the page is silent (H1-H5):
  H1  tiles are tile_rows x tile_cols blocks on a regular grid: tile-row b
      holds rows [b*tile_rows, min(R, (b+1)*tile_rows)) (the last one may be
      shorter), tile-column j holds columns [j*tile_cols, (j+1)*tile_cols);
      K is a multiple of tile_cols and tile_cols of 16;
  H2  flags[b, j] = 1 keeps tile (b, j) dense, 0 makes it 2:4;
  H3  a row stores its tiles in column order: a dense tile contributes its
      tile_cols values, a 2:4 tile its tile_cols/2 survivors (pushed left,
      positions ascending), and the row's index bits are the 2:4 tiles' bit
      streams (2 bits per survivor, LSB first) concatenated in the same order,
      tile_cols/8 bytes per 2:4 tile (whole bytes).  A dense tile's values
      keep their bits; within each block of 16 along K they are stored as the
      values at positions 0 and 1 of the block's four groups of four, then
      those at positions 2 and 3 (columns 0 1 4 5 8 9 12 13, then 2 3 6 7 10
      11 14 15): the block as two 2:4 halves with fixed positions, the form a
      2:4 instruction takes;
  H4  the rows of a tile-row share one length (their tiles have the same
      flags), Lv[b] values and Li[b] index bytes; rows are stored one after
      another with those strides, and the tile-rows one after another;
  H5  tile_meta[b, j] = (offset of the tile's first value in its tile-row's
      first row, offset of its first index byte there or -1 for a dense tile),
      row_meta[b] = (Lv[b], Li[b], offset of the tile-row's first value, offset
      of its first index byte); the index array is zero-padded to a whole
      number of 16-byte blocks (a block read never leaves it).

The mask learning itself is training and is not reproduced: flags are inputs.
"""
from __future__ import annotations

import numpy as np

from . import nm_oracle as O


def tile_grid(R: int, K: int, tile_rows: int, tile_cols: int):
    """(number of tile-rows, number of tile-columns) under H1."""
    if tile_rows <= 0 or tile_cols <= 0 or tile_cols % 16 or K % tile_cols:
        raise ValueError("tile_cols must divide K and be a multiple of 16; tile_rows > 0")
    return -(-R // tile_rows), K // tile_cols


def rows_of(b: int, R: int, tile_rows: int) -> int:
    """Rows in tile-row b (H1)."""
    return min(R, (b + 1) * tile_rows) - b * tile_rows


# H3: storage order of a dense block of 16 columns (entry p is the column
# stored at position p): positions 0 and 1 of the four groups, then 2 and 3
DENSE_BLOCK_ORDER = np.array([0, 1, 4, 5, 8, 9, 12, 13, 2, 3, 6, 7, 10, 11, 14, 15])


def dense_store(cols: np.ndarray) -> np.ndarray:
    """H3: a dense tile row's values in storage order (blocks of 16 reordered)."""
    blocks = np.asarray(cols).reshape(-1, 16)
    return blocks[:, DENSE_BLOCK_ORDER].reshape(-1)


def dense_load(stored: np.ndarray) -> np.ndarray:
    """Inverse of dense_store: the tile row's values in column order."""
    blocks = np.asarray(stored).reshape(-1, 16)
    out = np.empty_like(blocks)
    out[:, DENSE_BLOCK_ORDER] = blocks
    return out.reshape(-1)


def hybrid_layout(R: int, K: int, tile_rows: int, tile_cols: int, flags):
    """H3-H5: (tile_meta [RB, KB, 2], row_meta [RB, 4], total values, total index bytes)."""
    RB, KB = tile_grid(R, K, tile_rows, tile_cols)
    flags = np.asarray(flags).reshape(RB, KB)
    tile_meta = np.zeros((RB, KB, 2), dtype=np.int64)
    row_meta = np.zeros((RB, 4), dtype=np.int64)
    vbase = ibase = 0
    for b in range(RB):
        v = i = 0  # position along the first row of tile-row b
        for j in range(KB):
            tile_meta[b, j, 0] = vbase + v
            if flags[b, j]:
                tile_meta[b, j, 1] = -1
                v += tile_cols
            else:
                tile_meta[b, j, 1] = ibase + i
                v += tile_cols // 2
                i += tile_cols // 8
        row_meta[b] = (v, i, vbase, ibase)
        vbase += rows_of(b, R, tile_rows) * v
        ibase += rows_of(b, R, tile_rows) * i
    return tile_meta, row_meta, vbase, -(-ibase // 16) * 16


def hybrid_pack(w_bits: np.ndarray, tile_rows: int, tile_cols: int, flags):
    """H3: (values uint16 [total], idx uint8 [total bytes]) of a weight matrix."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    R, K = w_bits.shape
    tile_meta, row_meta, nv, ni = hybrid_layout(R, K, tile_rows, tile_cols, flags)
    RB, KB = tile_meta.shape[:2]
    flags = np.asarray(flags).reshape(RB, KB)
    values = np.zeros(nv, dtype=np.uint16)
    idx = np.zeros(ni, dtype=np.uint8)
    for b in range(RB):
        r0, nr = b * tile_rows, rows_of(b, R, tile_rows)
        Lv, Li = row_meta[b, :2]
        for j in range(KB):
            block = w_bits[r0:r0 + nr, j * tile_cols:(j + 1) * tile_cols]
            v0, i0 = tile_meta[b, j]
            for q in range(nr):
                if flags[b, j]:
                    values[v0 + q * Lv: v0 + q * Lv + tile_cols] = dense_store(block[q])
                else:
                    pv, pw = O.prune_pack(block[q:q + 1], 2, 4)
                    values[v0 + q * Lv: v0 + q * Lv + tile_cols // 2] = pv[0]
                    # the tile's bit stream: its first tile_cols/8 bytes
                    idx[i0 + q * Li: i0 + q * Li + tile_cols // 8] = \
                        pw[0].astype("<u4").view(np.uint8)[:tile_cols // 8]
    return values, idx


def hybrid_decompress(values, idx, R: int, K: int, tile_rows: int, tile_cols: int, flags) -> np.ndarray:
    """The weight matrix the packed form stands for (uint16 bits, dropped weights 0)."""
    tile_meta, row_meta, _, _ = hybrid_layout(R, K, tile_rows, tile_cols, flags)
    RB, KB = tile_meta.shape[:2]
    flags = np.asarray(flags).reshape(RB, KB)
    values = np.asarray(values, dtype=np.uint16)
    idx = np.asarray(idx, dtype=np.uint8)
    w = np.zeros((R, K), dtype=np.uint16)
    for b in range(RB):
        r0, nr = b * tile_rows, rows_of(b, R, tile_rows)
        Lv, Li = row_meta[b, :2]
        for j in range(KB):
            v0, i0 = tile_meta[b, j]
            c0 = j * tile_cols
            for q in range(nr):
                if flags[b, j]:
                    w[r0 + q, c0:c0 + tile_cols] = dense_load(values[v0 + q * Lv: v0 + q * Lv + tile_cols])
                else:
                    pv = values[v0 + q * Lv: v0 + q * Lv + tile_cols // 2]
                    pb = idx[i0 + q * Li: i0 + q * Li + tile_cols // 8]
                    padded = np.zeros(-(-len(pb) // 4) * 4, dtype=np.uint8)
                    padded[:len(pb)] = pb
                    words = padded.view("<u4").astype(np.uint32)
                    w[r0 + q, c0:c0 + tile_cols] = O.decompress(pv[None, :], words[None, :], tile_cols, 2, 4)[0]
    return w


def hybrid_spmm_ref(values, idx, R: int, K: int, tile_rows: int, tile_cols: int, flags, act_bits,
                    dtype: str) -> np.ndarray:
    """Y = W_hat X in float64, [R, T]: decompress, then a dense product (X = act^T)."""
    wd = O.half_bits_to_f64(hybrid_decompress(values, idx, R, K, tile_rows, tile_cols, flags), dtype)
    x = O.half_bits_to_f64(np.asarray(act_bits, dtype=np.uint16), dtype).T
    return wd @ x

