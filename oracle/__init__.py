"""CPU oracle (test infrastructure only; see nm_oracle's module docstring)."""
from .nm_oracle import *  # noqa: F401,F403
from .nm_oracle import (  # noqa: F401
    half_bits_to_f64, magnitude_keys, index_bits, survivors_per_row, idx_words_per_row,
    select_survivors, pack_values, pack_indices, prune_pack, unpack_indices, decompress,
    spmm_ref, spmm_rows_ref, relative_error,
)
