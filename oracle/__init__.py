"""Oracle for the EXL3 trellis tile encoder -- TEST INFRASTRUCTURE ONLY.

A plain CPU implementation of what the GPU library computes, written from the
sources' description.  It is imported only by the test-suite, by
``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``; the
library never imports, links or calls it, and it never imports the library.

Every function here is pinned by a check that does not reuse its own formula
(brute force on tiny trellises, closed forms, invariants, special cases); the
one part with no such pin -- agreement of the mul1 levels with the upstream
codebook -- is marked "parity unpinned" in ``reference.py``.
"""
from .reference import (  # noqa: F401
    GOLDEN, MUL1_MULTIPLIER, STATE_BITS, encode_sequences, encode_tiles, forward,
    from_tiles, fwht_rows_blockwise, golden_section, hadamard_norm, matrix_rms,
    mul1_levels_fp16, pack_states, quantize_matrix, regularize, sample_tiles,
    scaled_levels, tile_sse, tile_sumsq, to_tiles, unpack_states, unregularize,
    default_threads, encode_sequences_f16, encode_tiles_f16, f16_sqadd, f16_sub, forward_f16,
    ldlq, quantize_matrix_ldlq, grid_search, GRID_DEFAULT, channel_normalize, CHANNEL_FLOOR,
    mcg_levels_fp16, inst3_levels_fp16, CODEBOOKS, to_f16_inputs, encode_tiles_f16_scaled,
    quantize_matrix_f16, check_order,
)
