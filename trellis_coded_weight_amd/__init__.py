"""EXL3 trellis tile encoder for AMD Instinct MI355X (gfx950).

The work happens in hand-written HIP kernels behind a small C ABI
(include/exl3.h, built as _lib/libexl3_gfx950.so); ``binding`` marshals torch
tensors into it.  There is no CPU fallback.
"""
from .binding import (  # noqa: F401
    CODEBOOK_KINDS, EXPORTED, GRID_PAGES, Context, Exl3Error, EXL3_BF16, EXL3_EHIP, EXL3_EINVAL, EXL3_ENOMEM,
    EXL3_ENONFINITE, EXL3_EUNSUPPORTED, EXL3_F32, EXL3_OK, EXL3_ROW_MAJOR, EXL3_TILE_MAJOR, library_path, load_library,
    quantize_matrix, scratch_per_tile, version,
)
