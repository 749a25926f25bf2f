"""The C-ABI library loads and exports every function include/exl3.h declares.

No compute call is made (there may be no GPU here).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "exl3.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(exl3_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("exl3_regularize", "exl3_encode_tiles", "exl3_decode_tiles",
                     "exl3_quantize_matrix", "exl3_ctx_create", "exl3_ctx_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol():
    from trellis_coded_weight_amd import binding
    path = binding.library_path()
    if not os.path.exists(path):
        pytest.skip("library not built")
    lib = ctypes.CDLL(path)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(binding.EXPORTED) == set(declared_functions())


def test_scratch_per_tile_without_gpu():
    from trellis_coded_weight_amd import binding
    if not os.path.exists(binding.library_path()):
        pytest.skip("library not built")
    lib = binding.load_library()
    assert lib.exl3_scratch_per_tile(2) == 255 * 1024 * 4
    assert lib.exl3_scratch_per_tile(3) == 255 * 1024 * 4
    assert lib.exl3_scratch_per_tile(4) == 255 * 1024 * 2
    assert lib.exl3_scratch_per_tile(5) == 0
    assert lib.exl3_version().decode().startswith("exl3-gfx950")


def test_oracle_and_library_share_no_code():
    """The oracle never imports the library and the library never imports the oracle."""
    for d, forbidden in (("oracle", "trellis_coded_weight_amd"), ("trellis_coded_weight_amd", "oracle")):
        for dirpath, _, files in os.walk(os.path.join(ROOT, d)):
            for f in files:
                if f.endswith((".py", ".c", ".cpp", ".hip", ".h")):
                    src = open(os.path.join(dirpath, f)).read()
                    assert not re.search(r"^\s*(import|from)\s+%s\b" % forbidden, src, re.M), f
                    assert "#include" not in src or forbidden not in re.findall(r'#include\s+"([^"]+)"', src)
