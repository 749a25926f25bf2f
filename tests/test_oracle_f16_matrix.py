"""Pins for the oracle's whole-matrix path with the binary16 encoder inside.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 1
(the encoder searches in half precision) and item 8 (scale search over the tile
sample); "JEV-9B EXL3 K=2 (mul1) Checkpoint" model card, section 2 (golden section).

Pinned independently of the oracle's own formulas: the encoder inputs against
exact rational division with a brute-force nearest binary32 then binary16
(ties to even), powers of two in closed form; the tile errors against exact
rational arithmetic within the sequential-sum bound (which also pins that the
dequantized value is the scaled level); the composition (fixed scale equals
the binary16 encoder on the converted tiles).  The whole search is checked
against the GPU library in the GPU tests (the binary16 oracle is too slow for
a search on the CPU suite's budget).
"""
from fractions import Fraction

import numpy as np

import oracle
import workloads


def _nearest(x: Fraction, candidates: np.ndarray) -> float:
    """Nearest of the candidate floats to x, ties to the even significand."""
    best = None
    for c in candidates.tolist():
        d = abs(Fraction(c) - x)
        key = (d, int(np.float32(c).view(np.uint32)) & 1 if candidates.dtype == np.float32
               else int(np.float16(c).view(np.uint16)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _ref_input_bits(w: float, s: float) -> int:
    q = Fraction(float(w)) / Fraction(float(s))
    f = np.float32(float(q))
    c32 = np.array([np.nextafter(f, -np.inf, dtype=np.float32), f,
                    np.nextafter(f, np.inf, dtype=np.float32)], np.float32)
    q32 = Fraction(_nearest(q, c32))
    h = np.float16(float(q32))
    c16 = np.array([np.nextafter(h, np.float16(-np.inf)), h,
                    np.nextafter(h, np.float16(np.inf))], np.float16)
    return int(np.float16(_nearest(q32, c16)).view(np.uint16))


def test_inputs_by_exact_division():
    rng = np.random.Generator(np.random.PCG64(3))
    w = (rng.standard_normal(400) * 0.02).astype(np.float32)
    for s in (np.float32(0.0173), np.float32(0.02291), np.float32(1e-3)):
        got = oracle.to_f16_inputs(w.reshape(1, -1)[:, :400], s).reshape(-1)
        for i in range(0, 400, 7):
            assert int(got[i]) == _ref_input_bits(w[i], s), (s, i)


def test_inputs_power_of_two_and_zero_scale():
    t = workloads.random_tiles(3, 4, std=1.0)
    got = oracle.to_f16_inputs(t, np.float32(0.25))
    assert np.array_equal(got, (t * np.float32(4.0)).astype(np.float16).view(np.uint16))
    assert not np.any(oracle.to_f16_inputs(t, 0.0))


def test_tile_errors_by_exact_arithmetic():
    t = workloads.random_tiles(4, 11, std=0.02)
    s = np.float32(0.0201)
    r = oracle.encode_tiles_f16_scaled(t, 2, s)
    levels = oracle.mul1_levels_fp16()
    for i in range(4):
        exact = Fraction(0)
        for j in range(256):
            v = np.float32(s * np.float32(levels[r["states"][i, j]]))   # rn32(scale * level)
            exact += (Fraction(float(t[i, j])) - Fraction(float(v))) ** 2
        assert abs(float(r["sse"][i]) - float(exact)) <= 3e-5 * float(exact)


def test_fixed_scale_is_the_encoder_on_converted_tiles():
    m = workloads.gaussian(64, 128, 0.02, 21, 22, K=2)
    s = np.float32(0.019)
    pick = [0, 13]
    out = oracle.quantize_matrix_f16(m.w, m.su, m.sv, 2, had_block=64, gss=None, fixed_scale=s,
                                     tiles_subset=pick)
    tiles = oracle.to_tiles(oracle.regularize(m.w, m.su, m.sv, 64))
    want = oracle.encode_tiles_f16(oracle.to_f16_inputs(tiles[pick], s), 2)
    assert np.array_equal(out["packed"], want["packed"])
    assert out["scale"] == s
