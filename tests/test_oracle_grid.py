"""Pins for the oracle's grid + parabolic scale search.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 8
(coarse grid 0.1..1.9 on a strided subsample, fine grid 0.075 around the coarse
minimum on the full sample, parabolic refinement with a 0.01 floor).

Parabolic interpolation through three equally spaced points recovers the vertex
of a quadratic exactly, so quadratic objectives pin the refinement formula (its
sign and its factor 2); piecewise objectives pin the grid geometry, the tie rule,
the edge case and the floor.
"""
import numpy as np
import pytest

import oracle
import workloads

G = oracle.GRID_DEFAULT


def _counting(f):
    calls = []

    def g(x):
        calls.append(x)
        return f(x)
    return g, calls


@pytest.mark.parametrize("g0", [0.8237, 1.3141, 0.3333])
def test_quadratic_vertex_is_recovered(g0):
    f = lambda g: 3.0 * (g - g0) ** 2 + 1.0
    fs, cs = _counting(f)
    ff, cf = _counting(f)
    g, trace = oracle.grid_search(fs, ff, G)
    assert abs(g - g0) < 1e-12
    assert len(cs) == 19 and len(cf) == 7
    assert cs[0] == pytest.approx(0.1) and cs[-1] == pytest.approx(1.9)
    # the fine grid is centred on the coarse point nearest g0
    gc = min((0.1 + k * 0.1 for k in range(19)), key=lambda x: abs(x - g0))
    assert cf[3] == pytest.approx(gc)
    assert cf[0] == pytest.approx(gc - 0.075) and cf[-1] == pytest.approx(gc + 0.075)


def test_coarse_ties_keep_the_lowest_multiplier():
    g, trace = oracle.grid_search(lambda g: 5.0, lambda g: (g - 0.05) ** 2, G)
    coarse = [t for t in trace if t[0] == "coarse"]
    fine = [t for t in trace if t[0] == "fine"]
    assert fine[3][1] == pytest.approx(0.1)            # centred on the first coarse point
    assert abs(g - 0.05) < 1e-12                       # then the quadratic vertex


def test_minimum_at_the_fine_edge_is_not_refined():
    g, trace = oracle.grid_search(lambda g: (g - 1.0) ** 2, lambda g: -g, G)
    assert g == pytest.approx(1.0 + 0.075)


def test_floor():
    grid = G[:6] + (0.06,)
    g, _ = oracle.grid_search(lambda g: (g - 0.1) ** 2, lambda g: (g - 0.04) ** 2, grid)
    assert g == 0.06


def test_matrix_scale_comes_from_the_search():
    m = workloads.gaussian(128, 256, 0.02, 5, 6, K=2)
    out = oracle.quantize_matrix(m.w, m.su, m.sv, 2, gss=None, grid=G)
    g = out["trace"][-1][1]
    assert out["scale"] == np.float32(g * out["rms"])
    # the coarse stage used every other sample tile, the fine stage all of them
    coarse = [t for t in out["trace"] if t[0] == "coarse"]
    fine = [t for t in out["trace"] if t[0] == "fine"]
    assert len(coarse) == 19 and len(fine) == 7
    tiles = oracle.to_tiles(oracle.regularize(m.w, m.su, m.sv, 128))
    for (_, g_, v), idx in ((coarse[7], out["sample"][::2]), (fine[2], out["sample"])):
        r = oracle.encode_tiles(tiles[idx], 2, np.float32(g_ * out["rms"]))
        assert v == sum(float(e) for e in r["sse"].tolist())
