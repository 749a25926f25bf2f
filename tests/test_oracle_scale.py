"""Pins for the oracle's codebook, scale search and distortion.

Sources: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture §5
(mul1 codebook: count and range of its distinct fp16 levels) and §8 (scale
search over a sampled tile set); "JEV-9B EXL3 K=2 (mul1) Checkpoint" model card
§2 (golden-section scale search) and §3 (K=2 distortion band).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fig():
    with open(os.path.join(GOLDEN, "pages_figures.json")) as f:
        return json.load(f)


def all_fp16_values():
    bits = np.arange(1 << 16, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    ok = np.isfinite(vals)
    return bits[ok], vals[ok]


def test_codebook_rounding_is_nearest_fp16():
    """Each level is the fp16 nearest to (beta - mean) / std (ties to even mantissa).

    The binary64 quotient is formed from exact integer sums; it is first checked
    against numpy's own mean/std, then every distinct value is rounded by a
    brute-force search over all finite fp16 numbers.
    """
    n = 1 << 16
    h = [(s * oracle.MUL1_MULTIPLIER) & 0xFFFFFFFF for s in range(n)]
    beta = np.array([sum((v >> (8 * i)) & 0xFF for i in range(4)) for v in h], np.int64)
    s1 = int(beta.sum())
    s2 = int((beta * beta).sum())
    z = (n * beta - s1).astype(np.float64) / math.sqrt(float(n * s2 - s1 * s1))
    bf = beta.astype(np.float64)
    assert np.max(np.abs(z - (bf - bf.mean()) / bf.std())) < 1e-12
    lv = oracle.mul1_levels_fp16()
    fbits, fvals = all_fp16_values()
    order = np.argsort(fvals, kind="stable")
    fvals, fbits = fvals[order], fbits[order]
    for zz in np.unique(z):
        i = int(np.searchsorted(fvals, zz))
        cand = [j for j in (i - 1, i) if 0 <= j < len(fvals)]
        dist = [abs(fvals[j] - zz) for j in cand]
        near = [cand[k] for k in range(len(cand)) if dist[k] == min(dist)]
        if len(near) > 1:
            near = [j for j in near if (int(fbits[j]) & 1) == 0]
        got = lv[np.flatnonzero(z == zz)]
        assert np.all(got.view(np.uint16) == fbits[near[0]])


def test_codebook_distribution_and_pages_probe():
    lv = oracle.mul1_levels_fp16().astype(np.float64)
    assert abs(lv.mean()) < 1e-3
    assert 0.95 < lv.var() < 1.05
    assert np.abs(lv).max() < 3.5
    fig = _fig()["mul1"]
    # the pages give the count of distinct levels; this construction matches it
    assert len(np.unique(lv)) == fig["distinct_levels"]
    # the range is reported, not asserted: upstream levels are not reproduced
    lo, hi = lv.min(), lv.max()
    assert lo < 0 < hi
    assert abs(lo - fig["range"][0]) < 0.1 and abs(hi - fig["range"][1]) < 0.1


def test_golden_section_on_quadratic():
    s0 = 1.234567
    calls = []

    def f(s):
        calls.append(s)
        return (s - s0) ** 2

    lo, hi, it = 0.5, 2.0, 12
    mid, trace = oracle.golden_section(f, lo, hi, it)
    assert len(calls) == it + 2 == len(trace)
    width = (hi - lo) * oracle.GOLDEN ** it
    assert abs(mid - s0) <= width / 2
    g = (math.sqrt(5) - 1) / 2
    assert abs(oracle.GOLDEN - g) < 1e-16
    # probes are symmetric in the first bracket
    assert abs((trace[0][0] - lo) - (hi - trace[1][0])) < 1e-12


def test_golden_section_picks_left_on_strict_less_only():
    # constant function: every comparison is "not less", so the left end moves up
    mid, trace = oracle.golden_section(lambda s: 1.0, 0.0, 1.0, 12)
    assert mid > 1.0 - oracle.GOLDEN ** 12


@pytest.mark.slow
def test_golden_section_real_objective_against_scan():
    m = workloads.config(1)[0]
    tiles = oracle.to_tiles(oracle.regularize(m.w, m.su, m.sv, 64))[:4]
    levels = oracle.mul1_levels_fp16()

    def f(s):
        r = oracle.encode_tiles(tiles, 2, np.float32(s), levels)
        return float(sum(float(e) for e in r["sse"]))

    mid, _ = oracle.golden_section(f, 0.5, 2.0, 12)
    scan = [f(s) for s in np.linspace(0.5, 2.0, 16)]
    assert f(mid) <= min(scan) * 1.01


@pytest.mark.parametrize("K", [2, 3, 4])
def test_gaussian_distortion_band(K):
    """Normalised MSE of an i.i.d. Gaussian lies between the rate-distortion bound
    2^(-2K) and the optimal scalar quantiser at K bits (Max, 1960)."""
    fig = _fig()
    x = workloads.random_tiles(6, 77)
    r = oracle.encode_tiles(x, K, 1.0)
    nmse = float(r["sse"].astype(np.float64).sum()) / float((x.astype(np.float64) ** 2).sum())
    assert 2.0 ** (-2 * K) < nmse < fig["lloyd_max_gaussian_mse"][str(K)]


def test_distortion_monotone_in_K():
    x = workloads.random_tiles(4, 78)
    m = [float(oracle.encode_tiles(x, K, 1.0)["sse"].astype(np.float64).sum()) for K in (2, 3, 4)]
    assert m[0] > m[1] > m[2]


@pytest.mark.slow
def test_config1_whole_path_matches_golden_and_pages_band():
    """Workload 1 end to end; stored values come from tests/golden/make_golden.py."""
    with open(os.path.join(GOLDEN, "config1_oracle.json")) as f:
        g = json.load(f)
    m = workloads.config(1)[0]
    out = oracle.quantize_matrix(m.w, m.su, m.sv, m.K, had_block=m.had_block, gss=None,
                                 fixed_scale=1.0)
    assert out["packed"].astype(np.int64).ravel().tolist() == g["packed"]
    assert [int(x) for x in out["X"]] == g["X"]
    assert out["sse"].view(np.uint32).tolist() == g["sse_bits"]
    rel_frob = math.sqrt(out["mse"] * m.w.size / float((m.w.astype(np.float64) ** 2).sum()))
    lo, hi = _fig()["k2_rel_frobenius_band"]
    assert lo <= rel_frob <= hi
