"""Pins for the oracle-written workload digests (tests/golden/config_digests.json).

The GPU check hashes the library's full outputs against this file, so the file
itself is checked here against things other than itself:
  * every run the five workloads call for is present, with its fields;
  * workload 1 (16 tiles), recomputed with the oracle now, matches its entry;
  * each stored MSE of a Gaussian workload lies between the rate-distortion
    bound of an i.i.d. Gaussian at K bits (2^-2K of the variance) and the
    optimal scalar quantiser's distortion at K bits (Lloyd-Max), the variance
    being the stored rms squared;
  * on every matrix of workload 5 the same 1,024 tiles' error falls from K = 2
    to 3 to 4, by at least a factor 2 per bit;
  * the stored scale lies in the search bracket [0.5, 2.0] x rms, and its bits
    are the binary32 rounding of the midpoint of the stored trace's last
    bracket as the golden section narrows it.
"""
import hashlib
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "config_digests.json")
LLOYD_MAX = {1: 0.3634, 2: 0.1175, 3: 0.03454, 4: 0.009497}


def _runs():
    with open(GOLDEN) as f:
        return json.load(f)["runs"]


def _expected_keys():
    keys = ["c1_c1_64x64_K2", "c2_c2_4096x4096_K2", "c3_c3_4096x4096_t4_K4",
            "c4_c4_4096x12288_K3", "c4_c4_12288x4096_K3", "f16_c2_c2_4096x4096_K2"]
    keys += ["c5_%s_K%d" % (name, K) for name, _, _ in workloads.LAYER_SHAPES for K in (2, 3, 4)]
    return keys


def _f32(bits):
    return np.uint32(int(bits, 16)).view(np.float32)


def test_every_run_is_present():
    runs = _runs()
    assert sorted(runs) == sorted(_expected_keys())
    for k, d in runs.items():
        for field in ("scale_bits", "packed_sha256", "sse_sha256", "sse_sum", "rms", "trace",
                      "n_tiles", "first_tile_packed", "first_tile_sse_bits"):
            assert field in d, (k, field)
        assert len(d["first_tile_packed"]) == 16 * d["K"]


def test_workload1_recomputed():
    d = _runs()["c1_c1_64x64_K2"]
    m = workloads.config(1)[0]
    r = oracle.quantize_matrix(m.w, m.su, m.sv, m.K, had_block=m.had_block, gss=None,
                               fixed_scale=1.0)
    assert d["scale_bits"] == "0x3f800000"
    assert hashlib.sha256(np.ascontiguousarray(r["packed"], "<u2").tobytes()).hexdigest() == \
        d["packed_sha256"]
    assert hashlib.sha256(np.ascontiguousarray(r["sse"], "<f4").tobytes()).hexdigest() == \
        d["sse_sha256"]
    assert repr(r["mse"]) == d["mse"]


def test_gaussian_distortion_bounds():
    for k, d in _runs().items():
        if d["config"] not in (1, 2, 4) or d["mse"] is None:
            continue
        nmse = float(d["mse"]) / float(d["rms"]) ** 2
        assert 2.0 ** (-2 * d["K"]) < nmse < LLOYD_MAX[d["K"]], (k, nmse)


def test_layer_error_falls_with_k():
    runs = _runs()
    for name, _, _ in workloads.LAYER_SHAPES:
        e = [float(runs["c5_%s_K%d" % (name, K)]["sse_sum"]) for K in (2, 3, 4)]
        assert e[0] > 2 * e[1] > 4 * e[2] > 0, (name, e)


def test_scale_is_the_final_bracket_midpoint():
    g = (math.sqrt(5.0) - 1.0) / 2.0
    for k, d in _runs().items():
        if d["gss"] is None:
            continue
        iters, lo, hi = d["gss"]
        rms = float(d["rms"])
        trace = [(float(s), float(f)) for s, f in d["trace"]]
        assert len(trace) == iters + 2
        # replay the bracket updates from the stored objective values
        a, b = lo * rms, hi * rms
        p, q = b - (b - a) * g, a + (b - a) * g
        fp, fq = trace[0][1], trace[1][1]
        assert (trace[0][0], trace[1][0]) == (p, q)
        for s, f in trace[2:]:
            if fp < fq:
                b, q, fq = q, p, fp
                p = b - (b - a) * g
                assert s == p
                fp = f
            else:
                a, p, fp = p, q, fq
                q = a + (b - a) * g
                assert s == q
                fq = f
        assert _f32(d["scale_bits"]) == np.float32((a + b) / 2.0), k
        assert lo * rms <= float(_f32(d["scale_bits"])) <= hi * rms
