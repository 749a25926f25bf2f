"""Every output of the five workloads, at full size, against the oracle's digests.

tests/golden/config_digests.json is written by tests/golden/make_config_digests.py,
which calls only the oracle and the seeded input generators.  For each
(workload, matrix, K) it stores the binary32 bits of the scale the golden-section
search chose, the SHA-256 of the container words and of the per-tile squared
errors, and the binary64 mean squared error.  Here the GPU library quantizes
the same matrices and its whole outputs are hashed the same way: bit-exact
agreement on every tile of workloads 1-4 and on every scale of workload 5
(with 1,024 evenly spaced tiles of each of its 21 runs), plus the binary16
whole-matrix path's scale on workload 2's matrix.  No oracle runs here.
"""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "config_digests.json")
RUNS = json.load(open(GOLDEN))["runs"] if os.path.exists(GOLDEN) else {}

_matrices = {}


def _matrix(config, name):
    if (config, name) not in _matrices:
        _matrices.clear()                   # keep one workload's matrices at a time
        for m in workloads.config(config):
            _matrices[(config, m.name)] = m
    return _matrices[(config, name)]


@pytest.fixture(scope="module")
def ctx():
    import trellis_coded_weight_amd as T
    c = T.Context(0)
    yield c
    c.close()


def _sha(a, dtype):
    return hashlib.sha256(np.ascontiguousarray(a, dtype=dtype).tobytes()).hexdigest()


def _bits(x):
    return "0x%08x" % int(np.float32(x).view(np.uint32))


@pytest.mark.parametrize("key", sorted(RUNS, key=lambda k: (RUNS[k]["config"], k)))
def test_workload_matches_oracle_digest(ctx, key):
    d = RUNS[key]
    m = _matrix(d["config"], d["matrix"])
    print("digest run %s: %dx%d K=%d" % (key, d["rows"], d["cols"], d["K"]), flush=True)
    dt = torch.bfloat16 if d["dtype"] == "bf16" else torch.float32
    w = torch.from_numpy(m.w).to(dt).to(DEV)
    su = torch.from_numpy(m.su).to(DEV)
    sv = torch.from_numpy(m.sv).to(DEV)
    gss = tuple(d["gss"]) if d["gss"] else None
    scale = d["fixed_scale"] if d["fixed_scale"] is not None else 1.0
    q = ctx.quantize_matrix_f16 if d["binary16_search"] else ctx.quantize_matrix
    got = q(w, d["K"], su, sv, had_block=d["had_block"], gss=gss, scale=scale,
            want_tile_sse=True)
    torch.cuda.synchronize()
    assert _bits(got["scale"]) == d["scale_bits"], "%s: scale %r" % (key, got["scale"])
    n = d["n_tiles"]
    packed = got["packed"].cpu().numpy().view(np.uint16).reshape(n, 16 * d["K"])
    sse = got["tile_sse"].cpu().numpy().reshape(n)
    if d["tiles"] == "all":
        sel = slice(None)
    else:
        count = d["tiles"]["evenly_spaced"]
        sel = (np.arange(count, dtype=np.int64) * n) // count
    p, e = packed[sel], sse[sel]
    assert [int(v) for v in p[0]] == d["first_tile_packed"], key
    assert _bits(e[0]) == d["first_tile_sse_bits"], key
    assert _sha(p, "<u2") == d["packed_sha256"], "%s: container words differ" % key
    assert _sha(e, "<f4") == d["sse_sha256"], "%s: per-tile squared errors differ" % key
    total = 0.0
    for v in e.tolist():
        total += float(v)
    assert repr(total) == d["sse_sum"], key
    if d["mse"] is not None:
        assert repr(float(got["mse"])) == d["mse"], "%s: mse %r" % (key, got["mse"])
