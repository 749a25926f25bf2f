"""Binary16 mode of the GPU encoder against the oracle, through the C ABI.

Source of the mode: "EXL3 Intel Arc Quantizer" README, Core Implemented
Architecture sections 1 and 4 (half-precision add-compare-select with one
fused rounding of the path cost; first branch wins on equal costs).

Bar: bit-exact states, packed words and binary16 path costs for every tile,
including batches split by a small scratch bound, inputs that drive every cost
to +inf (all ties), constant tiles (many ties), subnormal inputs and an empty
call.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ctx():
    import trellis_coded_weight_amd as T
    c = T.Context(0)
    yield c
    c.close()


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


def _half_tiles(n, seed, std=1.0):
    return workloads.random_tiles(n, seed, std).astype(np.float16)


def _check(ctx, xh, K, tag):
    print("\nf16 %s K=%d n=%d" % (tag, K, xh.shape[0]), flush=True)
    want = oracle.encode_tiles_f16(xh.view(np.uint16), K)
    packed, states, cost = ctx.encode_tiles_f16(torch.from_numpy(xh).to(DEV), K)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(states), want["states"].astype(np.uint16))
    assert np.array_equal(_u16(packed), want["packed"])
    assert np.array_equal(_u16(cost), want["cost"])


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_f16_encode_bit_exact(ctx, K):
    _check(ctx, _half_tiles(21, 300 + K), K, "gaussian")


@pytest.mark.parametrize("K", [2, 4])
def test_f16_encode_wide_inputs(ctx, K):
    # inputs well outside the level range: large costs, coarse binary16 steps
    _check(ctx, _half_tiles(6, 310 + K, std=12.0), K, "wide")


def test_f16_encode_edge_tiles(ctx):
    K = 2
    rng = np.random.default_rng(7)
    tiles = [
        np.zeros(256, np.float16),                              # exact zeros
        np.full(256, 0.5, np.float16),                          # constant: many ties
        np.full(256, 60000.0, np.float16),                      # every cost +inf: all ties
        (rng.standard_normal(256) * 1e-6).astype(np.float16),   # subnormal inputs
        np.where(np.arange(256) % 2 == 0, 200.0, -200.0).astype(np.float16),  # costs overflow
    ]
    _check(ctx, np.stack(tiles), K, "edge")


def test_f16_batches_and_empty(ctx):
    import trellis_coded_weight_amd as T
    K = 3
    xh = _half_tiles(11, 333)
    want = oracle.encode_tiles_f16(xh.view(np.uint16), K)
    xd = torch.from_numpy(xh).to(DEV)
    # scratch for 4 tiles: batches of 4, 4, 3
    with T.Context(0, scratch_bytes=T.scratch_per_tile(K) * 4) as small:
        packed, states, cost = small.encode_tiles_f16(xd, K)
        torch.cuda.synchronize()
    assert np.array_equal(_u16(packed), want["packed"])
    assert np.array_equal(_u16(states), want["states"].astype(np.uint16))
    assert np.array_equal(_u16(cost), want["cost"])
    empty = torch.empty(0, 256, dtype=torch.float16, device=DEV)
    p0, s0, c0 = ctx.encode_tiles_f16(empty, K)
    assert p0.shape == (0, 16 * K) and c0.shape == (0,)


def test_f16_rejects_bad_k(ctx):
    import trellis_coded_weight_amd as T
    with pytest.raises(T.Exl3Error):
        ctx.encode_tiles_f16(torch.zeros(1, 256, dtype=torch.float16, device=DEV), 5)


def test_f16_decode_roundtrip(ctx):
    """The container written in binary16 mode decodes to the levels of its states."""
    K = 2
    xh = _half_tiles(5, 340)
    packed, states, _ = ctx.encode_tiles_f16(torch.from_numpy(xh).to(DEV), K)
    dec = ctx.decode_tiles(packed, K, 1.0).cpu().numpy()
    lv = oracle.mul1_levels_fp16().astype(np.float32)
    assert np.array_equal(dec, lv[_u16(states).astype(np.int64)])
