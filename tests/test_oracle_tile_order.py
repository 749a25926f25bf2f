"""Pins for the oracle's within-tile order (the tensor-core permutation hook).

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 5
(a fixed 256-element permutation of the positions within a tile and its
inverse, for the tensor-core decoder; the table itself is not printed) and
item 3 (LDLQ permutes the target tiles before encoding and reconstructs in
matrix order).

Pinned without the oracle's own indexing: the transposing order against NumPy's
transpose of the matrix, round trips for random orders, the identity against the
default, and, at the whole-matrix level, that an order only relabels positions:
with a scalar-quantiser level table (level = function of the low K bits only,
where each position is quantized on its own) the reconstruction in matrix order
does not depend on the order.
"""
import numpy as np
import pytest

import oracle
import workloads

TRANSPOSE = np.array([16 * (t % 16) + t // 16 for t in range(256)])


def test_transposing_order_is_the_transposed_matrix():
    m = np.random.default_rng(4).standard_normal((32, 48)).astype(np.float32)
    got = oracle.to_tiles(m, TRANSPOSE)
    # tile (tr, tc) in transposed order = tile (tc, tr) of m^T in row-major order
    want_t = oracle.to_tiles(np.ascontiguousarray(m.T))
    TR, TC = 2, 3
    for tr in range(TR):
        for tc in range(TC):
            assert np.array_equal(got[tr * TC + tc], want_t[tc * TR + tr])


def test_position_t_holds_element_order_t():
    # a cyclic shift is not its own inverse, so this fixes the direction of the
    # table: position t holds element order[t] (not element t at position order[t])
    m = np.arange(16 * 16, dtype=np.float32).reshape(16, 16)   # element e has value e
    shift = (np.arange(256) + 1) % 256
    t = oracle.to_tiles(m, shift)[0]
    assert t[0] == 1.0 and t[15] == 16.0 and t[255] == 0.0


def test_round_trip_and_identity():
    rng = np.random.default_rng(5)
    m = rng.standard_normal((48, 32)).astype(np.float32)
    for _ in range(3):
        o = rng.permutation(256)
        t = oracle.to_tiles(m, o)
        assert np.array_equal(oracle.from_tiles(t, 48, 32, o), m)
        assert not np.array_equal(t, oracle.to_tiles(m))
    assert np.array_equal(oracle.to_tiles(m, np.arange(256)), oracle.to_tiles(m))


@pytest.mark.parametrize("bad", [np.arange(255), np.r_[np.arange(255), 0], np.arange(1, 257)])
def test_rejects_non_permutations(bad):
    with pytest.raises(ValueError):
        oracle.to_tiles(np.zeros((16, 16), np.float32), bad)


def test_scalar_quantiser_reconstruction_is_order_free():
    # levels depend only on the low 2 bits of the state: every position is then
    # quantized on its own (nearest level), so only the labelling changes
    lev = np.array([-1.25, -0.375, 0.5, 1.5], np.float16)
    lv = lev[np.arange(65536) & 3]
    m = workloads.gaussian(64, 64, 1.0, 31, 32, K=2)
    o = np.random.default_rng(6).permutation(256)
    a = oracle.quantize_matrix(m.w, m.su, m.sv, 2, had_block=64, gss=None, fixed_scale=1.0,
                               levels=lv)
    b = oracle.quantize_matrix(m.w, m.su, m.sv, 2, had_block=64, gss=None, fixed_scale=1.0,
                               levels=lv, order=o)
    v = oracle.scaled_levels(lv, 1.0)
    ra = oracle.from_tiles(v[a["states"]], 64, 64)
    rb = oracle.from_tiles(v[b["states"]], 64, 64, o)
    assert np.array_equal(ra, rb)
    # and the tile energies are sums of the same squares in another order
    assert np.allclose(a["sumsq"], b["sumsq"], rtol=1e-5)


def test_ldlq_scalar_quantiser_is_order_free():
    # the same at the LDLQ level: targets, reconstruction and errors in matrix
    # order do not depend on the order when each position is quantized alone
    lev = np.array([-1.25, -0.375, 0.5, 1.5], np.float16)
    lv = lev[np.arange(65536) & 3]
    rng = np.random.default_rng(7)
    w = rng.standard_normal((32, 64)).astype(np.float32)
    L = np.tril(rng.standard_normal((64, 64)).astype(np.float32) * np.float32(0.1), -16)
    o = rng.permutation(256)
    a = oracle.ldlq(w, L, 2, np.float32(1.0), lv)
    b = oracle.ldlq(w, L, 2, np.float32(1.0), lv, order=o)
    assert np.array_equal(a["what"], b["what"])
    assert np.array_equal(a["targets"], b["targets"])
    # each position's own code (the state's low K bits) moves with the relabelling;
    # the higher bits hold earlier positions' codes and do not
    assert np.array_equal(oracle.from_tiles(a["states"] & 3, 32, 64),
                          oracle.from_tiles(b["states"] & 3, 32, 64, o))
