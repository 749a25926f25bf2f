"""Pins for the oracle's regularization (sign flips + blockwise Sylvester Hadamard).

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture §7
(natural Sylvester H_128, orthonormalised by 1/sqrt(128), symmetric and its own
inverse, applied per 128-row block on the left and per 128-column block on the
right rather than as one Kronecker transform; decode order H_l, x su, H_r, x sv).
"""
import numpy as np
import pytest

import oracle


def sylvester(B):
    H = np.array([[1]], dtype=np.int64)
    while H.shape[0] < B:
        H = np.block([[H, H], [H, -H]])
    return H


@pytest.mark.parametrize("B", [64, 128])
def test_fwht_equals_dense_sylvester(B):
    rng = np.random.default_rng(B)
    a = rng.integers(-8, 9, size=(2 * B, 5)).astype(np.int64)
    got = oracle.fwht_rows_blockwise(a.astype(np.float32), B)
    H = sylvester(B)
    want = np.concatenate([H @ a[:B], H @ a[B:]])
    assert np.array_equal(got.astype(np.int64), want)      # small integers: exact
    assert np.array_equal(H @ H, B * np.eye(B, dtype=np.int64))
    assert np.array_equal(H, H.T)


def test_normalisation_constants():
    assert oracle.hadamard_norm(64) == np.float32(0.125)
    c = oracle.hadamard_norm(128)
    exact = 1.0 / np.sqrt(128.0)
    assert c == np.float32(exact)
    assert abs(float(c) - exact) <= np.spacing(np.float32(c)) / 2
    with pytest.raises(ValueError):
        oracle.hadamard_norm(32)


@pytest.mark.parametrize("B", [64, 128])
def test_single_entry_closed_form(B):
    R, C = 2 * B, B
    i, j, a = B + 3, 5, np.float32(0.7)
    w = np.zeros((R, C), np.float32)
    w[i, j] = a
    su = np.ones(R, np.float32)
    sv = np.ones(C, np.float32)
    su[i] = -1.0
    out = oracle.regularize(w, su, sv, B)
    c = oracle.hadamard_norm(B)
    mag = np.float32(np.float32(a * c) * c)
    H = sylvester(B)
    want = np.zeros((R, C), np.float32)
    blk = i // B
    want[blk * B:(blk + 1) * B, :] = (-1.0 * H[:, i % B][:, None] * H[j % B, :][None, :]) * mag
    assert np.array_equal(out, want)


@pytest.mark.parametrize("B", [64, 128])
def test_orthonormal_and_invertible(B):
    rng = np.random.default_rng(1)
    w = rng.standard_normal((2 * B, 3 * B)).astype(np.float32)
    su = (2 * rng.integers(0, 2, 2 * B) - 1).astype(np.float32)
    sv = (2 * rng.integers(0, 2, 3 * B) - 1).astype(np.float32)
    out = oracle.regularize(w, su, sv, B)
    n0 = np.linalg.norm(w.astype(np.float64))
    assert abs(np.linalg.norm(out.astype(np.float64)) - n0) <= 2e-6 * n0
    back = oracle.unregularize(out, su, sv, B)
    assert np.max(np.abs(back - w)) <= 2e-6 * np.max(np.abs(w))
    # against the dense definition in binary64
    H = sylvester(B).astype(np.float64) / np.sqrt(B)
    Hl = np.kron(np.eye(2), H)
    Hr = np.kron(np.eye(3), H)
    dense = Hl @ (su[:, None] * w.astype(np.float64) * sv[None, :]) @ Hr
    assert np.max(np.abs(out - dense)) <= 1e-5 * np.max(np.abs(dense))


def test_left_and_right_commute_exactly_on_integers():
    rng = np.random.default_rng(2)
    a = rng.integers(-4, 5, size=(128, 128)).astype(np.float32)
    lr = oracle.fwht_rows_blockwise(oracle.fwht_rows_blockwise(a, 128).T, 128).T
    rl = oracle.fwht_rows_blockwise(oracle.fwht_rows_blockwise(a.T, 128).T, 128)
    assert np.array_equal(lr, rl)


def test_unregularize_against_the_dense_definition():
    """W = diag(su) H_l W_reg H_r diag(sv) in binary64, with non-unit su (folded channel
    scales) -- the inverse's own order of operations is not reused."""
    rng = np.random.default_rng(9)
    B = 64
    w_reg = rng.standard_normal((128, 192)).astype(np.float32)
    su = (rng.standard_normal(128) * 0.3).astype(np.float32)
    sv = (2 * rng.integers(0, 2, 192) - 1).astype(np.float32)
    got = oracle.unregularize(w_reg, su, sv, B)
    H = sylvester(B).astype(np.float64) / np.sqrt(B)
    dense = (su[:, None].astype(np.float64) * (np.kron(np.eye(2), H) @ w_reg.astype(np.float64)
                                               @ np.kron(np.eye(3), H)) * sv[None, :])
    assert np.max(np.abs(got - dense)) <= 2e-6 * np.max(np.abs(dense))
