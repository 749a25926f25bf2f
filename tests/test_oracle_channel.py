"""Pins for the oracle's out-channel RMS normalization.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 8
(out-channel RMS normalization, sign + scale folding, zero-channel floor and the
zero-sign rule).  The pins use closed forms (rows of one power-of-two magnitude
have that magnitude as their rms, so the normalized row is exactly +-1),
invariants (scaling a row by a power of two changes only its folded sign), the
exact sum of squares, and the decode round trip through the regularization.
A transposed axis, a wrong divisor, a missing square root or a dropped sign
fails at least one of them.
"""
import math

import numpy as np

import oracle
import workloads


def _signs(n, seed):
    return workloads.signs(np.random.Generator(np.random.PCG64(seed)), n)


def test_power_of_two_rows_normalize_to_signs():
    R, C = 32, 64                                   # non-square: pins the axis and divisor
    k = np.arange(R) % 7 - 3                        # magnitudes 2^-3 .. 2^3 by row
    pattern = _signs(R * C, 1).reshape(R, C)
    w = pattern * np.ldexp(np.float32(1.0), k)[:, None].astype(np.float32)
    su = _signs(R, 2)
    w_n, su_f, r = oracle.channel_normalize(w, su)
    assert np.array_equal(w_n, pattern)
    assert np.array_equal(r, np.ldexp(1.0, k))
    assert np.array_equal(su_f, su * np.ldexp(np.float32(1.0), k).astype(np.float32))


def test_zero_channel_folds_to_zero():
    m = workloads.channel_spread(48, 32, 11, 12, bf16=False, dead=0.05)
    dead = np.flatnonzero(~m.w.any(axis=1))
    assert dead.size == 2
    w_n, su_f, r = oracle.channel_normalize(m.w, m.su)
    assert np.all(np.isfinite(w_n))
    assert np.all(w_n[dead] == 0.0) and np.all(su_f[dead] == 0.0) and np.all(r[dead] == 0.0)
    live = np.setdiff1d(np.arange(48), dead)
    assert np.all(np.sign(su_f[live]) == m.su[live])
    assert oracle.CHANNEL_FLOOR == 0.1


def test_rms_is_the_exact_mean_square_root():
    m = workloads.channel_spread(40, 96, 21, 22, bf16=True)
    _, _, r = oracle.channel_normalize(m.w, m.su)
    for i in range(40):
        exact = math.sqrt(math.fsum(float(x) ** 2 for x in m.w[i]) / 96)
        assert abs(r[i] - exact) <= 4e-16 * max(exact, 1e-300)


def test_row_scaling_moves_only_the_folded_sign():
    m = workloads.channel_spread(16, 128, 31, 32, bf16=False, dead=0.0)
    w2 = m.w.copy()
    w2[3] *= np.float32(8.0)
    w2[9] *= np.float32(0.25)
    a = oracle.channel_normalize(m.w, m.su)
    b = oracle.channel_normalize(w2, m.su)
    assert np.array_equal(a[0], b[0])
    ratio = np.ones(16, np.float32)
    ratio[3], ratio[9] = 8.0, 0.25
    assert np.array_equal(b[1], a[1] * ratio)


def test_normalized_rows_have_unit_rms_and_columns_do_not():
    m = workloads.channel_spread(64, 256, 41, 42, bf16=True, dead=0.0)
    w_n, _, _ = oracle.channel_normalize(m.w, m.su)
    row_rms = np.sqrt(np.mean(w_n.astype(np.float64) ** 2, axis=1))
    assert np.max(np.abs(row_rms - 1.0)) < 1e-6
    col_rms = np.sqrt(np.mean(w_n.astype(np.float64) ** 2, axis=0))
    assert np.max(np.abs(col_rms - 1.0)) > 0.05


def test_decode_with_folded_signs_restores_the_matrix():
    B = 64
    m = workloads.channel_spread(128, 192, 51, 52, bf16=True, dead=0.01)
    w_n, su_f, _ = oracle.channel_normalize(m.w, m.su)
    w_reg = oracle.regularize(w_n, m.su, m.sv, B)
    back = oracle.unregularize(w_reg, np.ones(128, np.float32), m.sv, B)
    w_rec = back.astype(np.float64) * su_f.astype(np.float64)[:, None]
    scale = np.max(np.abs(m.w), axis=1, keepdims=True) + 1e-30
    assert np.max(np.abs(w_rec - m.w) / scale) < 2e-6
