"""Pins for the oracle's LDLQ error-feedback loop.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 3
(one-sided block LDLQ: bottom-up span traversal, additive target correction from
the strictly lower L blocks, trailing-span residual feedback).

* identity factor: no feedback, so the loop must equal independent tile encoding;
* the target correction against the dense product in binary64, within the
  rounding bound of a sequential binary32 sum;
* the LDLQ residual identity  tr(E H E^T) = sum_j tr((T_j - What_j) D_j (T_j - What_j)^T)
  for H = L D L^T, which fails for a transposed factor, a wrong traversal order or
  feedback of the target instead of the weight;
* on a strongly correlated Hessian the proxy loss falls below independent encoding's.
"""
import numpy as np
import pytest

import oracle
import workloads


def _w(R, C, seed):
    return (np.random.default_rng(seed).standard_normal((R, C)) * 0.02).astype(np.float32)


def _scale(K):
    # a fixed scale near the optimum for N(0, 0.02^2) entries
    return np.float32({1: 0.022, 2: 0.017, 3: 0.014, 4: 0.012}[K])


def _proxy(E, H):
    E = E.astype(np.float64)
    return float(np.trace(E @ H @ E.T))


@pytest.mark.parametrize("K", [2, 3])
def test_identity_factor_is_independent_encoding(K):
    R, C = 48, 64
    W = _w(R, C, 1)
    L = np.eye(C, dtype=np.float32)
    out = oracle.ldlq(W, L, K, _scale(K))
    ref = oracle.encode_tiles(oracle.to_tiles(W), K, _scale(K))
    assert np.array_equal(out["states"], ref["states"])
    assert np.array_equal(out["packed"], ref["packed"])
    assert np.array_equal(out["targets"], W)
    assert np.array_equal(out["err"].view(np.uint32), ref["sse"].view(np.uint32))


def test_target_correction_matches_dense_product():
    R, C, K = 32, 96, 2
    W = _w(R, C, 2)
    L, _ = workloads.ldl_factor(C, 7, off_std=2.0)
    out = oracle.ldlq(W, L, K, _scale(K))
    E = (W - out["what"]).astype(np.float64)
    L64 = L.astype(np.float64)
    u = 2.0 ** -24
    for j in range(C // 16):
        cj = slice(16 * j, 16 * j + 16)
        rest = slice(16 * (j + 1), C)
        exact = W[:, cj].astype(np.float64) + E[:, rest] @ L64[rest, cj]
        n = C - 16 * (j + 1)
        mag = np.abs(W[:, cj]).astype(np.float64) + np.abs(E[:, rest]) @ np.abs(L64[rest, cj])
        bound = 2.0 * (n + 1) * u * mag + 1e-30
        assert np.all(np.abs(out["targets"][:, cj] - exact) <= bound), j
    # a transposed factor gives a different correction
    outT = oracle.ldlq(W, np.ascontiguousarray(L.T), K, _scale(K))
    assert not np.array_equal(outT["targets"], out["targets"])


@pytest.mark.parametrize("K", [1, 2, 4])
def test_ldlq_residual_identity(K):
    R, C = 32, 80
    W = _w(R, C, 3 + K)
    L, D = workloads.ldl_factor(C, 11 + K, off_std=1.5)
    out = oracle.ldlq(W, L, K, _scale(K))
    L64 = L.astype(np.float64)
    Dfull = np.zeros((C, C))
    for j in range(C // 16):
        Dfull[16 * j:16 * j + 16, 16 * j:16 * j + 16] = D[j]
    H = L64 @ Dfull @ L64.T
    lhs = _proxy(W - out["what"], H)
    rhs = 0.0
    for j in range(C // 16):
        cj = slice(16 * j, 16 * j + 16)
        Rj = out["targets"][:, cj].astype(np.float64) - out["what"][:, cj]
        rhs += float(np.trace(Rj @ D[j] @ Rj.T))
    assert abs(lhs - rhs) <= 1e-4 * rhs


def _block_ldl(H):
    """Block LDL of an SPD matrix through its Cholesky factor (test helper, binary64)."""
    C = H.shape[0]
    Lc = np.linalg.cholesky(H)
    L = np.zeros_like(H)
    D = []
    for j in range(C // 16):
        cj = slice(16 * j, 16 * j + 16)
        B = Lc[cj, cj]
        L[:, cj] = Lc[:, cj] @ np.linalg.inv(B)
        D.append(B @ B.T)
    return L, np.stack(D)


def test_feedback_lowers_proxy_loss_on_correlated_hessian():
    R, C, K = 64, 128, 2
    rng = np.random.default_rng(5)
    # activations with strongly correlated neighbouring features (AR(1), rho = 0.95)
    n = 4096
    X = np.empty((n, C))
    X[:, 0] = rng.standard_normal(n)
    for c in range(1, C):
        X[:, c] = 0.95 * X[:, c - 1] + np.sqrt(1 - 0.95 ** 2) * rng.standard_normal(n)
    H = X.T @ X / n + 1e-3 * np.eye(C)
    L, D = _block_ldl(H)
    Dfull = np.zeros((C, C))
    for j in range(C // 16):
        Dfull[16 * j:16 * j + 16, 16 * j:16 * j + 16] = D[j]
    assert np.allclose(L @ Dfull @ L.T, H)               # the factorisation is exact
    W = _w(R, C, 6)
    out = oracle.ldlq(W, L.astype(np.float32), K, _scale(K))
    ref = oracle.encode_tiles(oracle.to_tiles(W), K, _scale(K))
    v = oracle.scaled_levels(oracle.mul1_levels_fp16(), _scale(K))
    what_ind = oracle.from_tiles(v[ref["states"]], R, C)
    with_fb = _proxy(W - out["what"], H)
    without = _proxy(W - what_ind, H)
    assert with_fb < 0.8 * without


def test_rows_are_independent():
    # the band property the full-size GPU check relies on: LDLQ on a subset of
    # whole tile rows reproduces those rows of the full run, bit for bit
    W = _w(96, 64, 31)
    L, _ = workloads.ldl_factor(64, 32, off_std=1.5)
    full = oracle.ldlq(W, L, 2, _scale(2))
    tile_rows = [1, 4]
    rows = np.concatenate([np.arange(16 * t, 16 * t + 16) for t in tile_rows])
    band = oracle.ldlq(W[rows], L, 2, _scale(2))
    TC = 64 // 16
    pk = full["packed"].reshape(6, TC, -1)[tile_rows].reshape(-1, full["packed"].shape[1])
    assert np.array_equal(band["packed"], pk)
    assert np.array_equal(band["what"], full["what"][rows])
    assert np.array_equal(band["err"].view(np.uint32),
                          full["err"].reshape(6, TC)[tile_rows].reshape(-1).view(np.uint32))
