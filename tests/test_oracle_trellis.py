"""Pins for the oracle's trellis search that do not reuse its own dynamic program.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture §1
(add-compare-select, two-pass tail-biting closure) and §4 (state algebra);
Test Suite & Verification (ring invariant, shift-register identity, path cost).

* brute force over every path of tiny trellises (Q = 8 state bits): because
  binary32 addition is monotone, the dynamic program's minimum must equal the
  minimum over all paths bit for bit;
* brute force over every circular bit string (tail-biting rings);
* the scalar-quantiser special case, where the answer is per-element nearest level;
* invariants at production size (Q = 16): ring closure and path-cost identity.
"""
import numpy as np
import pytest

import oracle


def _q(xt, v, S):
    d = np.float32(xt) - v[S]
    return d * d


def all_paths(x, v, Q, K):
    """Every path S_0..S_{L-1}; returns (cost, S_0, S_{L/2-1}, S_{L-1})."""
    L = len(x)
    n = 1 << (Q + (L - 1) * K)
    p = np.arange(n, dtype=np.int64)
    S = p >> ((L - 1) * K)
    cost = np.zeros(n, dtype=np.float32) + _q(x[0], v, S)
    S0 = S.copy()
    mid = S.copy() if L // 2 - 1 == 0 else None
    for t in range(1, L):
        b = (p >> ((L - 1 - t) * K)) & ((1 << K) - 1)
        S = ((S << K) | b) & ((1 << Q) - 1)
        cost = cost + _q(x[t], v, S)
        if t == L // 2 - 1:
            mid = S.copy()
    return cost, S0, mid, S


def all_rings(x, v, Q, K):
    """Every circular K-bit symbol string; returns (cost, S_{L-1})."""
    L = len(x)
    assert Q % K == 0
    n = 1 << (L * K)
    r = np.arange(n, dtype=np.int64)
    sym = [(r >> ((L - 1 - t) * K)) & ((1 << K) - 1) for t in range(L)]
    cost = np.zeros(n, dtype=np.float32)
    S = None
    for t in range(L):
        S = np.zeros(n, dtype=np.int64)
        for j in range(Q // K):
            S = (S << K) | sym[(t - (Q // K - 1) + j) % L]
        cost = cost + _q(x[t], v, S)
    return cost, S


def seq_cost(x, v, states):
    c = np.float32(0.0)
    for t in range(len(x)):
        d = np.float32(x[t]) - v[states[t]]
        c = np.float32(c + d * d)
    return c


TINY = [(8, 1, 16), (8, 2, 8)]


def _tiny_inputs(Q, L, seed, kind):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(L).astype(np.float32)
    if kind == "generic":
        v = rng.standard_normal(1 << Q).astype(np.float32)
    else:  # few distinct levels: many exact ties
        v = rng.choice(np.array([-1.0, 0.0, 0.5], np.float32), size=1 << Q)
        x = np.round(x * 2) / 2
        x = x.astype(np.float32)
    return x, v


@pytest.mark.parametrize("Q,K,L", TINY)
@pytest.mark.parametrize("kind", ["generic", "ties"])
def test_forward_min_equals_bruteforce(Q, K, L, kind):
    x, v = _tiny_inputs(Q, L, 10 + Q + K, kind)
    C, _ = oracle.forward(x, Q, K, v, np.zeros(1 << (Q - K), np.float32))
    cost, _, _, S_last = all_paths(x, v, Q, K)
    # unconstrained: min over all paths
    assert C.min() == cost.min()
    # per end state: min over paths ending there
    for s in range(0, 1 << Q, 7):
        assert C[s] == cost[S_last == s].min()


@pytest.mark.parametrize("Q,K,L", TINY)
def test_forward_constrained_start(Q, K, L):
    x, v = _tiny_inputs(Q, L, 3, "generic")
    e0 = 0x15 & ((1 << (Q - K)) - 1)
    M0 = np.full(1 << (Q - K), np.inf, np.float32)
    M0[e0] = 0.0
    C, _ = oracle.forward(x, Q, K, v, M0)
    cost, S0, _, S_last = all_paths(x, v, Q, K)
    ok = (S0 >> K) == e0
    for s in range(0, 1 << Q, 5):
        sel = ok & (S_last == s)
        assert C[s] == cost[sel].min()
    # states that cannot be reached from the admitted start stay at +inf: none
    # here, since L*K >= Q; every state is reachable
    assert np.isfinite(C).all()


@pytest.mark.parametrize("Q,K,L", TINY)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_two_pass_closure_against_rings(Q, K, L, seed):
    x, v = _tiny_inputs(Q, L, 100 + seed, "generic")
    states, X, cost = oracle.encode_sequences(x[None, :], K, v, Q=Q, threads=1)
    states, X, cost = states[0], int(X[0]), cost[0]
    ring_cost, ring_last = all_rings(x, v, Q, K)
    # two-pass result is a ring, so it cannot beat the best ring ...
    assert cost >= ring_cost.min()
    # ... and it is the best ring among those that end in X
    assert cost == ring_cost[ring_last == X].min()
    # the reported cost is the path's own sequential cost
    assert seq_cost(x, v, states) == cost
    # ring closure
    mask = (1 << (Q - K)) - 1
    assert states[-1] == X
    for t in range(1, L):
        assert (states[t] >> K) == (states[t - 1] & mask)
    assert (states[0] >> K) == (states[-1] & mask)


@pytest.mark.parametrize("Q,K,L", TINY)
def test_pass1_end_state_lies_on_an_optimal_rotated_path(Q, K, L):
    x, v = _tiny_inputs(Q, L, 7, "generic")
    _, X, _ = oracle.encode_sequences(x[None, :], K, v, Q=Q, threads=1)
    xr = np.roll(x, -(L // 2))          # x'_j = x_{(j + L/2) mod L}
    cost, _, mid, _ = all_paths(xr, v, Q, K)
    best = cost == cost.min()
    assert int(X[0]) in set(mid[best].tolist())


def _ring_ok(states, K, Q=16):
    mask = (1 << (Q - K)) - 1
    s = np.asarray(states, np.int64)
    ok = np.all((s[:, 1:] >> K) == (s[:, :-1] & mask))
    ok &= np.all((s[:, 0] >> K) == (s[:, -1] & mask))
    return bool(ok)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_production_ring_and_cost_identity(K):
    x = np.random.default_rng(K).standard_normal((3, 256)).astype(np.float32)
    levels = oracle.mul1_levels_fp16()
    v = oracle.scaled_levels(levels, 1.0)
    states, X, cost = oracle.encode_sequences(x, K, v)
    assert _ring_ok(states, K)
    assert np.array_equal(states[:, -1], X)
    sse = oracle.tile_sse(x, states, v)
    assert np.array_equal(sse.view(np.uint32), cost.view(np.uint32))
    for i in range(3):
        assert seq_cost(x[i], v, states[i]) == cost[i]
    words = oracle.pack_states(states, K)
    assert words.shape == (3, 16 * K)
    assert np.array_equal(oracle.unpack_states(words, K), states)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_scalar_quantiser_special_case(K):
    """Levels that depend only on the newest K bits: the trellis is a scalar quantiser."""
    rng = np.random.default_rng(50 + K)
    lev = np.sort(rng.standard_normal(1 << K)).astype(np.float32)
    v = lev[np.arange(1 << 16) & ((1 << K) - 1)]
    x = rng.standard_normal((2, 256)).astype(np.float32)
    states, X, cost = oracle.encode_sequences(x, K, v)
    err = (x[:, :, None] - lev[None, None, :]) ** 2
    want_b = np.argmin(err, axis=2)
    assert np.array_equal(states & ((1 << K) - 1), want_b)
    for i in range(2):
        c = np.float32(0.0)
        for t in range(256):
            d = np.float32(x[i, t] - lev[want_b[i, t]])
            c = np.float32(c + d * d)
        assert c == cost[i]


def test_zero_scale_gives_state_zero():
    """All levels scale to 0: every cost ties, every tie goes to index 0."""
    x = np.random.default_rng(0).standard_normal((1, 256)).astype(np.float32)
    v = np.zeros(1 << 16, np.float32)
    states, X, cost = oracle.encode_sequences(x, 2, v)
    assert not states.any() and X[0] == 0


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.encode_sequences(np.zeros((1, 7), np.float32), 2,
                                np.zeros(1 << 16, np.float32))
