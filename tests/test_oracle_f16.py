"""Pins for the oracle's fp16 mode (the pages' own numeric contract).

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture §1
(exact fp16 add-compare-select: binary16 difference and single-rounded fused
multiply-add into binary16 costs) and §4 (first-branch strict "<" ties).

* the two arithmetic primitives against exact rational arithmetic and a
  brute-force search for the nearest binary16 (ties to even, overflow to inf);
* exhaustive path search on tiny trellises: binary16 rounding is monotone, so
  the dynamic program's minimum equals the minimum over all paths bit for bit;
* the scalar-quantiser special case and the ring invariant at Q = 16.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

_BITS = np.arange(1 << 16, dtype=np.uint16)
_VALS = _BITS.view(np.float16)
_FIN = np.isfinite(_VALS)
_FBITS = _BITS[_FIN]
_FFRAC = [Fraction(float(v)) for v in _VALS[_FIN].astype(np.float64)]
_ORDER = sorted(range(len(_FFRAC)), key=lambda i: (_FFRAC[i], int(_FBITS[i]) >> 15 == 0))
_SORTED = [_FFRAC[i] for i in _ORDER]
_SBITS = [int(_FBITS[i]) for i in _ORDER]
_MAXF = Fraction(65504)
_HALF_ULP_TOP = Fraction(16)          # ulp at the top binade is 32


def nearest_f16(v: Fraction) -> int:
    """Binary16 bits nearest to v, ties to even mantissa, overflow to +-inf."""
    if v >= _MAXF + _HALF_ULP_TOP:
        return 0x7C00
    if v <= -(_MAXF + _HALF_ULP_TOP):
        return 0xFC00
    if v == 0:
        return 0x0000
    import bisect
    i = bisect.bisect_left(_SORTED, v)
    cands = [j for j in (i - 1, i, i + 1) if 0 <= j < len(_SORTED)]
    best = min(abs(_SORTED[j] - v) for j in cands)
    near = [j for j in cands if abs(_SORTED[j] - v) == best]
    bits = sorted({_SBITS[j] for j in near if _SORTED[j] != 0 or True})
    # zero has two encodings; a nonzero v never rounds to zero's sign-opposite
    if len(bits) > 1:
        nonneg = [b for b in bits if (b & 0x3FF) % 2 == 0]
        bits = nonneg or bits
    b = bits[0]
    if _SORTED[near[0]] == 0:
        b = 0x8000 if v < 0 else 0x0000
    return b


def frac16(bits: int) -> Fraction:
    return Fraction(float(np.uint16(bits).view(np.float16)))


def _samples(rng, n):
    # mixture: random finite bit patterns, normal-ish values, tiny values, near-max values
    a = rng.choice(_FBITS, n)
    b = np.float16(rng.standard_normal(n)).view(np.uint16)
    c = np.float16(rng.standard_normal(n) * 1e-6).view(np.uint16)
    d = np.float16(rng.uniform(-65504, 65504, n)).view(np.uint16)
    return np.concatenate([a, b, c, d])


def test_f16_sub_is_the_exactly_rounded_difference():
    rng = np.random.default_rng(1)
    xs, ys = _samples(rng, 600), _samples(rng, 600)
    for x, y in zip(xs.tolist(), ys.tolist()):
        want = nearest_f16(frac16(x) - frac16(y))
        got = oracle.f16_sub(x, y)
        if want == 0 and got in (0, 0x8000):
            continue
        assert got == want, (hex(x), hex(y), hex(got), hex(want))


def test_f16_sqadd_is_one_rounding_of_the_exact_value():
    rng = np.random.default_rng(2)
    ds = _samples(rng, 600)
    ms = np.abs(_samples(rng, 600).view(np.float16)).astype(np.float16).view(np.uint16)
    for d, m in zip(ds.tolist(), ms.tolist()):
        want = nearest_f16(frac16(d) * frac16(d) + frac16(m))
        assert oracle.f16_sqadd(d, m) == want, (hex(d), hex(m))


def test_f16_sqadd_differs_from_two_roundings_somewhere():
    """The fused form is not the two-rounding form: find inputs where they differ."""
    rng = np.random.default_rng(3)
    d = np.float16(rng.standard_normal(4000)).view(np.uint16)
    m = np.float16(np.abs(rng.standard_normal(4000)) * 3).view(np.uint16)
    diff = 0
    for a, b in zip(d.tolist(), m.tolist()):
        sq = nearest_f16(frac16(a) * frac16(a))
        two = nearest_f16(frac16(sq) + frac16(b))
        diff += oracle.f16_sqadd(a, b) != two
    assert diff > 0


def test_f16_special_values():
    inf = 0x7C00
    one = int(np.float16(1.0).view(np.uint16))
    assert oracle.f16_sqadd(one, inf) == inf
    assert oracle.f16_sqadd(int(np.float16(256.0).view(np.uint16)), 0) == inf   # 65536
    big = int(np.float16(255.875).view(np.uint16))                                # ^2 = 65472.016
    assert oracle.f16_sqadd(big, 0) == int(np.float16(65472).view(np.uint16))
    tiny = 0x0001                                                                 # 2^-24
    assert oracle.f16_sqadd(tiny, 0) == 0                                         # 2^-48 -> 0
    assert oracle.f16_sub(tiny, 0) == tiny


def _all_paths_f16(x, c, Q, K, start_e=None):
    """Every path: sequential fused binary16 cost; returns (cost bits, S_0, S_last)."""
    L = len(x)
    n = 1 << (Q + (L - 1) * K)
    p = np.arange(n, dtype=np.int64)
    S = p >> ((L - 1) * K)
    # per (step, state) branch term via the oracle primitives, tabulated
    table = np.zeros((L, 1 << Q), np.uint16)
    for t in range(L):
        for s in range(1 << Q):
            table[t, s] = oracle.f16_sub(int(x[t]), int(c[s]))
    cost = np.array([oracle.f16_sqadd(int(table[0, s]), 0) for s in range(1 << Q)],
                    np.uint16)[S]
    S0 = S.copy()
    sq = {}
    for t in range(1, L):
        b = (p >> ((L - 1 - t) * K)) & ((1 << K) - 1)
        S = ((S << K) | b) & ((1 << Q) - 1)
        d = table[t, S]
        key = d.astype(np.uint32) << 16 | cost.astype(np.uint32)
        uk, inv = np.unique(key, return_inverse=True)
        vals = np.array([sq.setdefault(int(k), oracle.f16_sqadd(int(k >> 16), int(k & 0xFFFF)))
                         for k in uk], np.uint16)
        cost = vals[inv]
    return cost, S0, S


@pytest.mark.parametrize("Q,K,L", [(6, 1, 12), (6, 2, 6)])
def test_f16_forward_min_equals_bruteforce(Q, K, L):
    rng = np.random.default_rng(Q + K)
    x = np.float16(rng.standard_normal(L)).view(np.uint16)
    c = np.float16(rng.standard_normal(1 << Q)).view(np.uint16)
    C, _ = oracle.forward_f16(x, Q, K, c, np.zeros(1 << (Q - K), np.uint16))
    cost, S0, S_last = _all_paths_f16(x, c, Q, K)
    for s in range(1 << Q):
        sel = cost[S_last == s]
        assert C[s] == sel.min()            # binary16 bits of non-negatives order as integers


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_f16_scalar_quantiser_case(K):
    """A codebook that depends only on the low K bits makes every step's choice free.

    Binary16 rounding is monotone in both operands of the fused update, so the path that
    takes the nearest level at every step (exact arithmetic) reaches the least accumulated
    cost of all paths: the unconstrained forward pass must find exactly that minimum.  The
    two-pass encode may do worse (its closure fixes the last steps from pass 1's path, and
    where rounding absorbed a difference pass 1's tie rule can pick a level that pass 2 then
    pays for), never better, and its reported cost is its own path's accumulated cost."""
    rng = np.random.default_rng(10 + K)
    lev = np.sort(rng.standard_normal(1 << K)).astype(np.float16)
    lbits = lev.view(np.uint16)
    c = lbits[np.arange(1 << 16) & ((1 << K) - 1)]
    x = np.float16(rng.standard_normal((1, 256))).view(np.uint16)
    xf = x.view(np.float16).astype(np.float64)[0]
    greedy = np.argmin((xf[:, None] - lev.astype(np.float64)[None, :]) ** 2, axis=1)

    def accumulate(choice):
        acc = 0
        for t in range(256):
            acc = oracle.f16_sqadd(oracle.f16_sub(int(x[0, t]), int(lbits[choice[t]])), acc)
        return acc

    best = accumulate(greedy)
    C, _ = oracle.forward_f16(x[0], 16, K, c, np.zeros(1 << (16 - K), np.uint16))
    assert int(C.min()) == best
    states, X, cost = oracle.encode_sequences_f16(x, K, c)
    assert accumulate(states[0] & ((1 << K) - 1)) == int(cost[0])
    assert int(cost[0]) >= best


@pytest.mark.parametrize("K", [1, 2, 4])
def test_f16_ring_and_cost(K):
    x = np.float16(np.random.default_rng(K).standard_normal((2, 256))).view(np.uint16)
    r = oracle.encode_tiles_f16(x, K)
    s = r["states"].astype(np.int64)
    mask = (1 << (16 - K)) - 1
    assert np.all((s[:, 1:] >> K) == (s[:, :-1] & mask))
    assert np.all((s[:, 0] >> K) == (s[:, -1] & mask))
    assert np.array_equal(s[:, -1], r["X"])
    c = oracle.mul1_levels_fp16().view(np.uint16)
    for i in range(2):
        acc = 0
        for t in range(256):
            acc = oracle.f16_sqadd(oracle.f16_sub(int(x[i, t]), int(c[s[i, t]])), acc)
        assert acc == r["cost"][i]
    assert np.array_equal(oracle.unpack_states(r["packed"], K), r["states"])
