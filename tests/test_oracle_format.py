"""Pins for the oracle's container, tile layout and statistics.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture §5
(MSB-first packing of the low K bits of each state, SWAP16 half-word swap,
decode of the state history) and §11 (int16 [k/16, n/16, 16*K] container);
§8 (per-tile energy used by the scale search).
"""
import math

import numpy as np
import pytest

import oracle


def pack_by_strings(b, K):
    """Independent packer: build the bit string as text, cut 16-bit words, swap pairs."""
    s = "".join(format(int(bt), "0%db" % K) for bt in b)
    words = [int(s[i:i + 16], 2) for i in range(0, len(s), 16)]
    for i in range(0, len(words), 2):
        words[i], words[i + 1] = words[i + 1], words[i]
    return np.array(words, dtype=np.uint16)


def random_ring(rng, K, L=256, Q=16):
    b = rng.integers(0, 1 << K, L)
    states = np.zeros(L, np.int64)
    for t in range(L):
        s = 0
        for j in range(-(Q // K) - 1, 1):          # enough symbols to fill Q bits
            s = ((s << K) | int(b[(t + j) % L])) & ((1 << Q) - 1)
        states[t] = s
    return b, states


@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 6, 8])
def test_pack_matches_string_packer(K):
    rng = np.random.default_rng(K)
    b, states = random_ring(rng, K)
    got = oracle.pack_states(states[None, :], K)[0]
    assert np.array_equal(got, pack_by_strings(b, K))
    assert np.array_equal(oracle.unpack_states(got[None, :], K)[0], states)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_pack_closed_forms(K):
    ones = np.full((1, 256), 0xFFFF, np.int64)
    assert np.all(oracle.pack_states(ones, K) == 0xFFFF)
    first = np.zeros((1, 256), np.int64)
    first[0, 0] = 1                       # b_0 = 1: stream bit K-1 is the only one set
    w = oracle.pack_states(first, K)[0]
    want = np.zeros(16 * K, np.uint16)
    want[1] = 1 << (16 - K)               # word 0 before the swap
    assert np.array_equal(w, want)
    last = np.zeros((1, 256), np.int64)
    last[0, 255] = 1                      # last stream bit: bit 0 of the last word
    w = oracle.pack_states(last, K)[0]
    want = np.zeros(16 * K, np.uint16)
    want[16 * K - 2] = 1
    assert np.array_equal(w, want)


def test_tile_layout_by_loops():
    R, C = 32, 48
    m = np.arange(R * C, dtype=np.float32).reshape(R, C)
    t = oracle.to_tiles(m)
    TC = C // 16
    for tau in range(t.shape[0]):
        tr, tc = divmod(tau, TC)
        for e in (0, 1, 15, 16, 17, 255):
            r, c = divmod(e, 16)
            assert t[tau, e] == m[16 * tr + r, 16 * tc + c]
    assert np.array_equal(oracle.from_tiles(t, R, C), m)


def test_tile_sumsq_closed_forms_and_bound():
    tiles = np.stack([np.ones(256, np.float32), np.full(256, 0.5, np.float32),
                      np.zeros(256, np.float32)])
    assert oracle.tile_sumsq(tiles).tolist() == [256.0, 64.0, 0.0]
    x = np.random.default_rng(0).standard_normal((4, 256)).astype(np.float32)
    got = oracle.tile_sumsq(x)
    for i in range(4):
        exact = math.fsum(float(a) * float(a) for a in x[i])
        # sequential binary32 sum: relative error below about n * 2^-24
        assert abs(float(got[i]) - exact) <= exact * 300 * 2.0 ** -24
    assert oracle.matrix_rms(np.array([256.0] * 4, np.float32), 1024) == 1.0


def test_sample_tiles_by_hand():
    # 2 x 3 tile grid: diagonal i < 3 -> (0,0), (1,1), (0,2) -> 0, 4, 2
    q = np.array([5, 1, 3, 9, 2, 9], np.float32)   # max at 3 (first of ties), min at 1
    assert oracle.sample_tiles(2, 3, q) == [0, 1, 2, 3, 4]
    # 3 x 2 grid: (0,0), (1,1), (2,0) -> 0, 3, 4
    q = np.array([1, 1, 1, 1, 1, 1], np.float32)   # all equal: max and min both 0
    assert oracle.sample_tiles(3, 2, q) == [0, 3, 4]
    # 256 x 256 grid (4096^2): diagonal only + 2 extremes -> at most 258
    q = np.ones(256 * 256, dtype=np.float32)
    q[1], q[2] = 10.0, 0.5                          # extremes off the diagonal
    s = oracle.sample_tiles(256, 256, q)
    assert len(s) == 258 and s[:4] == [0, 1, 2, 257] and s[-1] == 256 * 256 - 1
