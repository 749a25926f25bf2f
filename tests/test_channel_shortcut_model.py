"""The exact block shortcut of the out-channel normalization kernel, modelled on the CPU.

The kernel (csrc/channel.hip) must reproduce the sequential binary64 row sums
of the squares ("EXL3 Intel Arc Quantizer" README, Core Implemented
Architecture item 8, read as sums in column order).  It adds a group of eight
16-byte blocks at once when a test proves that no addition of the group
rounds, and otherwise block by block, failing blocks one square at a time.
This test runs the same decisions in Python (same bounds, same groups, the
group's squares summed in a different order than the kernel's, which the
argument allows) against the plain sequential sum, on rows built to round:
values spread over 190 binades, subnormals, tiny values among large ones,
zeros, infinities and NaNs, bf16 (8 values per block) and fp32 (4 per block).
The GPU tests check the kernel itself bit for bit against the oracle.
"""
import math
import random
import struct

import pytest

BIG = 1 << 20


def _f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _bf16(x):
    b = struct.unpack("<I", struct.pack("<f", x))[0] & 0xFFFF0000
    return struct.unpack("<f", struct.pack("<I", b))[0]


def _exp_bound(x, sig):
    """Lower bound on the exponent of the lowest set bit of a binary32 value from its
    exponent field alone; BIG for zero, -BIG for NaN / infinity."""
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    e = (b >> 23) & 0xFF
    if e == 0xFF:
        return -BIG
    if b & 0x7FFFFFFF == 0:
        return BIG
    return max(e, 1) - 127 - (sig - 1)


def _bound(m):
    return math.inf if m == BIG else 0.0 if m == -BIG else math.ldexp(1.0, 53 + 2 * m)


def _next_binade(a):
    if math.isinf(a):
        return math.inf
    return math.ldexp(1.0, math.frexp(a)[1])


def _shortcut_sum(vals, epb, sig, group=8):
    nb = len(vals) // epb
    blocks = [vals[i * epb:(i + 1) * epb] for i in range(nb)]
    S = []
    for blk in blocks:
        sq = [v * v for v in blk]
        while len(sq) > 1:                       # a tree, as the kernel's loaders sum
            sq = [sq[i] + sq[i + 1] for i in range(0, len(sq), 2)]
        S.append(sq[0])
    T = [_bound(min(_exp_bound(v, sig) for v in blk)) for blk in blocks]
    acc, gb, failed = 0.0, math.inf, 0
    for g0 in range(0, nb, group):
        idx = range(g0, min(nb, g0 + group))
        gs = [S[i] for i in idx]
        while len(gs) > 1:                       # the group's sums, again in a tree
            gs = [gs[i] + (gs[i + 1] if i + 1 < len(gs) else 0.0) for i in range(0, len(gs), 2)]
        a = acc + gs[0]
        tg = min(T[i] for i in idx)
        if a < gb and a < tg:
            acc, gb = a, min(gb, tg)
            continue
        failed += 1
        x, g = acc, gb
        for i in idx:
            A = x + S[i]
            g = min(g, T[i])
            if A < g:
                x = A
            else:
                for v in blocks[i]:
                    x = x + v * v
                g = _next_binade(x) if x > 0.0 else g
        acc, gb = x, g
    return acc, failed


def _sequential(vals):
    acc = 0.0
    for v in vals:
        acc = acc + v * v
    return acc


def _row(rng, n, kind, bf16):
    out = []
    for _ in range(n):
        if kind == 0:
            x = rng.gauss(0, 0.02)
        elif kind == 1:
            x = rng.choice([-1, 1]) * 2.0 ** rng.uniform(-149, 40)
        elif kind == 2:
            x = rng.choice([0.0, 0.0, rng.gauss(0, 1e-40), rng.gauss(0, 1)])
        elif kind == 3:
            x = rng.gauss(0, 1) if rng.random() < 0.97 else rng.gauss(0, 1) * 2.0 ** -35
        elif kind == 4:
            x = rng.choice([1.0, 3.0, 2.0 ** 26 + 1, 2.0 ** -30, 0.0])
        else:
            x = (rng.choice([math.inf, -math.inf, math.nan]) if rng.random() < 0.03
                 else rng.gauss(0, 1))
        if math.isfinite(x):
            x = _bf16(x) if bf16 else _f32(x)
        out.append(x)
    return out


@pytest.mark.parametrize("bf16", [True, False])
def test_shortcut_matches_the_sequential_sum(bf16):
    rng = random.Random(17 if bf16 else 19)
    epb, sig = (8, 8) if bf16 else (4, 24)
    failed = 0
    for trial in range(300):
        vals = _row(rng, epb * rng.randint(1, 80), trial % 6, bf16)
        got, f = _shortcut_sum(vals, epb, sig)
        want = _sequential(vals)
        assert got == want or (math.isnan(got) and math.isnan(want)), (trial, got, want)
        failed += f
    assert failed > 0                           # the block-by-block path ran


def test_gaussian_rows_mostly_take_the_shortcut():
    rng = random.Random(23)
    groups = failed = 0
    for _ in range(8):
        vals = [_bf16(rng.gauss(0, 0.02)) for _ in range(4096)]
        got, f = _shortcut_sum(vals, 8, 8)
        assert got == _sequential(vals)
        groups += 64
        failed += f
    assert failed < 0.05 * groups
