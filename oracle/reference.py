"""Reference implementation of the EXL3 trellis tile encoder -- TEST INFRASTRUCTURE ONLY.

This module is the oracle.  Only the test-suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import it.  It shares no code with the
GPU library: it has its own codebook generator, its own Hadamard transform, its
own packer and its own scale search.  It is plain and slow on purpose, so that
each step can be checked by eye against the sources:

  [P1] "EXL3 Intel Arc Quantizer" (project README), section "Core Implemented
       Architecture" -- item 1 (SYCL XPU tile encoder: add-compare-select,
       two-pass tail-biting closure), item 4 (CPU reference encoder: state
       algebra), item 5 (format primitives: mul1 codebook, MSB-first container,
       SWAP16), item 7 (Sylvester Hadamard, blockwise, decode order), item 8
       (regularization, wrapped-diagonal tile sample for the scale search);
       section "Test Suite & Verification" (ring invariant, shift-register
       identity, round trips).
  [P2] "JEV-9B EXL3 K=2 (mul1) Checkpoint for Intel Arc XPU" (model card),
       section 2 "Quantization & Bitrate Breakdown" (golden-section scale
       search) and section 3 "Verification & Metrics" (distortion band).

Readings taken where the sources leave a step open (each is listed in the
design notes with its reason):

  * numerics: binary32, each subtract / multiply / add rounded on its own, no
    fused multiply-add, lowest index on equal costs; host control in binary64;
  * mul1 levels: the sources give only the name, the count of distinct levels
    and their range.  This oracle uses a multiply-then-byte-sum construction:
    h = (A * s) mod 2^32 for an odd constant A chosen here, beta = the sum of
    the four bytes of h, level = fp16 round-to-nearest-even of
    (beta - mean) / std over all 2^16 states (computed with exact integers and
    two correctly rounded binary64 operations).  Compatibility with upstream
    levels is NOT claimed (parity unpinned against upstream);
  * search domain: the tile input is compared with v = rn(scale * level);
  * regularization: signs, then blockwise left FWHT, x rn(1/sqrt(B)), then
    blockwise right FWHT, x rn(1/sqrt(B)); natural Sylvester order;
  * tile geometry: row-major tile grid, row-major 16x16 inside a tile (the
    tensor-core permutation is not reproduced);
  * statistics: sequential binary32 sum of squares per tile, binary64 sum over
    tiles in ascending order;
  * scale search: textbook golden section over [lo, hi] * rms with 2 initial
    probes and `iters` reductions, strict "<" keeps the left part, result is the
    midpoint of the final bracket rounded to binary32;
  * scale-search tile set: the wrapped diagonal plus the tiles with the largest
    and the smallest sum of squares (lowest index on ties), ascending order.
"""
from __future__ import annotations

import ctypes
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

# --------------------------------------------------------------------------
# C core (forward dynamic program and two-pass closure)
# --------------------------------------------------------------------------
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
        u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
        lib.oracle_forward.argtypes = [f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       f32p, f32p, f32p, u8p]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_encode_many.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, f32p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_encode_many.restype = ctypes.c_int
        u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
        lib.oracle_f16_sub.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        lib.oracle_f16_sub.restype = ctypes.c_uint16
        lib.oracle_f16_sqadd.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        lib.oracle_f16_sqadd.restype = ctypes.c_uint16
        lib.oracle_forward_f16.argtypes = [u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           u16p, u16p, u16p, u8p]
        lib.oracle_forward_f16.restype = ctypes.c_int
        lib.oracle_encode_many_f16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, u16p,
                                               ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p]
        lib.oracle_encode_many_f16.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    # at most 16 worker threads (the host share of one GPU on the target boxes)
    return max(1, min(os.cpu_count() or 1, 16))


# --------------------------------------------------------------------------
# Codebook  [P1 item 5]
# --------------------------------------------------------------------------
MUL1_MULTIPLIER = 0x9E3779B1   # odd 32-bit constant chosen here (golden-ratio hash)
STATE_BITS = 16


def mul1_levels_fp16() -> np.ndarray:
    """fp16 level of each of the 2^16 states (the reading described in the header)."""
    n = 1 << STATE_BITS
    s = np.arange(n, dtype=np.uint64)
    h = (s * np.uint64(MUL1_MULTIPLIER)) & np.uint64(0xFFFFFFFF)
    beta = np.zeros(n, dtype=np.int64)
    for byte in range(4):
        beta += ((h >> np.uint64(8 * byte)) & np.uint64(0xFF)).astype(np.int64)
    s1 = int(beta.sum())
    s2 = int((beta * beta).sum())
    # (beta - s1/n) / (sqrt(n*s2 - s1^2)/n) == (n*beta - s1) / sqrt(n*s2 - s1^2)
    numer = (n * beta - s1).astype(np.float64)          # exact integers
    denom = math.sqrt(float(n * s2 - s1 * s1))          # exact integer, one rounding
    z = numer / denom                                   # one rounding per state
    return z.astype(np.float16)                         # round-to-nearest-even


# The two other procedural codebooks (README item 5 names them and prints their
# counts of distinct levels, 10,746 and 10,598).  Both map a state to a 32-bit
# word, keep the sign bit and 12 low bits of each 16-bit half and xor in a
# fixed pattern, which puts each half's exponent field in 12..15, so each half
# is a binary16 number of magnitude in [1/8, 2); the level is the binary16 sum
# of the two halves.  3INST is the published three-instruction decoder of the
# QTIP trellis codes (a 32-bit linear congruential step, the mask, the xor);
# mcg replaces the congruential step by a multiplicative one.  The pages give
# no multiplier: this reading takes the first odd multiplier at or above the
# golden-ratio constant 0x9E3779B1 (MUL1_MULTIPLIER) whose table has exactly
# the printed 10,746 distinct levels (mcg_multiplier_scan repeats the search).
INST3_A, INST3_B = 89226354, 64248484
MCG_SCAN_START = 0x9E3779B1
MCG_MULTIPLIER = 0x9E378FED
HALVES_MASK, HALVES_XOR = 0x8FFF8FFF, 0x3B603B60


def _halves_sum_fp16(words: np.ndarray) -> np.ndarray:
    m = (words & np.uint64(HALVES_MASK)) ^ np.uint64(HALVES_XOR)
    lo = (m & np.uint64(0xFFFF)).astype(np.uint16).view(np.float16).astype(np.float64)
    hi = (m >> np.uint64(16)).astype(np.uint16).view(np.float16).astype(np.float64)
    return (lo + hi).astype(np.float16)        # exact binary64 sum, one RNE rounding


def inst3_levels_fp16() -> np.ndarray:
    s = np.arange(1 << STATE_BITS, dtype=np.uint64)
    return _halves_sum_fp16((s * np.uint64(INST3_A) + np.uint64(INST3_B)) & np.uint64(0xFFFFFFFF))


def mcg_multiplier_scan(target=10746, start=MCG_SCAN_START, limit=1 << 16):
    """First odd multiplier a >= start (scanning a, a + 2, ...) whose halves
    table has `target` distinct levels, and the number of odd values scanned."""
    s = np.arange(1 << STATE_BITS, dtype=np.uint64)
    a = start | 1
    for i in range(limit):
        words = (s * np.uint64(a)) & np.uint64(0xFFFFFFFF)
        if len(np.unique(_halves_sum_fp16(words))) == target:
            return a, i + 1
        a += 2
    raise ValueError("no multiplier within %d odd values" % limit)


def mcg_levels_fp16() -> np.ndarray:
    s = np.arange(1 << STATE_BITS, dtype=np.uint64)
    return _halves_sum_fp16((s * np.uint64(MCG_MULTIPLIER)) & np.uint64(0xFFFFFFFF))


CODEBOOKS = {"mul1": mul1_levels_fp16, "mcg": mcg_levels_fp16, "3inst": inst3_levels_fp16}


def scaled_levels(levels_fp16: np.ndarray, scale) -> np.ndarray:
    """v[s] = rn(scale * level[s]) in binary32."""
    return (np.float32(scale) * levels_fp16.astype(np.float32)).astype(np.float32)


# --------------------------------------------------------------------------
# Trellis search  [P1 items 1 and 4]
# --------------------------------------------------------------------------
def forward(x, Q, K, v, M0):
    """One forward pass; returns (final-step costs C[2^Q], predecessors [L-1, 2^(Q-K)])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    M0 = np.ascontiguousarray(M0, dtype=np.float32)
    L = x.shape[0]
    C = np.empty(1 << Q, dtype=np.float32)
    bp = np.empty(((L - 1), 1 << (Q - K)), dtype=np.uint8)
    rc = _load().oracle_forward(x, L, Q, K, v, M0, C, bp)
    if rc != 0:
        raise ValueError("oracle_forward rejected its arguments (rc=%d)" % rc)
    return C, bp


def encode_sequences(x, K, v, Q=STATE_BITS, threads=None):
    """Two-pass tail-biting encode of each row of x [n, L].

    Returns (states int32 [n, L], X int32 [n], cost float32 [n]); cost is the
    pass-2 cost of X at the last step.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be [n, L]")
    n, L = x.shape
    states = np.empty((n, L), dtype=np.int32)
    X = np.empty(n, dtype=np.int32)
    cost = np.empty(n, dtype=np.float32)
    if n == 0:
        return states, X, cost
    lib = _load()
    threads = threads or default_threads()
    chunks = np.array_split(np.arange(n), min(threads, n))

    def run(idx):
        if idx.size == 0:
            return 0
        i0 = int(idx[0])
        m = int(idx.size)
        return lib.oracle_encode_many(
            x[i0:].ctypes.data, m, L, Q, K, v,
            states[i0:].ctypes.data, X[i0:].ctypes.data, cost[i0:].ctypes.data)

    if len(chunks) == 1:
        rcs = [run(chunks[0])]
    else:
        with ThreadPoolExecutor(max_workers=len(chunks)) as ex:
            rcs = list(ex.map(run, chunks))
    if any(rc != 0 for rc in rcs):
        raise ValueError("oracle_encode_many rejected its arguments (rc=%s)" % rcs)
    return states, X, cost


def tile_sse(x, states, v):
    """Sequential binary32 sum over t of rn(rn(x_t - v[S_t])^2), from +0."""
    x = np.asarray(x, dtype=np.float32)
    what = v[states]
    acc = np.zeros(x.shape[0], dtype=np.float32)
    for t in range(x.shape[1]):
        d = x[:, t] - what[:, t]
        acc = acc + d * d
    return acc


# --------------------------------------------------------------------------
# Container  [P1 item 5: MSB-first packing of the low K bits, SWAP16]
# --------------------------------------------------------------------------
def pack_states(states, K):
    """[n, 256] states -> [n, 16*K] uint16 words (MSB-first stream, then SWAP16)."""
    states = np.asarray(states, dtype=np.int64)
    n, L = states.shape
    if n == 0:
        return np.zeros((0, (L * K) // 16), np.uint16)
    b = states & ((1 << K) - 1)
    # stream bit j = bit (K-1-(j mod K)) of b_(j div K)
    shifts = np.arange(K - 1, -1, -1)
    bits = (b[:, :, None] >> shifts[None, None, :]) & 1          # [n, L, K]
    bits = bits.reshape(n, (L * K) // 16, 16)
    weights = (1 << np.arange(15, -1, -1)).astype(np.int64)
    words = (bits * weights).sum(axis=2)                          # stream bit 16w -> bit 15
    swapped = words.reshape(n, -1, 2)[:, :, ::-1].reshape(n, -1)  # words 2i <-> 2i+1
    return swapped.astype(np.uint16)


def unpack_states(words, K, L=256):
    """Inverse view: S_t = the 16-bit window of the circular stream ending at bit (t+1)K-1."""
    words = np.asarray(words, dtype=np.int64)
    n = words.shape[0]
    w = words.reshape(n, -1, 2)[:, :, ::-1].reshape(n, -1)        # undo SWAP16
    bits = (w[:, :, None] >> np.arange(15, -1, -1)[None, None, :]) & 1
    stream = bits.reshape(n, -1)                                  # [n, L*K]
    nbits = L * K
    out = np.zeros((n, L), dtype=np.int64)
    for t in range(L):
        end = (t + 1) * K                                         # exclusive
        idx = np.arange(end - 16, end) % nbits
        val = np.zeros(n, dtype=np.int64)
        for j in idx:
            val = (val << 1) | stream[:, j]
        out[:, t] = val
    return out.astype(np.int32)


# --------------------------------------------------------------------------
# Regularization  [P1 items 7 and 8]
# --------------------------------------------------------------------------
def hadamard_norm(B: int) -> np.float32:
    """Binary32 normalisation constant 1/sqrt(B) for the supported block sizes."""
    if B == 64:
        return np.float32(0.125)
    if B == 128:
        return np.frombuffer(np.uint32(0x3DB504F3).tobytes(), dtype=np.float32)[0]
    raise ValueError("Hadamard block must be 64 or 128")


def fwht_rows_blockwise(a, B):
    """In-place-order fast Walsh-Hadamard transform along axis 0, in blocks of B rows.

    Levels h = 1, 2, 4, ..., B/2; at each level every pair (p, p+h) with
    p mod 2h < h becomes (a+b, a-b), each rounded to binary32.
    """
    a = np.asarray(a, dtype=np.float32)
    R, C = a.shape
    if R % B:
        raise ValueError("rows not a multiple of the block")
    y = a.reshape(R // B, B, C).copy()
    h = 1
    while h < B:
        y = y.reshape(R // B, B // (2 * h), 2, h, C)
        top = y[:, :, 0]
        bot = y[:, :, 1]
        s = top + bot
        d = top - bot
        y = np.stack([s, d], axis=2)
        h *= 2
    return y.reshape(R, C)


def regularize(w, su, sv, B):
    """W_reg = H_l diag(su) W diag(sv) H_r, evaluated in the fixed order of the header."""
    w = np.asarray(w, dtype=np.float32)
    su = np.asarray(su, dtype=np.float32)
    sv = np.asarray(sv, dtype=np.float32)
    c = hadamard_norm(B)
    y = (w * su[:, None]) * sv[None, :]             # exact: sign flips
    y = fwht_rows_blockwise(y, B) * c               # left side, then normalise
    y = fwht_rows_blockwise(y.T, B).T * c           # right side, then normalise
    return np.ascontiguousarray(y, dtype=np.float32)


def unregularize(w_reg, su, sv, B):
    """Inverse of regularize (H is its own inverse); validation only."""
    c = hadamard_norm(B)
    y = fwht_rows_blockwise(np.asarray(w_reg, np.float32), B) * c
    y = fwht_rows_blockwise(y.T, B).T * c
    return (y * np.asarray(su, np.float32)[:, None]) * np.asarray(sv, np.float32)[None, :]


CHANNEL_FLOOR = 0.1


def channel_normalize(w, su, floor=CHANNEL_FLOOR):
    """Out-channel RMS normalization with the scale folded into the sign vector.

    [P1 item 8: out-channel RMS normalization, sign + scale folding, the
    zero-channel floor and the zero-sign rule.]  The output channels are the
    rows of W (the LDLQ factor acts on the columns, the input side), so the
    scale folds into su.  Per row i, in this order:
      r_i  = sqrt(sum_j (double)w_ij^2 / C), j ascending, binary64;
      r_i  = floor if r_i == 0 (an all-zero channel), and su'_i = 0;
      f_i  = (float)(1.0 / r_i)              (binary64 divide, one rounding);
      w'_ij = rn32(w_ij * f_i);  su'_i = su_i * (float)r_i.
    Regularizing W' with the +-1 su and decoding with su' gives back W up to
    the roundings of f_i, w' and (float)r_i.  Returns (w', su', r) with r the
    binary64 rms before the floor.
    """
    w = np.asarray(w, dtype=np.float32)
    su = np.asarray(su, dtype=np.float32)
    R, C = w.shape
    r = np.empty(R, dtype=np.float64)
    for i in range(R):
        acc = 0.0
        for val in w[i].tolist():
            acc += val * val                 # binary64; the square of a binary32 is exact
        r[i] = math.sqrt(acc / C)
    r_eff = np.where(r == 0.0, float(floor), r)
    f = np.array([np.float32(1.0 / x) for x in r_eff.tolist()], dtype=np.float32)
    w_n = (w * f[:, None]).astype(np.float32)
    su_f = np.where(r == 0.0, np.float32(0.0), su * r.astype(np.float32)).astype(np.float32)
    return np.ascontiguousarray(w_n), su_f, r


def check_order(order):
    """A within-tile order: trellis position t of a tile holds the tile's element
    order[t] (element 16*r + c).  The pages name a fixed 256-entry permutation
    for tensor-core decoding without printing it (README, Format Primitives);
    None is the natural row-major order."""
    if order is None:
        return None
    o = np.asarray(order, dtype=np.int64)
    if o.shape != (256,) or not np.array_equal(np.sort(o), np.arange(256)):
        raise ValueError("a within-tile order is a permutation of 0..255")
    return o


def to_tiles(m, order=None):
    """[R, C] -> [R/16 * C/16, 256]; tile tr*TC + tc; position t holds element
    16*r + c = order[t] (t itself without an order)."""
    R, C = m.shape
    t = m.reshape(R // 16, 16, C // 16, 16).transpose(0, 2, 1, 3).reshape(-1, 256)
    o = check_order(order)
    return np.ascontiguousarray(t if o is None else t[:, o])


def from_tiles(tiles, R, C, order=None):
    t = np.asarray(tiles).reshape(-1, 256)
    o = check_order(order)
    if o is not None:
        rm = np.empty_like(t)
        rm[:, o] = t
        t = rm
    return np.ascontiguousarray(
        t.reshape(R // 16, C // 16, 16, 16).transpose(0, 2, 1, 3).reshape(R, C))


# --------------------------------------------------------------------------
# Statistics, tile sample and scale search  [P1 item 8; P2 section 2]
# --------------------------------------------------------------------------
def tile_sumsq(tiles):
    """Sequential binary32 sum over t of rn(w_t * w_t), per tile."""
    tiles = np.asarray(tiles, dtype=np.float32)
    acc = np.zeros(tiles.shape[0], dtype=np.float32)
    for t in range(tiles.shape[1]):
        acc = acc + tiles[:, t] * tiles[:, t]
    return acc


def matrix_rms(sumsq, n_elems):
    total = 0.0
    for q in sumsq.tolist():                # ascending tile index, binary64
        total += float(q)
    return math.sqrt(total / n_elems)


def sample_tiles(TR, TC, sumsq):
    """Wrapped diagonal plus the largest- and smallest-energy tiles, ascending."""
    picked = set()
    for i in range(max(TR, TC)):
        picked.add((i % TR) * TC + (i % TC))
    picked.add(int(np.argmax(sumsq)))       # first occurrence = lowest index
    picked.add(int(np.argmin(sumsq)))
    return sorted(picked)


GOLDEN = (math.sqrt(5.0) - 1.0) / 2.0


def golden_section(f, lo, hi, iters):
    """Golden-section minimisation of f on [lo, hi]; returns (midpoint, trace).

    Two probes p < q inside the bracket; if f(p) < f(q) the right end moves to
    q, otherwise the left end moves to p; one new probe per reduction.
    """
    a, b = lo, hi
    p = b - (b - a) * GOLDEN
    q = a + (b - a) * GOLDEN
    fp = f(p)
    fq = f(q)
    trace = [(p, fp), (q, fq)]
    for _ in range(iters):
        if fp < fq:
            b = q
            q = p
            fq = fp
            p = b - (b - a) * GOLDEN
            fp = f(p)
            trace.append((p, fp))
        else:
            a = p
            p = q
            fp = fq
            q = a + (b - a) * GOLDEN
            fq = f(q)
            trace.append((q, fq))
    return (a + b) / 2.0, trace


GRID_DEFAULT = (0.1, 1.9, 0.1, 2, 0.075, 0.025, 0.01)


def grid_search(f_sub, f_full, grid=GRID_DEFAULT):
    """The pages' scale search over a multiplier g of the matrix rms
    [P1 item 8: coarse grid on a strided subsample, fine grid around the
    coarse minimum on the full sample, parabolic refinement with a floor].

    grid = (coarse_lo, coarse_hi, coarse_step, stride, fine_radius, fine_step,
    floor); f_sub / f_full map g to the objective on the subsample / full
    sample.  Readings: coarse points lo + k * step for k = 0 .. round((hi - lo) /
    step); the least objective wins, the lowest g on ties; fine points g_c + m *
    fine_step for |m| <= round(fine_radius / fine_step); if the fine minimum g_f
    is interior and d = f(g_f - h) - 2 f(g_f) + f(g_f + h) > 0, the vertex
    g_f + h (f(g_f - h) - f(g_f + h)) / (2 d) replaces it; the result is at least
    floor.  Returns (g, trace)."""
    lo, hi, step, _stride, radius, fstep, floor = grid
    n_c = int(round((hi - lo) / step))
    trace = []
    best_g, best_f = None, None
    for k in range(n_c + 1):
        g = lo + k * step
        v = f_sub(g)
        trace.append(("coarse", g, v))
        if best_f is None or v < best_f:
            best_g, best_f = g, v
    g_c = best_g
    M = int(round(radius / fstep))
    fine = []
    for m in range(-M, M + 1):
        g = g_c + m * fstep
        v = f_full(g)
        trace.append(("fine", g, v))
        fine.append((g, v))
    i_best = 0
    for i in range(1, len(fine)):
        if fine[i][1] < fine[i_best][1]:
            i_best = i
    g_f, f0 = fine[i_best]
    g = g_f
    if 0 < i_best < len(fine) - 1:
        fm, fp = fine[i_best - 1][1], fine[i_best + 1][1]
        d = fm - 2.0 * f0 + fp
        if d > 0.0:
            g = g_f + fstep * (fm - fp) / (2.0 * d)
    g = max(g, floor)
    trace.append(("result", g, None))
    return g, trace


def encode_tiles(tiles, K, scale, levels=None, threads=None):
    """Encode tiles [n, 256] at a fixed binary32 scale.

    Returns dict(states, X, sse, packed).  sse is the pass-2 path cost, which is
    also the sequential sum of squared errors of the dequantised tile.
    """
    if levels is None:
        levels = mul1_levels_fp16()
    v = scaled_levels(levels, scale)
    states, X, cost = encode_sequences(tiles, K, v, threads=threads)
    return {"states": states, "X": X, "sse": cost, "packed": pack_states(states, K)}


def quantize_matrix(w, su, sv, K, had_block=128, gss=(12, 0.5, 2.0), fixed_scale=1.0,
                    levels=None, threads=None, tiles_subset=None, grid=None, order=None):
    """Whole-matrix path: regularize, statistics, scale search, final encode.

    gss=None uses fixed_scale; grid (a GRID_DEFAULT-shaped tuple), if given,
    replaces the golden-section search with grid_search, the scale being
    (float)(g * rms).  tiles_subset, if given, restricts the FINAL encode to
    those tile indices (the scale search always uses its full sample), which is
    how large matrices are checked one sampled tile at a time.  order, if given,
    is the within-tile order of the tiles (to_tiles).
    """
    w = np.asarray(w, dtype=np.float32)
    R, C = w.shape
    if levels is None:
        levels = mul1_levels_fp16()
    w_reg = regularize(w, su, sv, had_block)
    tiles = to_tiles(w_reg, order)
    TR, TC = R // 16, C // 16
    sumsq = tile_sumsq(tiles)
    rms = matrix_rms(sumsq, R * C)
    out = {"tiles": tiles, "sumsq": sumsq, "rms": rms}
    if grid is not None:
        sample = sample_tiles(TR, TC, sumsq)
        out["sample"] = sample
        if rms == 0.0:
            scale = np.float32(0.0)
            out["trace"] = []
        else:
            stride = grid[3]

            def objective(g, idx):
                r = encode_tiles(tiles[idx], K, np.float32(g * rms), levels, threads)
                total = 0.0
                for e in r["sse"].tolist():
                    total += float(e)
                return total

            sub = sample[::stride]
            g, trace = grid_search(lambda g: objective(g, sub), lambda g: objective(g, sample),
                                   grid)
            scale = np.float32(g * rms)
            out["trace"] = trace
    elif gss is None:
        scale = np.float32(fixed_scale)
        out["sample"] = []
        out["trace"] = []
    else:
        iters, lo, hi = gss
        sample = sample_tiles(TR, TC, sumsq)
        out["sample"] = sample
        if rms == 0.0:
            scale = np.float32(0.0)
            out["trace"] = []
        else:
            xs = tiles[sample]

            def objective(s):
                r = encode_tiles(xs, K, np.float32(s), levels, threads)
                total = 0.0
                for e in r["sse"].tolist():
                    total += float(e)
                return total

            mid, trace = golden_section(objective, lo * rms, hi * rms, iters)
            scale = np.float32(mid)
            out["trace"] = trace
    out["scale"] = scale
    idx = np.arange(TR * TC) if tiles_subset is None else np.asarray(tiles_subset)
    r = encode_tiles(tiles[idx], K, scale, levels, threads)
    out.update({"index": idx, "states": r["states"], "X": r["X"], "sse": r["sse"],
                "packed": r["packed"]})
    if tiles_subset is None:
        total = 0.0
        for e in r["sse"].tolist():
            total += float(e)
        out["mse"] = total / (R * C)
    return out


# --------------------------------------------------------------------------
# LDLQ error feedback  [P1 item 3: one-sided block LDLQ, bottom-up span
# traversal, additive target correction from the strictly lower L blocks]
# --------------------------------------------------------------------------
def ldlq(w_reg, L, K, scale, levels=None, threads=None, order=None):
    """Quantize the regularized matrix span by span with LDLQ error feedback.

    Readings (listed in the design notes): H = L D L^T over the columns, L unit
    block-lower-triangular with 16x16 blocks (only the blocks below the
    diagonal are read); spans are 16-column tile columns, processed from the
    last to the first; the target of span j is
        T_j = W_j + sum_{i > j} E_i L_ij,   E_i = W_i - What_i   (binary32),
    accumulated per element in the order i ascending, then row t of the block
    ascending, each product and each sum rounded on its own; span j's tiles are
    then encoded at the fixed scale and What_j = v[states].  Tiles are formed
    in the within-tile order `order` (to_tiles) for encoding and put back in
    matrix order for the feedback.
    Returns dict(what [R, C], targets [R, C], states [TR*TC, 256] in tile order,
    packed [TR*TC, 16K], err: per tile sequential binary32 sum of (W - What)^2).
    """
    W = np.asarray(w_reg, dtype=np.float32)
    L = np.asarray(L, dtype=np.float32)
    R, C = W.shape
    TR, TC = R // 16, C // 16
    if levels is None:
        levels = mul1_levels_fp16()
    v = scaled_levels(levels, scale)
    what = np.empty((R, C), np.float32)
    E = np.empty((R, C), np.float32)
    targets = np.empty((R, C), np.float32)
    states = np.empty((TR, TC, 256), np.int32)
    for j in range(TC - 1, -1, -1):
        cj = slice(16 * j, 16 * j + 16)
        T = W[:, cj].copy()
        for i in range(j + 1, TC):
            for t in range(16):
                col = 16 * i + t
                T = T + E[:, col:col + 1] * L[col:col + 1, cj]
        targets[:, cj] = T
        r = encode_tiles(to_tiles(T, order), K, scale, levels, threads)
        states[:, j, :] = r["states"]
        what[:, cj] = from_tiles(v[r["states"]], R, 16, order)
        E[:, cj] = W[:, cj] - what[:, cj]
    st = states.reshape(TR * TC, 256)
    return {"what": what, "targets": targets, "states": st,
            "packed": pack_states(st, K), "err": tile_sse(to_tiles(W, order), st, v)}


def quantize_matrix_ldlq(w, su, sv, K, L, had_block=128, gss=(12, 0.5, 2.0), fixed_scale=1.0,
                         levels=None, threads=None, order=None):
    """Regularize, choose the scale exactly as quantize_matrix does (on the
    matrix without feedback), then run ldlq at that scale."""
    base = quantize_matrix(w, su, sv, K, had_block, gss, fixed_scale, levels, threads,
                           tiles_subset=np.zeros(0, np.int64), order=order)
    R, C = np.asarray(w).shape
    w_reg = from_tiles(base["tiles"], R, C, order)
    out = ldlq(w_reg, L, K, base["scale"], levels, threads, order)
    total = 0.0
    for e in out["err"].tolist():
        total += float(e)
    out.update({"scale": base["scale"], "rms": base["rms"], "w_reg": w_reg,
                "mse": total / (R * C)})
    return out


# --------------------------------------------------------------------------
# fp16 mode  [P1 items 1 and 4: binary16 difference, single-rounded fused
# multiply-add into binary16 path costs, first-branch strict "<" ties]
# --------------------------------------------------------------------------
def f16_sub(a: int, b: int) -> int:
    """Bits of fp16(a - b) for binary16 bit patterns a, b (one rounding)."""
    return int(_load().oracle_f16_sub(a, b))


def f16_sqadd(d: int, m: int) -> int:
    """Bits of fp16(d*d + m), rounded once (fused), for binary16 bit patterns."""
    return int(_load().oracle_f16_sqadd(d, m))


def forward_f16(x_bits, Q, K, c_bits, M0_bits):
    """fp16 forward pass; returns (final-step costs as uint16 bits, predecessors)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    c = np.ascontiguousarray(c_bits, dtype=np.uint16)
    M0 = np.ascontiguousarray(M0_bits, dtype=np.uint16)
    L = x.shape[0]
    C = np.empty(1 << Q, dtype=np.uint16)
    bp = np.empty(((L - 1), 1 << (Q - K)), dtype=np.uint8)
    rc = _load().oracle_forward_f16(x, L, Q, K, c, M0, C, bp)
    if rc != 0:
        raise ValueError("oracle_forward_f16 rejected its arguments (rc=%d)" % rc)
    return C, bp


def encode_sequences_f16(x_bits, K, c_bits, Q=STATE_BITS, threads=None):
    """fp16 two-pass encode of each row of x_bits [n, L] (binary16 bit patterns).

    Returns (states int32 [n, L], X int32 [n], cost uint16 bits [n]).
    """
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    c = np.ascontiguousarray(c_bits, dtype=np.uint16)
    n, L = x.shape
    states = np.empty((n, L), dtype=np.int32)
    X = np.empty(n, dtype=np.int32)
    cost = np.empty(n, dtype=np.uint16)
    if n == 0:
        return states, X, cost
    lib = _load()
    threads = threads or default_threads()
    chunks = np.array_split(np.arange(n), min(threads, n))

    def run(idx):
        if idx.size == 0:
            return 0
        i0 = int(idx[0])
        return lib.oracle_encode_many_f16(
            x[i0:].ctypes.data, int(idx.size), L, Q, K, c,
            states[i0:].ctypes.data, X[i0:].ctypes.data, cost[i0:].ctypes.data)

    if len(chunks) == 1:
        rcs = [run(chunks[0])]
    else:
        with ThreadPoolExecutor(max_workers=len(chunks)) as ex:
            rcs = list(ex.map(run, chunks))
    if any(rc != 0 for rc in rcs):
        raise ValueError("oracle_encode_many_f16 rejected its arguments (rc=%s)" % rcs)
    return states, X, cost


def encode_tiles_f16(x_bits, K, levels=None, threads=None):
    """fp16-mode encode of tiles [n, 256] given as binary16 bits, raw level table."""
    if levels is None:
        levels = mul1_levels_fp16()
    states, X, cost = encode_sequences_f16(x_bits, K, levels.view(np.uint16), threads=threads)
    return {"states": states, "X": X, "cost": cost, "packed": pack_states(states, K)}


def to_f16_inputs(tiles, scale) -> np.ndarray:
    """Binary16 encoder inputs of regularized tiles at a scale: each weight
    divided by the scale (one binary32 division, correctly rounded), then
    rounded to binary16 (nearest even); all zeros when the scale is 0.
    Returned as binary16 bit patterns."""
    t = np.asarray(tiles, np.float32)
    s = np.float32(scale)
    if s == 0:
        return np.zeros(t.shape, np.uint16)
    return (t / s).astype(np.float32).astype(np.float16).view(np.uint16)


def encode_tiles_f16_scaled(tiles, K, scale, levels=None, threads=None):
    """Binary16-mode search on fp16(w / scale); the result dequantized as
    w_hat = rn32(scale * level) and scored with the same sequential binary32
    squared error as the binary32 path (tile_sse)."""
    if levels is None:
        levels = mul1_levels_fp16()
    x16 = to_f16_inputs(tiles, scale)
    r = encode_tiles_f16(x16, K, levels, threads)
    v = scaled_levels(levels, scale)
    sse = tile_sse(np.asarray(tiles, np.float32), r["states"], v)
    r.update({"x16": x16, "sse": sse})
    return r


def quantize_matrix_f16(w, su, sv, K, had_block=128, gss=(12, 0.5, 2.0), fixed_scale=1.0,
                        levels=None, threads=None, tiles_subset=None, order=None):
    """Whole-matrix path with the binary16 encoder inside the scale search.

    Regularization, statistics, tile sample and golden section exactly as in
    quantize_matrix; the objective at scale s is the binary64 ascending sum of
    the binary32 squared errors of the sample tiles encoded by
    encode_tiles_f16_scaled at s; the final encode likewise."""
    w = np.asarray(w, dtype=np.float32)
    R, C = w.shape
    if levels is None:
        levels = mul1_levels_fp16()
    tiles = to_tiles(regularize(w, su, sv, had_block), order)
    TR, TC = R // 16, C // 16
    sumsq = tile_sumsq(tiles)
    rms = matrix_rms(sumsq, R * C)
    out = {"tiles": tiles, "sumsq": sumsq, "rms": rms}
    if gss is None:
        scale = np.float32(fixed_scale)
        out["sample"], out["trace"] = [], []
    else:
        iters, lo, hi = gss
        sample = sample_tiles(TR, TC, sumsq)
        out["sample"] = sample
        if rms == 0.0:
            scale = np.float32(0.0)
            out["trace"] = []
        else:
            xs = tiles[sample]

            def objective(s):
                r = encode_tiles_f16_scaled(xs, K, np.float32(s), levels, threads)
                total = 0.0
                for e in r["sse"].tolist():
                    total += float(e)
                return total

            mid, trace = golden_section(objective, lo * rms, hi * rms, iters)
            scale = np.float32(mid)
            out["trace"] = trace
    out["scale"] = scale
    idx = np.arange(TR * TC) if tiles_subset is None else np.asarray(tiles_subset)
    r = encode_tiles_f16_scaled(tiles[idx], K, scale, levels, threads)
    out.update({"index": idx, "states": r["states"], "sse": r["sse"], "packed": r["packed"]})
    if tiles_subset is None:
        total = 0.0
        for e in r["sse"].tolist():
            total += float(e)
        out["mse"] = total / (R * C)
    return out
