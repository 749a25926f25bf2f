"""GPU library on the full-size workloads, checked against the oracle on sampled outputs.

Every matrix runs through exl3_quantize_matrix exactly as the benchmark runs it.
The oracle then recomputes, one by one:
  * sampled 128x128 regularization blocks (blocks are independent) and their tiles'
    energies -- bit-exact;
  * for samples of 258 tiles (4096x4096 and 4096x1024 shapes), the whole golden-section
    search -- the chosen scale must be identical (inside the 1e-5 relative bound);
  * sampled tiles of the final encode at the GPU's scale -- packed words and squared
    errors bit-exact.
Properties that hold at any size: the reported MSE is the ascending binary64 sum of the
per-tile errors; the scale lies in the search bracket; normalised distortion of the
Gaussian workloads lies between the rate-distortion bound and Lloyd-Max; in the layer
workload the MSE falls with K for every matrix.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def ctx():
    import trellis_coded_weight_amd as T
    c = T.Context(0)
    yield c
    c.close()


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _lloyd(K):
    with open(os.path.join(GOLDEN, "pages_figures.json")) as f:
        return json.load(f)["lloyd_max_gaussian_mse"][str(K)]


def _sample_tiles(TR, TC, n=24, seed=0):
    rng = np.random.default_rng(seed)
    picks = {0, TR * TC - 1, TC - 1, (TR - 1) * TC}
    picks.update(int(i) for i in rng.integers(0, TR * TC, n))
    return sorted(picks)


def _oracle_block_tiles(m, br, bc, B=128):
    """Oracle regularization of block (br, bc) -> its tiles, indexed by global tile id."""
    w = m.w[br * B:(br + 1) * B, bc * B:(bc + 1) * B]
    reg = oracle.regularize(w, m.su[br * B:(br + 1) * B], m.sv[bc * B:(bc + 1) * B], B)
    t = oracle.to_tiles(reg)
    TC = m.w.shape[1] // 16
    ids = [(br * (B // 16) + i) * TC + bc * (B // 16) + j
           for i in range(B // 16) for j in range(B // 16)]
    return dict(zip(ids, t))


def _oracle_tiles(m, tile_ids, B=128):
    """Oracle tiles for arbitrary tile ids, regularizing only the blocks they sit in."""
    TC = m.w.shape[1] // 16
    per = B // 16
    out = {}
    blocks = sorted({((t // TC) // per, (t % TC) // per) for t in tile_ids})
    for br, bc in blocks:
        out.update(_oracle_block_tiles(m, br, bc, B))
    return np.stack([out[t] for t in tile_ids])


def _run(ctx, m, K):
    w = torch.from_numpy(m.w).to(torch.bfloat16 if m.dtype == "bf16" else torch.float32).to(DEV)
    su = torch.from_numpy(m.su).to(DEV)
    sv = torch.from_numpy(m.sv).to(DEV)
    got = ctx.quantize_matrix(w, K, su, sv, had_block=m.had_block, gss=m.gss,
                              want_tile_sse=True)
    reg, sums, flag = ctx.regularize(w, su, sv, m.had_block)
    torch.cuda.synchronize()
    return got, reg, sums, flag


def _check_matrix(ctx, m, K, exact_gss, levels=None):
    R, C = m.w.shape
    TR, TC = R // 16, C // 16
    print("\n%s %dx%d K=%d" % (m.name, R, C, K), flush=True)
    got, reg, sums, flag = _run(ctx, m, K)
    assert int(flag.item()) == 0
    sums = sums.cpu().numpy()
    # sampled regularization blocks and their energies
    rng = np.random.default_rng(R * 7 + C)
    blocks = {(0, 0), (R // 128 - 1, C // 128 - 1)}
    blocks.update((int(rng.integers(0, R // 128)), int(rng.integers(0, C // 128))) for _ in range(3))
    reg_np = None
    for br, bc in sorted(blocks):
        want = _oracle_block_tiles(m, br, bc)
        ids = sorted(want)
        if reg_np is None:
            reg_np = reg.cpu().numpy()
        assert np.array_equal(_bits(reg_np[ids]), _bits(np.stack([want[i] for i in ids])))
        assert np.array_equal(_bits(sums[ids]),
                              _bits(oracle.tile_sumsq(np.stack([want[i] for i in ids]))))
    rms = oracle.matrix_rms(sums, R * C)
    lo, hi = m.gss[1] * rms, m.gss[2] * rms
    scale = np.float32(got["scale"])
    assert lo <= float(scale) <= hi
    # the whole scale search, when the sample is small enough to redo on the host
    if exact_gss:
        sample = oracle.sample_tiles(TR, TC, sums)
        xs = _oracle_tiles(m, sample)
        lv = oracle.mul1_levels_fp16() if levels is None else levels

        def f(s):
            r = oracle.encode_tiles(xs, K, np.float32(s), lv)
            tot = 0.0
            for e in r["sse"].tolist():
                tot += float(e)
            return tot

        mid, _ = oracle.golden_section(f, lo, hi, m.gss[0])
        assert abs(float(scale) - mid) <= 1e-5 * abs(mid)
        assert scale == np.float32(mid)
    # sampled tiles of the final encode at the chosen scale
    ids = _sample_tiles(TR, TC, seed=R + C + K)
    xs = _oracle_tiles(m, ids)
    want = oracle.encode_tiles(xs, K, scale, levels)
    packed = got["packed"].cpu().numpy().view(np.uint16).reshape(-1, 16 * K)
    tsse = got["tile_sse"].cpu().numpy()
    assert np.array_equal(packed[ids], want["packed"])
    assert np.array_equal(_bits(tsse[ids]), _bits(want["sse"]))
    # reported MSE = ascending binary64 sum of the per-tile errors
    tot = 0.0
    for e in tsse.tolist():
        tot += float(e)
    assert got["mse"] == tot / (R * C)
    return got, rms


def test_workload2_4096x4096_k2(ctx):
    m = workloads.config(2)[0]
    got, rms = _check_matrix(ctx, m, 2, exact_gss=True)
    nmse = got["mse"] / rms ** 2
    assert 2.0 ** -4 < nmse < _lloyd(2)
    # relative Frobenius error inside the K = 2 band the checkpoint card prints
    with open(os.path.join(GOLDEN, "pages_figures.json")) as f:
        lo, hi = json.load(f)["k2_rel_frobenius_band"]
    assert lo <= math.sqrt(nmse) <= hi


def test_workload2_at_k1(ctx):
    """The 4096x4096 matrix at K = 1 (the benchmark's K = 1 figure), in its 8,192-tile
    launches: sampled tiles bit-exact, the scale in the bracket, the MSE sum."""
    m = workloads.config(2)[0]
    got, rms = _check_matrix(ctx, m, 1, exact_gss=False)
    assert 0.0 < got["mse"] / rms ** 2 < _lloyd(1)


def test_workload3_heavy_tailed_k4(ctx):
    m = workloads.config(3)[0]
    got, rms = _check_matrix(ctx, m, 4, exact_gss=True)
    assert 0.0 < got["mse"] / rms ** 2 < 2 * _lloyd(4)


def test_workload4_mlp_k3(ctx):
    for m in workloads.config(4):
        got, rms = _check_matrix(ctx, m, 3, exact_gss=False)
        assert 2.0 ** -6 < got["mse"] / rms ** 2 < _lloyd(3)


def test_workload5_layer_all_k(ctx):
    for m in workloads.config(5):
        mses = []
        for K in (2, 3, 4):
            small = m.w.shape[1] == 1024 and K == 3
            got, rms = _check_matrix(ctx, m, K, exact_gss=small)
            nmse = got["mse"] / rms ** 2
            assert 2.0 ** (-2 * K) < nmse < _lloyd(K)
            mses.append(got["mse"])
        assert mses[0] > mses[1] > mses[2]


def test_workload2_grid_search_scale(ctx):
    """The pages' grid + parabolic search on the 4096x4096 matrix: the chosen scale is
    the oracle's (19 coarse probes on 129 sample tiles, 7 fine probes on 258)."""
    import trellis_coded_weight_amd as T
    m = workloads.config(2)[0]
    R, C = m.w.shape
    print("\ngrid search 4096x4096 K=2", flush=True)
    w = torch.from_numpy(m.w).to(torch.bfloat16).to(DEV)
    su, sv = torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV)
    got = ctx.quantize_matrix_grid(w, 2, su, sv, grid=T.GRID_PAGES, want_tile_sse=True)
    reg, sums, _ = ctx.regularize(w, su, sv, 128)
    sums = sums.cpu().numpy()
    rms = oracle.matrix_rms(sums, R * C)
    sample = oracle.sample_tiles(R // 16, C // 16, sums)
    xs = _oracle_tiles(m, sample)

    def f(idx_pos):
        def obj(g):
            r = oracle.encode_tiles(xs[idx_pos], 2, np.float32(g * rms))
            return sum(float(e) for e in r["sse"].tolist())
        return obj

    g, _ = oracle.grid_search(f(np.arange(len(sample))[::2]), f(np.arange(len(sample))),
                              oracle.GRID_DEFAULT)
    assert np.float32(got["scale"]) == np.float32(g * rms)


@pytest.mark.parametrize("name", ["mcg", "3inst"])
def test_workload2_other_codebooks(ctx, name):
    """The 4096x4096 matrix at K=2 with the mcg / 3INST tables: regularization blocks,
    bracket, sampled final tiles and the MSE sum, as for mul1."""
    m = workloads.config(2)[0]
    ctx.set_codebook_kind(name)
    try:
        got, rms = _check_matrix(ctx, m, 2, exact_gss=False, levels=oracle.CODEBOOKS[name]())
    finally:
        ctx.set_codebook_kind("mul1")
    assert 2.0 ** -4 < got["mse"] / rms ** 2 < _lloyd(2)


@pytest.mark.parametrize("K", [2, 3, 4, 1])
def test_workload2_binary16_all_tiles(ctx, K):
    """All 65,536 tiles of the 4096x4096 matrix in binary16 mode (regularized, divided by
    a scale, rounded to binary16 -- the benchmark's input), in the batches the benchmark
    uses; sampled tiles bit-exact against the oracle's binary16 encoder."""
    m = workloads.config(2)[0]
    R, C = m.w.shape
    print("\nbinary16 4096x4096 K=%d" % K, flush=True)
    w = torch.from_numpy(m.w).to(torch.bfloat16).to(DEV)
    su, sv = torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV)
    reg, _, _ = ctx.regularize(w, su, sv, 128)
    xh = (reg / 0.0202).to(torch.float16).contiguous()
    packed, states, cost = ctx.encode_tiles_f16(xh, K)
    torch.cuda.synchronize()
    ids = _sample_tiles(R // 16, C // 16, n=12, seed=K)
    xb = xh.cpu().numpy().view(np.uint16)[ids]
    want = oracle.encode_tiles_f16(xb, K)
    assert np.array_equal(states.cpu().numpy().view(np.uint16)[ids], want["states"])
    assert np.array_equal(packed.cpu().numpy().view(np.uint16)[ids], want["packed"])
    assert np.array_equal(cost.cpu().numpy().view(np.uint16)[ids], np.asarray(want["cost"], np.uint16))
