"""Whole-matrix path with the binary16 encoder, GPU library against the oracle, through the C ABI.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture items 1 and 4
(half-precision search) and item 8 (scale search); "JEV-9B EXL3 K=2 (mul1) Checkpoint"
model card, section 2 (golden section).

Small matrices: the chosen scale, container words, per-tile binary32 errors, dequantized
tiles and MSE bit-exact against oracle.quantize_matrix_f16 (golden section, and a fixed
scale).  At 4096x4096: the scale in the search bracket, sampled tiles of the final encode
bit-exact at the GPU's scale, the MSE the ascending sum of the tile errors.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ctx():
    import trellis_coded_weight_amd as T
    c = T.Context(0)
    yield c
    c.close()


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _dev(m):
    w = torch.from_numpy(m.w).to(torch.bfloat16 if m.dtype == "bf16" else torch.float32).to(DEV)
    return w, torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV)


@pytest.mark.parametrize("K,gss", [(2, (12, 0.5, 2.0)), (3, None)])
def test_f16_matrix_bit_exact_small(ctx, K, gss):
    print("\nf16 matrix 64x64 K=%d gss=%s" % (K, gss), flush=True)
    m = workloads.gaussian(64, 64, 0.02, 40 + K, 50 + K, K=K, had_block=64, gss=gss)
    want = oracle.quantize_matrix_f16(m.w, m.su, m.sv, K, had_block=64, gss=gss,
                                      fixed_scale=0.0187)
    w, su, sv = _dev(m)
    got = ctx.quantize_matrix_f16(w, K, su, sv, had_block=64, gss=gss, scale=0.0187,
                                  want_w_hat=True, want_tile_sse=True)
    assert np.float32(got["scale"]) == want["scale"]
    assert np.array_equal(got["packed"].cpu().numpy().view(np.uint16).reshape(-1, 16 * K),
                          want["packed"])
    assert np.array_equal(_bits(got["tile_sse"].cpu().numpy()), _bits(want["sse"]))
    v = oracle.scaled_levels(oracle.mul1_levels_fp16(), want["scale"])
    assert np.array_equal(_bits(got["w_hat"].cpu().numpy()), _bits(v[want["states"]]))
    assert got["mse"] == want["mse"]


def test_zero_matrix(ctx):
    import trellis_coded_weight_amd as T
    w = torch.zeros(64, 64, dtype=torch.bfloat16, device=DEV)
    su = torch.ones(64, device=DEV)
    got = ctx.quantize_matrix_f16(w, 2, su, su, had_block=64, want_tile_sse=True)
    assert got["scale"] == 0.0 and got["mse"] == 0.0
    assert not torch.any(got["tile_sse"] != 0)


@pytest.mark.slow
def test_f16_matrix_4096(ctx):
    m = workloads.config(2)[0]
    R, C = m.w.shape
    print("\nf16 matrix 4096x4096 K=2", flush=True)
    w, su, sv = _dev(m)
    got = ctx.quantize_matrix_f16(w, 2, su, sv, want_tile_sse=True)
    reg, sums, _ = ctx.regularize(w, su, sv, 128)
    torch.cuda.synchronize()
    rms = oracle.matrix_rms(sums.cpu().numpy(), R * C)
    scale = np.float32(got["scale"])
    assert 0.5 * rms <= float(scale) <= 2.0 * rms
    rng = np.random.default_rng(5)
    ids = sorted({0, R * C // 256 - 1} | set(rng.integers(0, R * C // 256, 10).tolist()))
    # the oracle's own regularization of the matrix (the GPU's is checked
    # against it elsewhere); the scale's bits are checked against the oracle's
    # golden section in the workload digests
    tiles = oracle.to_tiles(oracle.regularize(m.w, m.su, m.sv, 128))[ids]
    want = oracle.encode_tiles_f16_scaled(tiles, 2, scale)
    packed = got["packed"].cpu().numpy().view(np.uint16).reshape(-1, 32)
    tsse = got["tile_sse"].cpu().numpy()
    assert np.array_equal(packed[ids], want["packed"])
    assert np.array_equal(_bits(tsse[ids]), _bits(want["sse"]))
    tot = 0.0
    for e in tsse.tolist():
        tot += float(e)
    assert got["mse"] == tot / (R * C)
