"""Within-tile order (the tensor-core permutation slot) of the GPU library against the oracle.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 5
(a 256-element permutation of the positions within a tile, not printed) and item 3
(LDLQ encodes permuted tiles and reconstructs in matrix order).

With a random order set on the context: tile-major regularization and its per-tile
energies, the inverse regularization, the whole-matrix path (golden section,
container, dequantized tiles, per-tile errors, MSE), the binary16 whole-matrix
path and LDLQ are bit-exact against the oracle given the same order; the tile
encoder itself does not depend on it; the identity and None restore the natural
order; a table that is not a permutation is rejected.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ORDER = np.random.default_rng(2024).permutation(256)


@pytest.fixture()
def ctx():
    import trellis_coded_weight_amd as T
    c = T.Context(0)
    c.set_tile_order(ORDER)
    yield c
    c.close()


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _dev(m):
    w = torch.from_numpy(m.w).to(torch.bfloat16 if m.dtype == "bf16" else torch.float32).to(DEV)
    return w, torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV)


@pytest.mark.parametrize("B", [64, 128])
def test_regularize_and_inverse(ctx, B):
    m = workloads.gaussian(2 * B, 3 * B, 0.02, 5 + B, 6 + B, K=2)
    w, su, sv = _dev(m)
    reg, sums, _ = ctx.regularize(w, su, sv, had_block=B)
    want = oracle.to_tiles(oracle.regularize(m.w, m.su, m.sv, B), ORDER)
    assert np.array_equal(_bits(reg.cpu().numpy()), _bits(want))
    assert np.array_equal(_bits(sums.cpu().numpy()), _bits(oracle.tile_sumsq(want)))
    back = ctx.unregularize(reg, 2 * B, 3 * B, su, sv, had_block=B)
    want_back = oracle.unregularize(oracle.from_tiles(want, 2 * B, 3 * B, ORDER), m.su, m.sv, B)
    assert np.array_equal(_bits(back.cpu().numpy()), _bits(want_back))


# 4096 x 4096: more blocks than workgroups resident at once (1,024 blocks of 128
# or 4,096 of 64), so each workgroup takes several blocks in turn, with the
# next block's loads (and its signs) issued early (bf16) or at the top of each
# block (fp32 at B = 128).  The row-major output (natural element order, the
# energies still in the tiles' order) goes back through LDS before its row
# stores.
@pytest.mark.parametrize("B,dtype,tile_major", [(128, torch.bfloat16, True),
                                                (64, torch.bfloat16, True),
                                                (128, torch.float32, True),
                                                (128, torch.bfloat16, False),
                                                (64, torch.float32, False)])
def test_regularize_many_blocks_per_workgroup(ctx, B, dtype, tile_major):
    m = workloads.gaussian(4096, 4096, 0.02, 31, 32, K=2)
    w = torch.from_numpy(m.w).to(dtype).to(DEV)
    su, sv = torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV)
    reg, sums, flag = ctx.regularize(w, su, sv, had_block=B, tile_major=tile_major)
    rm = oracle.regularize(w.cpu().float().numpy(), m.su, m.sv, B)
    want = oracle.to_tiles(rm, ORDER)
    assert np.array_equal(_bits(reg.cpu().numpy()), _bits(want if tile_major else rm))
    assert np.array_equal(_bits(sums.cpu().numpy()), _bits(oracle.tile_sumsq(want)))
    assert int(flag.item()) == 0


def test_whole_matrix_golden_section(ctx):
    m = workloads.gaussian(128, 256, 0.02, 11, 12, K=2)
    w, su, sv = _dev(m)
    want = oracle.quantize_matrix(m.w, m.su, m.sv, 2, had_block=128, gss=(12, 0.5, 2.0),
                                  order=ORDER)
    got = ctx.quantize_matrix(w, 2, su, sv, had_block=128, gss=(12, 0.5, 2.0), want_w_hat=True,
                              want_tile_sse=True)
    assert np.float32(got["scale"]) == want["scale"]
    assert np.array_equal(_u16(got["packed"]).reshape(-1, 32), want["packed"])
    assert np.array_equal(_bits(got["tile_sse"].cpu().numpy()), _bits(want["sse"]))
    v = oracle.scaled_levels(oracle.mul1_levels_fp16(), want["scale"])
    assert np.array_equal(_bits(got["w_hat"].cpu().numpy()), _bits(v[want["states"]]))
    assert got["mse"] == want["mse"]


def test_binary16_whole_matrix(ctx):
    m = workloads.gaussian(64, 128, 0.02, 21, 22, K=2)
    w, su, sv = _dev(m)
    s = np.float32(0.019)
    want = oracle.quantize_matrix_f16(m.w, m.su, m.sv, 2, had_block=64, gss=None, fixed_scale=s,
                                      order=ORDER)
    got = ctx.quantize_matrix_f16(w, 2, su, sv, had_block=64, gss=None, scale=float(s),
                                  want_tile_sse=True)
    assert np.array_equal(_u16(got["packed"]).reshape(-1, 32), want["packed"])
    assert np.array_equal(_bits(got["tile_sse"].cpu().numpy()), _bits(want["sse"]))


@pytest.mark.parametrize("K", [2, 3])
def test_ldlq(ctx, K):
    m = workloads.gaussian(128, 256, 0.02, 60 + K, 70 + K, K=K, gss=None)
    L, _ = workloads.ldl_factor(256, 80 + K, off_std=1.5)
    scale = 0.017
    want = oracle.quantize_matrix_ldlq(m.w, m.su, m.sv, K, L, had_block=128, gss=None,
                                       fixed_scale=scale, order=ORDER)
    w, su, sv = _dev(m)
    got = ctx.quantize_matrix_ldlq(w, K, su, sv, torch.from_numpy(L).to(DEV), had_block=128,
                                   gss=None, scale=scale, want_w_hat=True, want_tile_err=True)
    assert np.array_equal(_u16(got["packed"]).reshape(-1, 16 * K), want["packed"])
    assert np.array_equal(_bits(got["w_hat"].cpu().numpy()),
                          _bits(oracle.to_tiles(want["what"], ORDER)))
    assert np.array_equal(_bits(got["tile_err"].cpu().numpy()), _bits(want["err"]))
    assert got["mse"] == want["mse"]


def test_tile_encoder_does_not_depend_on_it(ctx):
    x = torch.from_numpy(workloads.random_tiles(5, 3)).to(DEV)
    a = ctx.encode_tiles(x, 2, 1.0)
    ctx.set_tile_order(None)
    b = ctx.encode_tiles(x, 2, 1.0)
    assert np.array_equal(_u16(a[0]), _u16(b[0]))


def test_identity_and_none_restore_natural_order(ctx):
    m = workloads.gaussian(128, 128, 0.02, 31, 32, K=2)
    w, su, sv = _dev(m)
    want = oracle.to_tiles(oracle.regularize(m.w, m.su, m.sv, 128))
    for o in (np.arange(256), None):
        ctx.set_tile_order(o)
        reg, _, _ = ctx.regularize(w, su, sv)
        assert np.array_equal(_bits(reg.cpu().numpy()), _bits(want))
        ctx.set_tile_order(ORDER)


def test_rejects_non_permutation(ctx):
    import trellis_coded_weight_amd as T
    bad = np.arange(256, dtype=np.uint8)
    bad[7] = 3
    rc = ctx.lib.exl3_set_tile_order(ctx.handle, ctypes.c_void_p(bad.ctypes.data))
    assert rc == T.EXL3_EINVAL
    assert "permutation" in ctx.last_error()
    # the order in force is unchanged
    m = workloads.gaussian(128, 128, 0.02, 41, 42, K=2)
    w, su, sv = _dev(m)
    reg, _, _ = ctx.regularize(w, su, sv)
    want = oracle.to_tiles(oracle.regularize(m.w, m.su, m.sv, 128), ORDER)
    assert np.array_equal(_bits(reg.cpu().numpy()), _bits(want))
