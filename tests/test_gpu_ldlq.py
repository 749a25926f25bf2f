"""LDLQ whole-matrix path of the GPU library against the oracle, through the C ABI.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 3.

Small matrices: scale, container words, dequantized tiles and per-tile errors bit-exact
against oracle.quantize_matrix_ldlq (synthetic factor from workloads.ldl_factor).
At 4096^2: eight whole tile rows of the full run bit-exact against the oracle's LDLQ on
those rows (rows are independent).  Properties at any size: an identity factor reproduces
exl3_quantize_matrix; the container decodes to the dequantized tiles; every sampled span
is the tile encoder's output on its target recomputed on the host from the regularized
matrix and the spans after it.
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


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _dev(m):
    w = torch.from_numpy(m.w).to(torch.bfloat16 if m.dtype == "bf16" else torch.float32).to(DEV)
    return w, torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV)


# 192 rows with 64-blocks: twelve tile rows, six per stream
@pytest.mark.parametrize("R,hb,K,gss", [(128, 128, 2, (12, 0.5, 2.0)), (128, 128, 1, None),
                                        (128, 128, 4, None), (192, 64, 3, None)])
def test_ldlq_bit_exact_small(ctx, R, hb, K, gss):
    m = workloads.gaussian(R, 256, 0.02, 60 + K, 70 + K, had_block=hb, K=K, gss=gss)
    L, _ = workloads.ldl_factor(256, 80 + K, off_std=1.5)
    scale = {1: 0.022, 2: 0.017, 3: 0.014, 4: 0.012}[K]
    print("\nldlq %dx256 hb=%d K=%d gss=%s" % (R, hb, K, gss), flush=True)
    want = oracle.quantize_matrix_ldlq(m.w, m.su, m.sv, K, L, had_block=hb, gss=gss,
                                       fixed_scale=scale)
    w, su, sv = _dev(m)
    got = ctx.quantize_matrix_ldlq(w, K, su, sv, torch.from_numpy(L).to(DEV), had_block=hb,
                                   gss=gss, scale=scale, want_w_hat=True, want_tile_err=True)
    assert np.float32(got["scale"]) == want["scale"]
    assert np.array_equal(_u16(got["packed"]).reshape(-1, 16 * K), want["packed"])
    assert np.array_equal(_bits(got["w_hat"].cpu().numpy()), _bits(oracle.to_tiles(want["what"])))
    assert np.array_equal(_bits(got["tile_err"].cpu().numpy()), _bits(want["err"]))
    assert got["mse"] == want["mse"]


def test_identity_factor_matches_plain_path(ctx):
    m = workloads.gaussian(256, 256, 0.02, 91, 92, K=2)
    w, su, sv = _dev(m)
    eye = torch.eye(256, dtype=torch.float32, device=DEV)
    a = ctx.quantize_matrix_ldlq(w, 2, su, sv, eye, gss=m.gss, want_tile_err=True)
    b = ctx.quantize_matrix(w, 2, su, sv, gss=m.gss, want_tile_sse=True)
    assert a["scale"] == b["scale"]
    assert np.array_equal(_u16(a["packed"]), _u16(b["packed"]))
    assert np.array_equal(_bits(a["tile_err"].cpu().numpy()), _bits(b["tile_sse"].cpu().numpy()))


def test_ldlq_rejects_null_factor(ctx):
    import ctypes
    import trellis_coded_weight_amd as T
    m = workloads.gaussian(128, 128, 0.02, 1, 2, K=2)
    w, su, sv = _dev(m)
    packed = torch.empty(8, 8, 32, dtype=torch.int16, device=DEV)
    s = ctypes.c_float(0.0)
    rc = ctx.lib.exl3_quantize_matrix_ldlq(
        ctx.handle, ctypes.c_void_p(w.data_ptr()), T.EXL3_BF16, 128, 128, 2, 128,
        ctypes.c_void_p(su.data_ptr()), ctypes.c_void_p(sv.data_ptr()), None, 1.0, None,
        ctypes.c_void_p(packed.data_ptr()), ctypes.byref(s), None, None, None)
    assert rc == T.EXL3_EINVAL


def _host_target(w_reg, what, L, j):
    """T_j from the regularized matrix and the dequantized spans after j, in the
    stated binary32 order (i ascending, then the block row ascending)."""
    C = w_reg.shape[1]
    cj = slice(16 * j, 16 * j + 16)
    E = (w_reg - what).astype(np.float32)
    T = w_reg[:, cj].copy()
    for col in range(16 * (j + 1), C):
        T = T + E[:, col:col + 1] * L[col:col + 1, cj]
    return T


@pytest.mark.slow
def test_ldlq_full_size_properties(ctx):
    K = 2
    m = workloads.config(2)[0]
    R, C = m.w.shape
    L, _ = workloads.ldl_factor(C, 2102)
    w, su, sv = _dev(m)
    print("\nldlq 4096x4096 K=2", flush=True)
    got = ctx.quantize_matrix_ldlq(w, K, su, sv, torch.from_numpy(L).to(DEV), gss=m.gss,
                                   want_w_hat=True, want_tile_err=True)
    plain = ctx.quantize_matrix(w, K, su, sv, gss=m.gss)
    assert got["scale"] == plain["scale"]
    scale = np.float32(got["scale"])
    wh_tiles = got["w_hat"]
    # the container decodes to the dequantized tiles
    dec = ctx.decode_tiles(got["packed"].reshape(-1, 16 * K), K, float(scale))
    assert torch.equal(dec, wh_tiles)
    # mse is the ascending binary64 sum of the per-tile errors
    tot = 0.0
    for e in got["tile_err"].cpu().numpy().tolist():
        tot += float(e)
    assert got["mse"] == tot / (R * C)
    # sampled spans: the span's tiles are the encoder's output on the recomputed target
    reg, _, _ = ctx.regularize(w, su, sv, 128)
    w_reg = oracle.from_tiles(reg.cpu().numpy(), R, C)
    what = oracle.from_tiles(wh_tiles.cpu().numpy(), R, C)
    TC = C // 16
    for j in (TC - 1, TC - 2, 131, 0):
        T = _host_target(w_reg, what, L, j)
        tiles = torch.from_numpy(oracle.to_tiles(T)).to(DEV)
        p, _, _ = ctx.encode_tiles(tiles, K, float(scale), want_states=False, want_sse=False)
        span = _u16(got["packed"])[:, j, :]
        assert np.array_equal(_u16(p), span), j


@pytest.mark.slow
def test_ldlq_full_size_bands_match_oracle(ctx):
    """At 4096^2, K = 2: rows of span j's target depend only on the same rows of
    the spans after it, so the oracle's LDLQ on a band of whole tile rows (its
    own regularization of the matrix, at the scale its own golden-section search
    chose, read from the stored workload digests) must reproduce those rows of
    the GPU's full run bit for bit: container words, dequantized tiles and
    per-tile errors."""
    import json
    import os
    K = 2
    m = workloads.config(2)[0]
    R, C = m.w.shape
    TC = C // 16
    digests = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                          "golden", "config_digests.json")))["runs"]
    scale = np.uint32(int(digests["c2_c2_4096x4096_K2"]["scale_bits"], 16)).view(np.float32)
    L, _ = workloads.ldl_factor(C, 2102)
    w, su, sv = _dev(m)
    print("\nldlq 4096x4096 K=2 against oracle bands", flush=True)
    got = ctx.quantize_matrix_ldlq(w, K, su, sv, torch.from_numpy(L).to(DEV), gss=m.gss,
                                   want_w_hat=True, want_tile_err=True)
    torch.cuda.synchronize()
    assert np.float32(got["scale"]) == scale
    tile_rows = [0, 1, 2, 3, 152, 153, 154, 155]
    rows = np.concatenate([np.arange(16 * t, 16 * t + 16) for t in tile_rows])
    w_reg = oracle.regularize(m.w, m.su, m.sv, 128)
    want = oracle.ldlq(w_reg[rows], L, K, scale)
    packed = _u16(got["packed"]).reshape(R // 16, TC, 16 * K)[tile_rows].reshape(-1, 16 * K)
    assert np.array_equal(packed, want["packed"])
    wh = got["w_hat"].cpu().numpy().reshape(R // 16, TC, 256)[tile_rows].reshape(-1, 256)
    assert np.array_equal(_bits(wh), _bits(oracle.to_tiles(want["what"])))
    err = got["tile_err"].cpu().numpy().reshape(R // 16, TC)[tile_rows].reshape(-1)
    assert np.array_equal(_bits(err), _bits(want["err"]))
