"""Inverse regularization of the GPU library against the oracle, through the C ABI.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 7 (decode
order H_l, x su, H_r, x sv; H is its own inverse) and item 8 (channel scales folded into
the sign vector).

Bit-exact against oracle.unregularize for tile-major and row-major inputs, both block
sizes, with +-1 signs and with folded channel scales; end to end, channel normalization ->
quantization -> dequantized tiles -> inverse with the folded signs matches the oracle's
reconstruction bit for bit.
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


@pytest.mark.parametrize("B,tile_major", [(64, True), (64, False), (128, False), (128, True)])
def test_unregularize_bit_exact(ctx, B, tile_major):
    rng = np.random.default_rng(B + tile_major)
    R, C = 2 * B, 3 * B
    w_reg = rng.standard_normal((R, C)).astype(np.float32)
    su = (rng.standard_normal(R) * 0.1).astype(np.float32)
    sv = (2 * rng.integers(0, 2, C) - 1).astype(np.float32)
    want = oracle.unregularize(w_reg, su, sv, B)
    src = oracle.to_tiles(w_reg) if tile_major else w_reg
    got = ctx.unregularize(torch.from_numpy(np.ascontiguousarray(src)).to(DEV), R, C,
                           torch.from_numpy(su).to(DEV), torch.from_numpy(sv).to(DEV),
                           had_block=B, tile_major=tile_major)
    assert np.array_equal(_bits(got.cpu().numpy()), _bits(want))


# Input and output four bytes past a 16-byte boundary (one element per access),
# through the C ABI.
@pytest.mark.parametrize("tile_major", [True, False])
def test_unregularize_unaligned(ctx, tile_major):
    import trellis_coded_weight_amd as T
    B, R, C = 128, 256, 384
    rng = np.random.default_rng(90 + tile_major)
    w_reg = rng.standard_normal((R, C)).astype(np.float32)
    su = (rng.standard_normal(R) * 0.1).astype(np.float32)
    sv = (2 * rng.integers(0, 2, C) - 1).astype(np.float32)
    want = oracle.unregularize(w_reg, su, sv, B)
    src = np.ascontiguousarray(oracle.to_tiles(w_reg) if tile_major else w_reg).reshape(-1)
    ibuf = torch.zeros(R * C + 1, device=DEV)
    ibuf[1:] = torch.from_numpy(src).to(DEV)
    obuf = torch.full((R * C + 1,), -1.0, device=DEV)
    sud, svd = torch.from_numpy(su).to(DEV), torch.from_numpy(sv).to(DEV)
    torch.cuda.synchronize()
    rc = ctx.lib.exl3_unregularize(ctx.handle, ibuf[1:].data_ptr(),
                                   T.EXL3_TILE_MAJOR if tile_major else T.EXL3_ROW_MAJOR, R, C, B,
                                   sud.data_ptr(), svd.data_ptr(), obuf[1:].data_ptr())
    assert rc == 0
    torch.cuda.synchronize()
    assert np.array_equal(_bits(obuf[1:].cpu().numpy()), _bits(want.reshape(-1)))
    assert obuf[0].item() == -1.0


def test_normalize_quantize_reconstruct(ctx):
    m = workloads.channel_spread(128, 256, 71, 72, dead=0.02)
    w_n, su_f, _ = oracle.channel_normalize(m.w, m.su)
    want = oracle.quantize_matrix(w_n, m.su, m.sv, 2, had_block=128, gss=(12, 0.5, 2.0))
    v = oracle.scaled_levels(oracle.mul1_levels_fp16(), want["scale"])
    w_hat = oracle.from_tiles(v[want["states"]], 128, 256)
    want_rec = oracle.unregularize(w_hat, su_f, m.sv, 128)

    su, sv = torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV)
    g_wn, g_suf, _ = ctx.channel_normalize(torch.from_numpy(m.w).to(torch.bfloat16).to(DEV), su)
    got = ctx.quantize_matrix(g_wn, 2, su, sv, want_w_hat=True)
    rec = ctx.unregularize(got["w_hat"], 128, 256, g_suf, sv)
    assert np.array_equal(_bits(rec.cpu().numpy()), _bits(want_rec))
    # the reconstruction is close to the original weights (dead rows exactly zero)
    dead = ~m.w.any(axis=1)
    r = rec.cpu().numpy()
    assert not np.any(r[dead])
    rel = np.linalg.norm(r - m.w) / np.linalg.norm(m.w)
    assert rel < 0.45


def test_rejects_overlap_and_bad_shape(ctx):
    import ctypes
    import trellis_coded_weight_amd as T
    x = torch.zeros(128 * 128, device=DEV)
    s = torch.ones(128, device=DEV)
    ctx._sync_stream()
    rc = ctx.lib.exl3_unregularize(ctx.handle, ctypes.c_void_p(x.data_ptr()), T.EXL3_ROW_MAJOR,
                                   128, 128, 128, ctypes.c_void_p(s.data_ptr()),
                                   ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(x.data_ptr()))
    assert rc == T.EXL3_EINVAL and "overlaps" in ctx.last_error()
    with pytest.raises(T.Exl3Error):
        ctx.unregularize(x.view(128, 128), 128, 128, s, s, had_block=96, tile_major=False)
