"""Out-channel RMS normalization of the GPU library against the oracle, through the C ABI.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 8.

Normalized matrix, folded signs and binary64 row rms bit-exact against
oracle.channel_normalize, for bf16 and fp32 inputs, ragged bands (rows not a
multiple of 16) and ragged column chunks (cols not a multiple of 256), all-zero
rows, and the 4096x4096 size of the projection workload; the normalized matrix
then quantizes bit-exactly like any other input; malformed arguments are rejected.
"""
import ctypes

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


def _bits32(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _check(ctx, m):
    want_w, want_su, want_r = oracle.channel_normalize(m.w, m.su)
    w = torch.from_numpy(m.w).to(torch.bfloat16 if m.dtype == "bf16" else torch.float32).to(DEV)
    got_w, got_su, got_r = ctx.channel_normalize(w, torch.from_numpy(m.su).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(got_r.cpu().numpy().view(np.uint64), want_r.view(np.uint64))
    assert np.array_equal(_bits32(got_su.cpu().numpy()), _bits32(want_su))
    assert np.array_equal(_bits32(got_w.cpu().numpy()), _bits32(want_w))


@pytest.mark.parametrize("rows,cols,bf16,dead", [
    (256, 384, True, 0.01),     # whole bands, one ragged chunk of columns
    (37, 300, False, 0.05),     # ragged last band and ragged chunk, fp32
    (16, 16, True, 0.0),        # one band, one partial chunk
    (5, 1, False, 0.2),         # single column
])
def test_channel_normalize_bit_exact(ctx, rows, cols, bf16, dead):
    print("\nchannel_normalize %dx%d bf16=%s dead=%g" % (rows, cols, bf16, dead), flush=True)
    m = workloads.channel_spread(rows, cols, 300 + rows, 400 + cols, bf16=bf16, dead=dead)
    _check(ctx, m)


def test_all_zero_matrix(ctx):
    w = torch.zeros(32, 64, dtype=torch.bfloat16, device=DEV)
    su = torch.ones(32, dtype=torch.float32, device=DEV)
    w_n, su_f, r = ctx.channel_normalize(w, su)
    assert not torch.any(w_n != 0) and not torch.any(su_f != 0) and not torch.any(r != 0)
    assert not torch.any(torch.signbit(su_f))


@pytest.mark.slow
def test_channel_normalize_4096(ctx):
    print("\nchannel_normalize 4096x4096 bf16", flush=True)
    m = workloads.channel_spread(4096, 4096, 1002, 2002)
    _check(ctx, m)


def test_normalized_matrix_quantizes_like_the_oracle(ctx):
    m = workloads.channel_spread(256, 256, 91, 92, dead=0.01)
    w_n, su_f, _ = oracle.channel_normalize(m.w, m.su)
    want = oracle.quantize_matrix(w_n, m.su, m.sv, 2, had_block=128, gss=(12, 0.5, 2.0))
    got_w, got_su, _ = ctx.channel_normalize(torch.from_numpy(m.w).to(torch.bfloat16).to(DEV),
                                             torch.from_numpy(m.su).to(DEV))
    got = ctx.quantize_matrix(got_w, 2, torch.from_numpy(m.su).to(DEV),
                              torch.from_numpy(m.sv).to(DEV), had_block=128)
    assert np.float32(got["scale"]) == want["scale"]
    assert np.array_equal(got["packed"].cpu().numpy().view(np.uint16).reshape(-1, 32),
                          want["packed"])
    assert np.array_equal(_bits32(got_su.cpu().numpy()), _bits32(su_f))


def test_rejects_malformed_arguments(ctx):
    import trellis_coded_weight_amd as T
    w = torch.randn(32, 64, device=DEV)
    su = torch.ones(32, device=DEV)
    with pytest.raises(T.Exl3Error) as e:
        ctx.channel_normalize(w, su, floor=0.0)
    assert e.value.code == T.EXL3_EINVAL
    bad = su.clone()
    bad[7] = 0.5
    with pytest.raises(T.Exl3Error) as e:
        ctx.channel_normalize(w, bad)
    assert e.value.code == T.EXL3_EINVAL and "su[7]" in e.value.msg
    # in place (w_norm over w) is refused before any launch
    su_f = torch.empty(32, device=DEV)
    ctx._sync_stream()
    rc = ctx.lib.exl3_channel_normalize(ctx.handle, ctypes.c_void_p(w.data_ptr()), T.EXL3_F32,
                                        32, 64, ctypes.c_void_p(su.data_ptr()), 0.1,
                                        ctypes.c_void_p(w.data_ptr()),
                                        ctypes.c_void_p(su_f.data_ptr()), None)
    assert rc == T.EXL3_EINVAL and "overlaps" in ctx.last_error()
