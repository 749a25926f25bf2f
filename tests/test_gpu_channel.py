"""Out-channel RMS normalization of the GPU library against the oracle, through the C ABI.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 8.

Normalized matrix, folded signs and binary64 row rms bit-exact against
oracle.channel_normalize, for bf16 and fp32 inputs, ragged bands (rows not a
multiple of 16) and ragged column chunks (cols not a multiple of 256), all-zero
rows, and the 4096x4096 size of the projection workload; rows whose sums round at
most additions (values spread over many binades, subnormals, a few tiny values
among large ones), so that the kernel's exact block shortcut is refused and its
one-square-at-a-time path runs; the normalized matrix then quantizes
bit-exactly like any other input; malformed arguments are rejected.
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


def _spread_rows(rows, cols, seed, bf16):
    """Rows whose binary64 sums round often: |values| 2^U(-149, 40) (fp32) or
    2^U(-133, 40) (bf16), random signs; one row of subnormals with every 64th
    value normal of standard deviation 1e-3; one row of N(0, 1) with every 97th value 2^-30."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lo = -149.0 if not bf16 else -133.0
    w = (rng.choice([-1.0, 1.0], (rows, cols)) * np.exp2(rng.uniform(lo, 40.0, (rows, cols))))
    w = w.astype(np.float32)
    w[0] = (rng.standard_normal(cols) * 1e-40).astype(np.float32)
    w[0, ::64] = (rng.standard_normal(len(w[0, ::64])) * 1e-3).astype(np.float32)
    w[1] = rng.standard_normal(cols).astype(np.float32)
    w[1, ::97] = np.float32(2.0 ** -30)
    if bf16:
        w = workloads.to_bf16_values(w)
    su = np.where(rng.random(rows) < 0.5, -1.0, 1.0).astype(np.float32)
    return workloads.Matrix("spread", w, "bf16" if bf16 else "f32", su, np.ones(cols, np.float32),
                            128, 2, None)


# bf16 rows of up to 16 chunks of 64 blocks take the resident-band kernel (up
# to 8 chunks, or up to 16), longer ones and binary32 rows the chunked one
@pytest.mark.parametrize("rows,cols,bf16", [
    (48, 1024, False),          # three whole bands, whole chunks
    (33, 2056, True),           # ragged band, a last chunk of one block (band, 8 chunks)
    (17, 4100, False),          # ragged band and chunk
    (12, 8192, True),           # band kernel, 16 whole chunks
    (9, 6000, True),            # band kernel, 16-chunk form, ragged last chunk and band
    (5, 8200, True),            # 17 chunks: the chunked kernel
])
def test_channel_normalize_rounding_rows(ctx, rows, cols, bf16):
    print("\nchannel_normalize rounding rows %dx%d bf16=%s" % (rows, cols, bf16), flush=True)
    _check(ctx, _spread_rows(rows, cols, 500 + rows, bf16))


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
