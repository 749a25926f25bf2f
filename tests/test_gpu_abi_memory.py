"""Array arguments the GPU cannot use are rejected at the C ABI before any launch.

Every entry point checks that each array lies inside one allocation the
context's GPU can address (device, managed or pinned host memory) and spans the
bytes the call touches; plain host memory, or a buffer that ends too early,
gives EXL3_EINVAL with the outputs untouched.  Each bad buffer here is made bad
by construction: its allocation's extent is read with hipMemGetAddressRange
first, and the call asks for more than that.
"""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def T():
    import trellis_coded_weight_amd as T
    return T


@pytest.fixture(scope="module")
def ctx(T):
    c = T.Context(0)
    yield c
    c.close()


def _bytes_left(ptr):
    """Bytes from ptr to the end of the allocation holding it."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemGetAddressRange.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    base, size = ctypes.c_void_p(), ctypes.c_size_t()
    assert hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size),
                                     ctypes.c_void_p(ptr)) == 0
    return base.value + size.value - ptr


def _vp(t):
    return ctypes.c_void_p(t.data_ptr())


def test_host_input_rejected(ctx, T):
    x = torch.zeros(4, 256)                                   # host memory
    packed = torch.full((4, 32), 7, dtype=torch.int16, device=DEV)
    rc = ctx.lib.exl3_encode_tiles(ctx.handle, _vp(x), 4, 2, ctypes.c_float(1.0), _vp(packed),
                                   None, None)
    assert rc == T.EXL3_EINVAL
    assert "x" in ctx.last_error() and "host" in ctx.last_error()
    assert bool((packed == 7).all())


def test_input_past_its_allocation_rejected(ctx, T):
    x = torch.zeros(4, 256, device=DEV)
    n = _bytes_left(x.data_ptr()) // 1024 + 1                # one tile more than the allocation
    packed = torch.full((n, 32), 7, dtype=torch.int16, device=DEV)
    rc = ctx.lib.exl3_encode_tiles(ctx.handle, _vp(x), n, 2, ctypes.c_float(1.0), _vp(packed),
                                   None, None)
    assert rc == T.EXL3_EINVAL
    assert "past the end" in ctx.last_error()
    assert bool((packed == 7).all())


def test_output_past_its_allocation_rejected(ctx, T):
    out = torch.full((1, 256), 3.0, device=DEV)
    n = _bytes_left(out.data_ptr()) // 1024 + 1               # one tile more than the allocation
    packed = torch.zeros(n, 32, dtype=torch.int16, device=DEV)
    rc = ctx.lib.exl3_decode_tiles(ctx.handle, _vp(packed), n, 2, ctypes.c_float(1.0), _vp(out))
    assert rc == T.EXL3_EINVAL
    assert "out" in ctx.last_error()
    assert bool((out == 3.0).all())


def test_whole_matrix_host_weights_rejected(ctx, T):
    w = torch.zeros(128, 128)                                 # host memory
    su = torch.ones(128, device=DEV)
    sv = torch.ones(128, device=DEV)
    packed = torch.full((8, 8, 32), 7, dtype=torch.int16, device=DEV)
    s_out = ctypes.c_float(-1.0)
    rc = ctx.lib.exl3_quantize_matrix(ctx.handle, _vp(w), T.EXL3_F32, 128, 128, 2, 128, _vp(su),
                                      _vp(sv), None, ctypes.c_float(1.0), _vp(packed),
                                      ctypes.byref(s_out), None, None, None)
    assert rc == T.EXL3_EINVAL
    assert "w" in ctx.last_error()
    assert s_out.value == -1.0
    assert bool((packed == 7).all())


def test_host_signs_rejected(ctx, T):
    w = torch.zeros(128, 128, device=DEV)
    su = torch.ones(128)                                      # host memory
    sv = torch.ones(128, device=DEV)
    out = torch.full((64, 256), 5.0, device=DEV)
    rc = ctx.lib.exl3_regularize(ctx.handle, _vp(w), T.EXL3_F32, 128, 128, 128, _vp(su),
                                 _vp(sv), _vp(out), T.EXL3_TILE_MAJOR, None, None)
    assert rc == T.EXL3_EINVAL
    assert "su" in ctx.last_error()
    assert bool((out == 5.0).all())


def test_pinned_host_memory_accepted(ctx, T):
    """Pinned host memory is addressable by the GPU: the call runs and matches the
    same call on device memory."""
    x = torch.randn(3, 256).mul_(0.02)
    xp = x.pin_memory()
    p1 = torch.empty(3, 32, dtype=torch.int16, device=DEV)
    rc = ctx.lib.exl3_encode_tiles(ctx.handle, _vp(xp), 3, 2, ctypes.c_float(0.02), _vp(p1),
                                   None, None)
    assert rc == T.EXL3_OK, ctx.last_error()
    p2, _, _ = ctx.encode_tiles(x.to(DEV), 2, 0.02)
    torch.cuda.synchronize()
    assert np.array_equal(p1.cpu().numpy(), p2.cpu().numpy())


def test_device_array_as_host_table_rejected(ctx, T):
    lv = torch.zeros(65536, dtype=torch.int16, device=DEV)
    rc = ctx.lib.exl3_set_codebook(ctx.handle, _vp(lv))
    assert rc == T.EXL3_EINVAL
    assert "device memory" in ctx.last_error()
    # the table in use is unchanged
    got = ctx.get_codebook().numpy().view(np.uint16)
    import oracle
    assert np.array_equal(got, oracle.mul1_levels_fp16().view(np.uint16))
