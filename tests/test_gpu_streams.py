"""Stream and device handling of the GPU library, through the C ABI: a context moved to
another stream orders the new stream after the work already enqueued on the old one (the
two share the context's backpointer scratch), so results do not change; a context on a
device that does not exist is refused with EXL3_EHIP.

Source of the requirement: "EXL3 Intel Arc Quantizer" README, Core Implemented
Architecture section 2 (a single stream-ordered scratch arena).
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_switching_streams_keeps_results():
    import trellis_coded_weight_amd as T
    ctx = T.Context(0)
    try:
        x1 = torch.from_numpy(workloads.random_tiles(2048, 31, 1.0)).to(DEV)
        x2 = torch.from_numpy(workloads.random_tiles(2048, 32, 1.0)).to(DEV)
        ref1 = [t.clone() for t in ctx.encode_tiles(x1, 2, 0.9)]
        ref2 = [t.clone() for t in ctx.encode_tiles(x2, 2, 0.9)]
        torch.cuda.synchronize()
        side = torch.cuda.Stream()          # default priority
        out1 = ctx.encode_tiles(x1, 2, 0.9)  # enqueued on the current stream, not awaited
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            out2 = ctx.encode_tiles(x2, 2, 0.9)
        torch.cuda.current_stream().wait_stream(side)
        out3 = ctx.encode_tiles(x1, 2, 0.9)  # and back
        torch.cuda.synchronize()
        for a, b in zip(out1, ref1):
            assert torch.equal(a, b)
        for a, b in zip(out2, ref2):
            assert torch.equal(a, b)
        for a, b in zip(out3, ref1):
            assert torch.equal(a, b)
    finally:
        ctx.close()


def test_context_on_a_missing_device_is_a_hip_error():
    import ctypes
    import trellis_coded_weight_amd as T
    lib = T.load_library()
    h = ctypes.c_void_p(1)
    rc = lib.exl3_ctx_create(ctypes.byref(h), 99, None, 0)
    assert rc == T.EXL3_EHIP and not h.value
    # the device that exists is unaffected
    ctx = T.Context(0)
    try:
        x = torch.from_numpy(workloads.random_tiles(4, 5, 1.0)).to(DEV)
        packed, _, _ = ctx.encode_tiles(x, 2, 1.0)
        torch.cuda.synchronize()
        assert packed.shape == (4, 32)
    finally:
        ctx.close()
