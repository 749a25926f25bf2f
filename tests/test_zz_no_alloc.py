"""The allocation-free tile encoder against the allocating one, through the C ABI.

exl3_encode_tiles_noalloc keeps its scratch in a fixed device array; it must
return exactly what exl3_encode_tiles returns (container words, states and
squared errors, bit for bit), on two calls in a row whose second is smaller
(the array keeps the first call's contents), without allocating device memory,
and must reject more tiles than its array holds before any launch.
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_TILES = {1: 256, 2: 256, 3: 256, 4: 512}


@pytest.fixture(scope="module")
def ctx():
    import trellis_coded_weight_amd as T
    c = T.Context(0)
    yield c
    c.close()


def _outputs(n, K):
    return (torch.full((n, 16 * K), -1, dtype=torch.int16, device=DEV),
            torch.full((n, 256), -1, dtype=torch.int16, device=DEV),
            torch.full((n,), -1.0, dtype=torch.float32, device=DEV))


def _same(a, b):
    return np.array_equal(a.cpu().numpy().view(np.uint8), b.cpu().numpy().view(np.uint8))


@pytest.mark.parametrize("K", [2, 3, 4, 1])
def test_noalloc_matches_encode_tiles(ctx, K):
    scale = 1.0
    # first call at the array's capacity, second smaller and ragged
    for n, seed in ((MAX_TILES[K], 700 + K), (37, 800 + K)):
        x = torch.from_numpy(workloads.random_tiles(n, seed)).to(DEV)
        want = ctx.encode_tiles(x, K, scale)
        got = _outputs(n, K)                  # allocated before the free-memory reading
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info(0)[0]
        ctx.encode_tiles_noalloc(x, K, scale, *got)
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info(0)[0]
        print("K=%d n=%d free device bytes %d -> %d" % (K, n, free0, free1), flush=True)
        for g, w, name in zip(got, want, ("packed", "states", "sse")):
            assert _same(g, w), "K=%d n=%d: %s differs from exl3_encode_tiles" % (K, n, name)
        assert free1 == free0, "K=%d n=%d: device memory was allocated" % (K, n)


def test_noalloc_rejects_too_many_tiles(ctx):
    from trellis_coded_weight_amd import Exl3Error
    for K in (2, 4):
        n = MAX_TILES[K] + 1
        x = torch.from_numpy(workloads.random_tiles(n, 900 + K)).to(DEV)
        packed = torch.full((n, 16 * K), 7, dtype=torch.int16, device=DEV)
        with pytest.raises(Exl3Error) as e:
            ctx.encode_tiles_noalloc(x, K, 1.0, packed)
        assert e.value.code == -1 and "exceeds" in e.value.msg
        torch.cuda.synchronize()
        assert bool((packed == 7).all()), "outputs touched by a rejected call"


def test_noalloc_empty_and_outputs_optional(ctx):
    x = torch.empty(0, 256, dtype=torch.float32, device=DEV)
    ctx.encode_tiles_noalloc(x, 2, 1.0, torch.empty(0, 32, dtype=torch.int16, device=DEV))
    x = torch.from_numpy(workloads.random_tiles(5, 950)).to(DEV)
    packed = torch.empty(5, 32, dtype=torch.int16, device=DEV)
    ctx.encode_tiles_noalloc(x, 2, 1.0, packed)
    want = ctx.encode_tiles(x, 2, 1.0, want_states=False, want_sse=False)[0]
    torch.cuda.synchronize()
    assert _same(packed, want)
