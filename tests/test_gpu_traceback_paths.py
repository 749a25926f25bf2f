"""The two traceback kernels of the GPU library agree, through the C ABI.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture
section 1 (traceback of the two-pass closure) and section 2 (results must not
depend on how tiles are batched).

Batches of up to 1,024 tiles trace back with one wave per tile and a
speculative walk; larger batches with one lane per tile.  The same tiles
encoded in one call of 1,100 and in two calls of 550 must give identical
states, container words and errors (binary32 and binary16, K = 1..4), and a
sample of tiles must match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N = 1100


@pytest.fixture(scope="module")
def ctx():
    import trellis_coded_weight_amd as T
    c = T.Context(0)
    yield c
    c.close()


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_binary32_one_call_equals_two_calls(ctx, K):
    print("\ntraceback paths binary32 K=%d" % K, flush=True)
    x = workloads.random_tiles(N, 900 + K, std=1.0)
    xd = torch.from_numpy(x).to(DEV)
    scale = 0.9
    big = ctx.encode_tiles(xd, K, scale)
    parts = [ctx.encode_tiles(xd[a:a + N // 2].contiguous(), K, scale) for a in (0, N // 2)]
    for i in range(3):
        whole = big[i].cpu().numpy()
        split = np.concatenate([p[i].cpu().numpy() for p in parts])
        assert np.array_equal(whole.view(np.uint8), split.view(np.uint8)), i
    pick = np.array([0, 1, 549, 550, 551, 1099, 777, 123])
    want = oracle.encode_tiles(x[pick], K, np.float32(scale))
    assert np.array_equal(_u16(big[1])[pick], want["states"])
    assert np.array_equal(_u16(big[0])[pick], want["packed"])
    assert np.array_equal(big[2].cpu().numpy()[pick].view(np.uint32), want["sse"].view(np.uint32))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_binary16_one_call_equals_two_calls(ctx, K):
    print("\ntraceback paths binary16 K=%d" % K, flush=True)
    x = workloads.random_tiles(N, 950 + K, std=1.0).astype(np.float16)
    xd = torch.from_numpy(x).to(DEV)
    big = ctx.encode_tiles_f16(xd, K)
    parts = [ctx.encode_tiles_f16(xd[a:a + N // 2].contiguous(), K) for a in (0, N // 2)]
    for i in range(3):
        whole = big[i].cpu().numpy()
        split = np.concatenate([p[i].cpu().numpy() for p in parts])
        assert np.array_equal(whole.view(np.uint8), split.view(np.uint8)), i
    pick = np.array([0, 549, 550, 1099, 321])
    want = oracle.encode_tiles_f16(x[pick].view(np.uint16), K)
    assert np.array_equal(_u16(big[1])[pick], want["states"])
    assert np.array_equal(_u16(big[0])[pick], want["packed"])
