"""The mcg and 3INST codebooks of the GPU library against the oracle, through the C ABI.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 5
(procedural codebooks mul1, mcg, 3INST; the encoder runs all three).

The library's host generators and the oracle's are separate code: the tables
must agree bit for bit.  With each table loaded, the binary32 and binary16
encoders (states, container words, path costs) and the whole-matrix path with
the golden-section scale search must match the oracle bit for bit.
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
    c.set_codebook_kind("mul1")
    c.close()


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["mcg", "3inst", "mul1"])
def test_table_matches_the_oracle(ctx, name):
    ctx.set_codebook_kind(name)
    got = ctx.get_codebook().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.CODEBOOKS[name]().view(np.uint16))


@pytest.mark.parametrize("name,K", [("mcg", 2), ("3inst", 3), ("mcg", 4), ("3inst", 1)])
def test_encode_with_codebook_bit_exact(ctx, name, K):
    print("\ncodebook %s K=%d" % (name, K), flush=True)
    levels = oracle.CODEBOOKS[name]()
    x = workloads.random_tiles(40, 500 + K, std=1.0)
    scale = np.float32(0.81)
    want = oracle.encode_tiles(x, K, scale, levels=levels)
    ctx.set_codebook_kind(name)
    packed, states, sse = ctx.encode_tiles(torch.from_numpy(x).to(DEV), K, float(scale))
    assert np.array_equal(_u16(states), want["states"])
    assert np.array_equal(_u16(packed), want["packed"])
    assert np.array_equal(sse.cpu().numpy().view(np.uint32), want["sse"].view(np.uint32))


@pytest.mark.parametrize("name,K", [("3inst", 2), ("mcg", 3)])
def test_binary16_encode_with_codebook_bit_exact(ctx, name, K):
    levels = oracle.CODEBOOKS[name]()
    x = (workloads.random_tiles(24, 600 + K, std=1.0)).astype(np.float16)
    want = oracle.encode_tiles_f16(x.view(np.uint16), K, levels=levels)
    ctx.set_codebook_kind(name)
    packed, states, cost = ctx.encode_tiles_f16(torch.from_numpy(x).to(DEV), K)
    assert np.array_equal(_u16(states), want["states"])
    assert np.array_equal(_u16(packed), want["packed"])
    assert np.array_equal(_u16(cost), np.asarray(want["cost"], np.uint16))


@pytest.mark.parametrize("name", ["mcg", "3inst"])
def test_quantize_matrix_with_codebook(ctx, name):
    m = workloads.gaussian(256, 384, 0.02, 700, 701, K=2)
    want = oracle.quantize_matrix(m.w, m.su, m.sv, 2, gss=(12, 0.5, 2.0),
                                  levels=oracle.CODEBOOKS[name]())
    ctx.set_codebook_kind(name)
    got = ctx.quantize_matrix(torch.from_numpy(m.w).to(torch.bfloat16).to(DEV), 2,
                              torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV))
    assert np.float32(got["scale"]) == want["scale"]
    assert np.array_equal(_u16(got["packed"]).reshape(-1, 32), want["packed"])
    assert got["mse"] == want["mse"]


def test_unknown_kind_is_rejected(ctx):
    import trellis_coded_weight_amd as T
    ctx._sync_stream()
    rc = ctx.lib.exl3_set_codebook_kind(ctx.handle, 3)
    assert rc == T.EXL3_EUNSUPPORTED
    ctx.set_codebook_kind("mul1")
    assert np.array_equal(ctx.get_codebook().numpy().view(np.uint16),
                          oracle.mul1_levels_fp16().view(np.uint16))
