"""GPU library against the oracle, element by element, through the C ABI.

Bar: bit-exact for states, packed words, backpointer-derived end states,
regularized weights, per-tile energies and squared errors, decoded values and
the scale chosen by the golden-section search (the fixed binary64 summation
order makes it exact, inside the 1e-5 relative bound).
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


def test_level_table_matches_oracle(ctx):
    lv = ctx.get_codebook().numpy().view(np.uint16)
    assert np.array_equal(lv, oracle.mul1_levels_fp16().view(np.uint16))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_encode_tiles_bit_exact(ctx, K):
    n = 37                                   # several workgroups, odd count
    x = workloads.random_tiles(n, 100 + K)
    want = oracle.encode_tiles(x, K, 1.0)
    xd = torch.from_numpy(x).to(DEV)
    packed, states, sse = ctx.encode_tiles(xd, K, 1.0)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(states), want["states"].astype(np.uint16))
    assert np.array_equal(_u16(packed), want["packed"])
    assert np.array_equal(_bits(sse.cpu().numpy()), _bits(want["sse"]))


@pytest.mark.parametrize("K,scale", [(1, 0.31), (2, 0.0173), (3, 2.5), (4, 0.9)])
def test_encode_tiles_scaled_inputs(ctx, K, scale):
    x = workloads.random_tiles(9, 200 + K, std=scale)
    want = oracle.encode_tiles(x, K, scale)
    packed, states, sse = ctx.encode_tiles(torch.from_numpy(x).to(DEV), K, scale)
    assert np.array_equal(_u16(states), want["states"].astype(np.uint16))
    assert np.array_equal(_bits(sse.cpu().numpy()), _bits(want["sse"]))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_edge_inputs(ctx, K):
    """Zeros, a constant tile, huge outliers, tiny (subnormal-producing) values,
    and squared errors past the binary32 range: from the step of an input of
    2e19 every cost is +inf, so every later minimum is a tie among infinities
    and the lowest index decides (at K = 2 the argmin compares {index, cost}
    register pairs as binary64, whose high word is then 0x7F800000)."""
    x = np.zeros((7, 256), np.float32)
    x[1] = 0.37
    x[2, ::17] = 1.0e4
    x[3] = np.float32(1e-20) * np.arange(256, dtype=np.float32)
    x[4] = workloads.random_tiles(1, 5)[0] * np.float32(1e-19)
    x[5] = workloads.random_tiles(1, 6)[0]
    x[5, 200] = 2.0e19
    x[6, ::2] = 2.0e19
    x[6, 1::2] = -2.0e19
    for scale in (1.0, 1e-19):
        want = oracle.encode_tiles(x, K, scale)
        _, states, sse = ctx.encode_tiles(torch.from_numpy(x).to(DEV), K, scale)
        assert np.array_equal(_u16(states), want["states"].astype(np.uint16))
        assert np.array_equal(_bits(sse.cpu().numpy()), _bits(want["sse"]))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_ties_follow_lowest_index(ctx, K):
    """A table with 5 distinct levels: exact ties everywhere; the tie rule decides."""
    rng = np.random.default_rng(K)
    lv = rng.choice(np.array([-1.5, -0.5, 0.0, 0.5, 1.5], np.float16), size=65536)
    x = (np.round(workloads.random_tiles(6, 300 + K) * 2) / 2).astype(np.float32)
    want = oracle.encode_tiles(x, K, 1.0, levels=lv)
    ctx.set_codebook(torch.from_numpy(lv))
    try:
        _, states, sse = ctx.encode_tiles(torch.from_numpy(x).to(DEV), K, 1.0)
        assert np.array_equal(_u16(states), want["states"].astype(np.uint16))
        assert np.array_equal(_bits(sse.cpu().numpy()), _bits(want["sse"]))
    finally:
        ctx.set_codebook(None)


def test_scalar_quantiser_case_on_gpu(ctx):
    K = 2
    lev = np.array([-1.25, -0.375, 0.5, 1.5], np.float16)
    lv = lev[np.arange(65536) & 3]
    x = workloads.random_tiles(4, 9)
    ctx.set_codebook(torch.from_numpy(lv))
    try:
        _, states, _ = ctx.encode_tiles(torch.from_numpy(x).to(DEV), K, 1.0)
    finally:
        ctx.set_codebook(None)
    err = (x[:, :, None] - lev.astype(np.float32)[None, None, :]) ** 2
    assert np.array_equal(_u16(states) & 3, np.argmin(err, axis=2).astype(np.uint16))


@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 8])
def test_decode_matches_oracle(ctx, K):
    rng = np.random.default_rng(K)
    n = 7
    b = rng.integers(0, 1 << K, (n, 256))
    states = np.zeros((n, 256), np.int64)
    for t in range(256):
        s = np.zeros(n, np.int64)
        for j in range(-(16 // K) - 1, 1):
            s = ((s << K) | b[:, (t + j) % 256]) & 0xFFFF
        states[:, t] = s
    packed = oracle.pack_states(states, K)
    v = oracle.scaled_levels(oracle.mul1_levels_fp16(), 0.75)
    out = ctx.decode_tiles(torch.from_numpy(packed.view(np.int16)).to(DEV), K, 0.75)
    assert np.array_equal(_bits(out.cpu().numpy()), _bits(v[states]))


# Arbitrary container words (every word pattern is a container) for 5,000 tiles:
# more than the resident workgroups decode in one round, so workgroups take
# several tiles per wave in turn.
@pytest.mark.parametrize("K", [1, 3, 4])
def test_decode_many_tiles(ctx, K):
    rng = np.random.default_rng(70 + K)
    n = 5000
    words = rng.integers(0, 1 << 16, (n, 16 * K)).astype(np.uint16)
    want = oracle.scaled_levels(oracle.mul1_levels_fp16(), 0.3)[oracle.unpack_states(words, K)]
    out = ctx.decode_tiles(torch.from_numpy(words.view(np.int16)).to(DEV), K, 0.3)
    assert np.array_equal(_bits(out.cpu().numpy()), _bits(want))


# The container and the output off their natural alignment (the container two
# bytes past a 4-byte boundary, the output four bytes past a 16-byte one),
# through the C ABI; 9 tiles, so that the last workgroup is partly empty.
@pytest.mark.parametrize("K", [1, 2, 3, 8])
def test_decode_unaligned_pointers(ctx, K):
    rng = np.random.default_rng(50 + K)
    n = 9
    states = np.zeros((n, 256), np.int64)
    b = rng.integers(0, 1 << K, (n, 256))
    for t in range(256):
        s = np.zeros(n, np.int64)
        for j in range(-(16 // K) - 1, 1):
            s = ((s << K) | b[:, (t + j) % 256]) & 0xFFFF
        states[:, t] = s
    packed = torch.from_numpy(oracle.pack_states(states, K).view(np.int16).reshape(-1))
    pbuf = torch.zeros(packed.numel() + 1, dtype=torch.int16, device=DEV)
    pbuf[1:] = packed.to(DEV)
    obuf = torch.full((n * 256 + 1,), -1.0, device=DEV)
    assert pbuf[1:].data_ptr() % 4 == 2 and obuf[1:].data_ptr() % 16 == 4
    torch.cuda.synchronize()
    rc = ctx.lib.exl3_decode_tiles(ctx.handle, pbuf[1:].data_ptr(), n, K, 0.5,
                                   obuf[1:].data_ptr())
    assert rc == 0
    torch.cuda.synchronize()
    v = oracle.scaled_levels(oracle.mul1_levels_fp16(), 0.5)
    assert np.array_equal(_bits(obuf[1:].cpu().numpy()), _bits(v[states].reshape(-1)))
    assert obuf[0].item() == -1.0


# misaligned: the weights start one element past a 16-byte boundary (the
# kernel then loads one element at a time)
@pytest.mark.parametrize("B,dtype,misaligned", [
    (64, torch.float32, False), (64, torch.bfloat16, False), (128, torch.bfloat16, False),
    (128, torch.float32, False), (64, torch.float32, True), (128, torch.bfloat16, True)])
def test_regularize_bit_exact(ctx, B, dtype, misaligned):
    R, C = 2 * B, 3 * B
    rng = np.random.default_rng(B)
    w = (rng.standard_normal((R, C)) * 0.02).astype(np.float32)
    wt = torch.from_numpy(w).to(dtype)
    w32 = wt.to(torch.float32).numpy()
    su = (2 * rng.integers(0, 2, R) - 1).astype(np.float32)
    sv = (2 * rng.integers(0, 2, C) - 1).astype(np.float32)
    want = oracle.regularize(w32, su, sv, B)
    wd = wt.to(DEV)
    if misaligned:
        buf = torch.zeros(R * C + 1, dtype=dtype, device=DEV)
        buf[1:] = wd.reshape(-1)
        wd = buf[1:].view(R, C)
        assert wd.data_ptr() % 16 != 0
    out, sums, flag = ctx.regularize(wd, torch.from_numpy(su).to(DEV),
                                     torch.from_numpy(sv).to(DEV), B)
    tiles = oracle.to_tiles(want)
    assert np.array_equal(_bits(out.cpu().numpy()), _bits(tiles))
    assert np.array_equal(_bits(sums.cpu().numpy()), _bits(oracle.tile_sumsq(tiles)))
    assert int(flag.item()) == 0
    rm, _, _ = ctx.regularize(wd, torch.from_numpy(su).to(DEV),
                              torch.from_numpy(sv).to(DEV), B, tile_major=False)
    assert np.array_equal(_bits(rm.cpu().numpy()), _bits(want))


# Sign entries other than +-1 (outside the header's contract, which the
# whole-matrix entry points enforce): the result is still the definition's,
# the two products, in every block; lanes whose signs are all +-1 and lanes
# with other values meet in the same blocks.
@pytest.mark.parametrize("B,dtype", [(128, torch.bfloat16), (128, torch.float32),
                                     (64, torch.bfloat16)])
def test_regularize_non_unit_signs(ctx, B, dtype):
    R, C = 2 * B, 2 * B
    rng = np.random.default_rng(100 + B)
    w = torch.from_numpy((rng.standard_normal((R, C)) * 0.02).astype(np.float32)).to(dtype)
    w32 = w.to(torch.float32).numpy()
    su = (2 * rng.integers(0, 2, R) - 1).astype(np.float32)
    sv = (2 * rng.integers(0, 2, C) - 1).astype(np.float32)
    su[[3, B + 17]] = [0.5, -3.0]
    sv[[9, B + 40]] = [1.5, -0.0]
    want = oracle.to_tiles(oracle.regularize(w32, su, sv, B))
    out, sums, flag = ctx.regularize(w.to(DEV), torch.from_numpy(su).to(DEV),
                                     torch.from_numpy(sv).to(DEV), B)
    assert np.array_equal(_bits(out.cpu().numpy()), _bits(want))
    assert np.array_equal(_bits(sums.cpu().numpy()), _bits(oracle.tile_sumsq(want)))
    assert int(flag.item()) == 0


# The non-finite flag: set by one NaN or infinity anywhere (bf16 and fp32
# weights, 16-byte and element-wise loads), left clear by the largest finite
# bf16 values, whose transforms overflow to infinity.
@pytest.mark.parametrize("B,dtype,misaligned", [
    (128, torch.bfloat16, False), (128, torch.float32, False), (64, torch.bfloat16, False),
    (128, torch.bfloat16, True)])
def test_regularize_nonfinite_flag(ctx, B, dtype, misaligned):
    R, C = 2 * B, 3 * B
    su = torch.ones(R, device=DEV)
    sv = -torch.ones(C, device=DEV)

    def flag_of(w):
        wd = w.to(dtype).to(DEV)
        if misaligned:
            buf = torch.zeros(R * C + 1, dtype=dtype, device=DEV)
            buf[1:] = wd.reshape(-1)
            wd = buf[1:].view(R, C)
        return int(ctx.regularize(wd, su, sv, B)[2].item())

    for (r, c) in ((0, 0), (R - 1, C - 1), (B + 5, 2 * B + 3)):
        for bad in (float("inf"), float("-inf"), float("nan")):
            w = torch.zeros(R, C)
            w[r, c] = bad
            assert flag_of(w) == 1, (r, c, bad)
    big = torch.full((R, C), float(torch.finfo(torch.bfloat16).max))
    assert flag_of(big) == 0


def test_workload1_whole_path(ctx):
    m = workloads.config(1)[0]
    want = oracle.quantize_matrix(m.w, m.su, m.sv, m.K, had_block=m.had_block, gss=None,
                                  fixed_scale=1.0)
    got = ctx.quantize_matrix(torch.from_numpy(m.w).to(DEV), m.K,
                              torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV),
                              had_block=m.had_block, gss=None, scale=1.0, want_w_hat=True,
                              want_tile_sse=True)
    assert got["scale"] == 1.0
    assert np.array_equal(_u16(got["packed"]).reshape(-1, 32), want["packed"])
    assert np.array_equal(_bits(got["tile_sse"].cpu().numpy()), _bits(want["sse"]))
    assert got["mse"] == want["mse"]
    v = oracle.scaled_levels(oracle.mul1_levels_fp16(), 1.0)
    assert np.array_equal(_bits(got["w_hat"].cpu().numpy()), _bits(v[want["states"]]))


@pytest.mark.parametrize("K", [1, 2, 4])
def test_small_matrix_with_scale_search(ctx, K):
    m = workloads.gaussian(256, 384, 0.02, 31 + K, 41 + K, K=K)
    want = oracle.quantize_matrix(m.w, m.su, m.sv, K, had_block=128, gss=m.gss)
    got = ctx.quantize_matrix(torch.from_numpy(m.w).to(torch.bfloat16).to(DEV), K,
                              torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV),
                              had_block=128, gss=m.gss, want_tile_sse=True)
    assert abs(got["scale"] - float(want["scale"])) <= 1e-5 * abs(float(want["scale"]))
    assert np.float32(got["scale"]) == want["scale"]
    assert np.array_equal(_u16(got["packed"]).reshape(-1, 16 * K), want["packed"])
    assert np.array_equal(_bits(got["tile_sse"].cpu().numpy()), _bits(want["sse"]))
    assert got["mse"] == want["mse"]


# the scale search runs on the device (one search step per probe): other
# reduction counts and brackets, down to a single reduction, against the
# oracle's golden section
@pytest.mark.parametrize("gss", [(1, 0.5, 2.0), (2, 0.5, 2.0), (3, 0.25, 4.0), (7, 0.9, 1.1)])
def test_scale_search_reductions_and_brackets(ctx, gss):
    m = workloads.gaussian(128, 256, 0.02, 81, 82, K=2)
    print("\nscale search gss=%s" % (gss,), flush=True)
    want = oracle.quantize_matrix(m.w, m.su, m.sv, 2, had_block=128, gss=gss)
    got = ctx.quantize_matrix(torch.from_numpy(m.w).to(torch.bfloat16).to(DEV), 2,
                              torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV),
                              had_block=128, gss=gss, want_tile_sse=True)
    assert np.float32(got["scale"]) == want["scale"]
    assert np.array_equal(_u16(got["packed"]).reshape(-1, 32), want["packed"])
    assert np.array_equal(_bits(got["tile_sse"].cpu().numpy()), _bits(want["sse"]))
    assert got["mse"] == want["mse"]


def test_module_level_quantize_matrix_tuple():
    """trellis_coded_weight_amd.quantize_matrix returns (packed, scale, mse) of the
    same search as the oracle's (a context per device kept for the process)."""
    import trellis_coded_weight_amd as T
    m = workloads.gaussian(256, 256, 0.02, 71, 72, K=2)
    want = oracle.quantize_matrix(m.w, m.su, m.sv, 2, had_block=128, gss=m.gss)
    packed, scale, mse = T.quantize_matrix(torch.from_numpy(m.w).to(torch.bfloat16).to(DEV), 2,
                                           torch.from_numpy(m.su).to(DEV),
                                           torch.from_numpy(m.sv).to(DEV))
    assert np.float32(scale) == want["scale"]
    assert np.array_equal(_u16(packed).reshape(-1, 32), want["packed"])
    assert mse == want["mse"]


@pytest.mark.parametrize("K", [2, 3])
def test_small_matrix_with_grid_search(ctx, K):
    import trellis_coded_weight_amd as T
    m = workloads.gaussian(256, 384, 0.02, 35 + K, 45 + K, K=K)
    want = oracle.quantize_matrix(m.w, m.su, m.sv, K, had_block=128, gss=None,
                                  grid=oracle.GRID_DEFAULT)
    got = ctx.quantize_matrix_grid(torch.from_numpy(m.w).to(torch.bfloat16).to(DEV), K,
                                   torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV),
                                   grid=T.GRID_PAGES, want_tile_sse=True)
    assert np.float32(got["scale"]) == want["scale"]
    assert np.array_equal(_u16(got["packed"]).reshape(-1, 16 * K), want["packed"])
    assert np.array_equal(_bits(got["tile_sse"].cpu().numpy()), _bits(want["sse"]))
    assert got["mse"] == want["mse"]


# The grid search encodes each phase's points as one batch with a scale per
# tile; a scratch bound of seven tiles splits those batches into launches whose
# boundaries fall inside points (each launch then reads its own slice of the
# per-tile scales).
def test_grid_search_with_split_batches():
    import trellis_coded_weight_amd as T
    K = 2
    m = workloads.gaussian(256, 384, 0.02, 61, 62, K=K)
    want = oracle.quantize_matrix(m.w, m.su, m.sv, K, had_block=128, gss=None,
                                  grid=oracle.GRID_DEFAULT)
    with T.Context(0, scratch_bytes=T.scratch_per_tile(K) * 7) as small:
        small.set_timing(True)
        got = small.quantize_matrix_grid(torch.from_numpy(m.w).to(torch.bfloat16).to(DEV), K,
                                         torch.from_numpy(m.su).to(DEV),
                                         torch.from_numpy(m.sv).to(DEV), grid=T.GRID_PAGES,
                                         want_tile_sse=True)
        _, launches, _ = small.read_timing("fwd1")
        small.set_timing(False)
    assert launches > 40
    assert np.float32(got["scale"]) == want["scale"]
    assert np.array_equal(_u16(got["packed"]).reshape(-1, 16 * K), want["packed"])
    assert np.array_equal(_bits(got["tile_sse"].cpu().numpy()), _bits(want["sse"]))
    assert got["mse"] == want["mse"]


def test_grid_rejects_malformed_grid(ctx):
    import trellis_coded_weight_amd as T
    m = workloads.gaussian(128, 128, 0.02, 1, 2, K=2)
    w = torch.from_numpy(m.w).to(torch.bfloat16).to(DEV)
    su, sv = torch.from_numpy(m.su).to(DEV), torch.from_numpy(m.sv).to(DEV)
    for bad in [(0.0, 1.9, 0.1, 2, 0.075, 0.025, 0.01), (0.1, 1.9, 0.0, 2, 0.075, 0.025, 0.01),
                (0.1, 1.9, 0.1, 0, 0.075, 0.025, 0.01), (0.1, 1.9, 0.1, 2, 0.075, 0.025, -1.0)]:
        with pytest.raises(T.Exl3Error) as e:
            ctx.quantize_matrix_grid(w, 2, su, sv, grid=bad)
        assert e.value.code == T.EXL3_EINVAL


def test_batching_does_not_change_results():
    import trellis_coded_weight_amd as T
    x = workloads.random_tiles(11, 77)
    xd = torch.from_numpy(x).to(DEV)
    outs = []
    for scratch in (0, T.scratch_per_tile(2) * 3, T.scratch_per_tile(2)):
        with T.Context(0, scratch_bytes=scratch) as c:
            p, s, e = c.encode_tiles(xd, 2, 1.0)
            torch.cuda.synchronize()
            outs.append((_u16(p), _u16(s), _bits(e.cpu().numpy())))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


def test_failed_scratch_allocation_halves_the_batch():
    """A scratch bound larger than the free device memory: the first allocation fails,
    the batch is halved, and the results equal those of the default context."""
    import trellis_coded_weight_amd as T
    K = 2
    per_tile = T.scratch_per_tile(K)
    free, _ = torch.cuda.mem_get_info()
    n = int(1.25 * free / per_tile) + 1               # one batch would not fit
    print("\nhalving: %d tiles, %.1f GB free" % (n, free / 1e9), flush=True)
    gen = torch.Generator(device=DEV).manual_seed(5)
    x = torch.randn(n, 256, generator=gen, device=DEV)
    with T.Context(0, scratch_bytes=n * per_tile) as big:
        big.set_timing(True)
        p1, _, e1 = big.encode_tiles(x, K, 1.0, want_states=False)
        torch.cuda.synchronize()
        _, launches, tiles = big.read_timing("fwd1")
        big.set_timing(False)
        assert launches >= 2 and tiles == n
        p1, e1 = p1.cpu(), e1.cpu()
    with T.Context(0) as small:
        p2, _, e2 = small.encode_tiles(x, K, 1.0, want_states=False)
        torch.cuda.synchronize()
    assert torch.equal(p1, p2.cpu()) and torch.equal(e1, e2.cpu())


def test_errors_leave_outputs_untouched(ctx):
    import trellis_coded_weight_amd as T
    x = torch.zeros(2, 256, device=DEV)
    with pytest.raises(T.Exl3Error) as e:
        ctx.encode_tiles(x, 5, 1.0)
    assert e.value.code == T.EXL3_EUNSUPPORTED
    with pytest.raises(T.Exl3Error) as e:
        ctx.encode_tiles(x, 0, 1.0)
    assert e.value.code == T.EXL3_EUNSUPPORTED
    with pytest.raises(T.Exl3Error) as e:
        ctx.encode_tiles(x, 2, float("nan"))
    assert e.value.code == T.EXL3_EINVAL
    w = torch.zeros(128, 128, device=DEV)
    su = torch.ones(128, device=DEV)
    bad = su.clone()
    bad[3] = 0.5
    with pytest.raises(T.Exl3Error) as e:
        ctx.quantize_matrix(w, 2, bad, su)
    assert e.value.code == T.EXL3_EINVAL
    with pytest.raises(T.Exl3Error) as e:
        ctx.quantize_matrix(torch.zeros(96, 128, device=DEV), 2, torch.ones(96, device=DEV), su)
    assert e.value.code == T.EXL3_EINVAL
    w2 = w.clone()
    w2[5, 7] = float("inf")
    with pytest.raises(T.Exl3Error) as e:
        ctx.quantize_matrix(w2, 2, su, su)
    assert e.value.code == T.EXL3_ENONFINITE
    with T.Context(0, scratch_bytes=1000) as small:
        packed = torch.full((2, 32), 7, dtype=torch.int16, device=DEV)
        rc = small.lib.exl3_encode_tiles(small.handle, x.data_ptr(), 2, 2, 1.0,
                                         packed.data_ptr(), None, None)
        assert rc == T.EXL3_ENOMEM
        assert bool((packed == 7).all())
    # the context still works after errors
    p, s, e2 = ctx.encode_tiles(x, 2, 1.0)
    want = oracle.encode_tiles(np.zeros((2, 256), np.float32), 2, 1.0)
    assert np.array_equal(_u16(s), want["states"].astype(np.uint16))


def test_zero_matrix_gives_zero_scale(ctx):
    w = torch.zeros(128, 128, device=DEV, dtype=torch.bfloat16)
    su = torch.ones(128, device=DEV)
    got = ctx.quantize_matrix(w, 2, su, su)
    assert got["scale"] == 0.0
    assert bool((got["packed"] == 0).all())


def test_empty_input(ctx):
    x = torch.empty(0, 256, device=DEV)
    p, s, e = ctx.encode_tiles(x, 3, 1.0)
    assert p.shape == (0, 48)
