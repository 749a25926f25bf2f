#!/usr/bin/env python3
"""Throughput of the EXL3 trellis tile encoder on one MI355X.

One step = the whole hot path on one 4096x4096 bf16 weight matrix (entries
N(0, 0.02^2), 128-block Hadamard with random signs, K=2, golden-section scale
search with 12 reductions over [0.5, 2.0] x rms): regularization, per-tile
energy, 14 probe encodes of the 258-tile sample, and the final encode of all
65,536 tiles.  The input is resident in HBM before the timed region.

Prints one JSON line.  `value` is matrix tiles encoded per second.
`roofline` rates the forward (add-compare-select) kernel, which holds almost
all of the time, against the FP32 vector peak; `cpu_baseline` is the oracle on
a bounded sample of the same matrix on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3      # 256 CU x 2.4 GHz x 256 FP32 flop/clk (FMA = 2 flops)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "viterbi_fwd_traffic.json")
FWD_SOURCE = os.path.join(ROOT, "trellis_coded_weight_amd", "csrc", "viterbi_fwd.hip")
METRIC = "encoded 16x16 tiles/sec at K=2/3/4 on 1 MI355X; % of FP32 VALU peak"


def ops_per_pass(K: int, first: bool) -> int:
    """Algorithmic FP32 operations of one forward pass over one tile:
    subtract, multiply and add for each of the 2^16 states at each of the 256
    steps, plus the 2^16 - 2^(16-K) compare-selects that eliminate non-survivors
    at each of the 255 transitions (+ the 2^16 - 1 comparisons of the final
    argmin in the first pass)."""
    n = 1 << 16
    ops = 256 * 3 * n + 255 * (n - (n >> K))
    return ops + (n - 1 if first else 0)


def ops_per_tile_encode(K: int) -> int:
    return ops_per_pass(K, True) + ops_per_pass(K, False)


def sample_size(TR: int, TC: int) -> int:
    # wrapped diagonal + two extremes (at most; the extremes may fall on it)
    return max(TR, TC) + 2


def file_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(K: int):
    """HBM bytes per forward launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != file_sha(FWD_SOURCE):
        return None
    return d.get("per_launch", {}).get("K%d" % K)


def summarize_traffic(fetch_csv, write_csv, copy_mib, out_path=TRAFFIC_FILE):
    """Per-tile HBM bytes of the forward kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for the plain device copy of known size that
    --copy-probe-mib runs first (the largest copy dispatch in the file)."""
    import collections
    import csv

    def per_dispatch(path, counter):
        vals = collections.defaultdict(float)
        meta = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            d = r["Dispatch_Id"]
            vals[d] += float(r["Counter_Value"])
            meta[d] = (r["Kernel_Name"], int(r["Grid_Size"]))
        return vals, meta

    out = {"source_sha256": file_sha(FWD_SOURCE), "per_launch": {}, "calibration": {}}
    per = collections.defaultdict(dict)
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals, meta = per_dispatch(path, counter)
        copies = [(meta[d][1], d) for d in vals if "copyBuffer" in meta[d][0]]
        grid, dcopy = max(copies)                # the probe: the largest copy
        copy_bytes = copy_mib * (1 << 20)          # it reads and writes this much
        scale = copy_bytes / (vals[dcopy] * 1024.0)
        out["calibration"][counter] = {"copy_bytes": copy_bytes,
                                       "counter_kib": vals[dcopy], "scale": scale}
        for d, v in vals.items():
            name, grid = meta[d]
            if "viterbi_fwd_kernel" not in name:
                continue
            k = name.split("viterbi_fwd_kernel<")[1].split(">")[0].replace(" ", "")
            tiles = grid // 1024
            acc = per[k].setdefault(counter, [0.0, 0])
            acc[0] += v * 1024.0 * scale
            acc[1] += tiles
    for k, d in per.items():
        K, pas = k.split(",")
        ent = out["per_launch"].setdefault("K%s" % K, {})
        ent["pass%s" % pas] = {
            "fetch_bytes_per_tile": d["FETCH_SIZE"][0] / d["FETCH_SIZE"][1],
            "write_bytes_per_tile": d["WRITE_SIZE"][0] / d["WRITE_SIZE"][1],
        }
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def host_threads():
    """Worker threads for the oracle: the host cores this process may run on,
    capped by the per-GPU share the host states in OMP_NUM_THREADS (a GPU machine
    here gives one GPU's jobs 16 cores, whatever nproc shows)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


LSCPU_FIELDS = ("Model name", "Vendor ID", "CPU family", "Model", "Stepping", "CPU max MHz",
                "BIOS Model name", "Socket(s)", "Core(s) per socket", "Thread(s) per core")


def cpu_description():
    """The host CPU as lscpu describes it (model name plus the identifying
    fields it prints; /proc/cpuinfo's model name if lscpu is missing)."""
    import subprocess
    info = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in LSCPU_FIELDS and v.strip():
                info[k.strip()] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    if "Model name" not in info:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        info["Model name"] = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    return info


def gss_probes(iters: int) -> int:
    """Sample encodes of a golden-section search with `iters` reductions: the two
    starting points and one new point per reduction except the last, whose
    score the result (the last bracket's midpoint) never reads."""
    return iters + 1


def cpu_baseline(m, K, scale, n_tiles, threads, sample_tiles):
    """Oracle on this host: full regularization and statistics, plus the final
    encode of `sample_tiles` tiles; extrapolated to the whole step."""
    import numpy as np
    import oracle
    levels = oracle.mul1_levels_fp16()
    t0 = time.perf_counter()
    w_reg = oracle.regularize(m.w, m.su, m.sv, m.had_block)
    tiles = oracle.to_tiles(w_reg)
    oracle.tile_sumsq(tiles)
    t_reg = time.perf_counter() - t0
    idx = np.linspace(0, n_tiles - 1, sample_tiles).astype(np.int64)
    t1 = time.perf_counter()
    oracle.encode_tiles(tiles[idx], K, np.float32(scale), levels, threads=threads)
    t_enc = time.perf_counter() - t1
    per_tile = t_enc / sample_tiles
    # one thread on a small slice of the same sample
    n1 = max(1, min(64, sample_tiles // 64))
    t2 = time.perf_counter()
    oracle.encode_tiles(tiles[idx[:n1]], K, np.float32(scale), levels, threads=1)
    per_tile_1 = (time.perf_counter() - t2) / n1
    TR, TC = m.w.shape[0] // 16, m.w.shape[1] // 16
    encodes = n_tiles + gss_probes(m.gss[0]) * sample_size(TR, TC)
    total = t_reg + per_tile * encodes
    return {
        "value": n_tiles / total,
        "unit": "tiles/s",
        "cores": threads,
        "kind": "oracle",
        "sample": ("full regularization + energy of the %dx%d matrix, then the final encode "
                   "of %d evenly spaced tiles at the chosen scale; extrapolated to %d "
                   "tile encodes (all tiles + %d scale-search probes)"
                   % (m.w.shape[0], m.w.shape[1], sample_tiles, encodes, encodes - n_tiles)),
        "measured_s": round(t_reg + t_enc, 2),
        "tile_encodes_per_s": 1.0 / per_tile,
        "single_thread_tile_encodes_per_s": 1.0 / per_tile_1,
        "single_thread_tiles_per_s": n_tiles / (t_reg + per_tile_1 * encodes),
        "nproc": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
        "cpu_model": cpu_description().get("Model name"),
        "lscpu": cpu_description(),
    }


def roofline_line(K, kern, encodes_per_s, steps):
    """The roofline of the dominant kernel: viterbi_fwd_kernel<K, 2>, pass 2 of
    the final encode (launches of 8,192 tiles), rated by its algorithmic
    binary32 operations per tile pass over its measured launch durations.
    Beside it: all forward launches on the library's stream, and the whole
    step's algorithmic operations over the step time (whole_path_frac)."""
    f1_ms, f1_n, f1_tiles = kern["fwd1"]
    f2_ms, f2_n, f2_tiles = kern["fwd2"]
    f3_ms, f3_n, f3_tiles = kern["fwd_cost"]
    ops_unit = ops_per_pass(K, False)
    achieved = f2_tiles * ops_unit / (f2_ms / 1000.0) / 1e12 if f2_ms > 0 else 0.0
    all_ops = ((f1_tiles * ops_per_pass(K, True)) + (f2_tiles + f3_tiles) * ops_unit)
    all_ms = f1_ms + f2_ms + f3_ms
    traffic = None
    per = load_traffic(K)
    if per and "pass2" in per and f2_n:
        traffic = ((per["pass2"]["fetch_bytes_per_tile"] + per["pass2"]["write_bytes_per_tile"])
                   * f2_tiles / f2_n)
    return {
        "bound": "alu",
        "achieved": round(achieved, 3),
        "peak": PEAK_FP32_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
        "traffic": traffic,
        "kernel": "viterbi_fwd_kernel<%d, 2>: forward pass 2 of the final encode" % K,
        "ops_per_tile_pass": ops_unit,
        "launches": f2_n,
        "avg_launch_ms": round(f2_ms / max(f2_n, 1), 4),
        "avg_tiles_per_launch": round(f2_tiles / max(f2_n, 1), 1),
        "all_forward_frac": round(all_ops / (all_ms / 1000.0) / 1e12 / PEAK_FP32_TFLOPS, 4)
                            if all_ms > 0 else None,
        "whole_path_frac": round(encodes_per_s * ops_per_tile_encode(K) / 1e12
                                 / PEAK_FP32_TFLOPS, 4),
        "note": "achieved = ops_per_tile_pass x tiles of the pass-2 launches / the sum of their "
                "durations (HIP events on the library's stream, in a second run of the same "
                "steps; the timed steps ran without events); all_forward_frac covers every "
                "forward launch on that stream (pass 1, pass 2, the probes' cost-only pass)",
    }


def f16_mode(ctx, w, su, sv, scale, n_tiles, steps):
    """Binary16-mode encode of every tile of the same matrix (regularized,
    divided by the chosen scale, rounded to binary16; prepared outside the
    timed region), for K = 1..4; and the whole binary16 path
    (exl3_quantize_matrix_f16: scale search with binary16 probes included).  Rated like the binary32 path: the same
    algorithmic operation count per tile over the forward kernel's own launch
    time, against the same vector peak (a packed binary16 FMA does two lanes'
    work per issue, as dual-issued binary32 does)."""
    import torch
    reg, _, _ = ctx.regularize(w, su, sv, 128)
    xh = (reg / scale).to(torch.float16).contiguous()
    del reg
    res = {"workload": "the 4096x4096 matrix's 65,536 tiles as binary16 (regularized / scale)",
           "tiles_per_s_by_K": {}, "fwd_frac_by_K": {}, "fwd_avg_launch_ms_by_K": {}}
    res["whole_matrix_tiles_per_s_by_K"] = {}
    for K in (2, 3, 4, 1):
        # the whole path (regularize, golden section with binary16 probes, final
        # encode, binary32 errors): exl3_quantize_matrix_f16
        ctx.quantize_matrix_f16(w, K, su, sv)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ctx.quantize_matrix_f16(w, K, su, sv)
        torch.cuda.synchronize()
        res["whole_matrix_tiles_per_s_by_K"][str(K)] = round(n_tiles / (time.perf_counter() - t0), 1)
        ctx.encode_tiles_f16(xh, K, want_states=False, want_cost=True)
        torch.cuda.synchronize()
        ctx.set_timing(True)
        t0 = time.perf_counter()
        for _ in range(max(1, steps // 2)):
            ctx.encode_tiles_f16(xh, K, want_states=False, want_cost=True)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        f1 = ctx.read_timing("fwd1")
        f2 = ctx.read_timing("fwd2")
        ctx.set_timing(False)
        ops = f1[2] * ops_per_pass(K, True) + f2[2] * ops_per_pass(K, False)
        ach = ops / ((f1[0] + f2[0]) / 1000.0) / 1e12
        res["tiles_per_s_by_K"][str(K)] = round(n_tiles * max(1, steps // 2) / dt, 1)
        res["fwd_frac_by_K"][str(K)] = round(ach / PEAK_FP32_TFLOPS, 4)
        res["fwd_avg_launch_ms_by_K"][str(K)] = round((f1[0] + f2[0]) / max(f1[1] + f2[1], 1), 4)
    return res


def ldlq_mode(ctx, m, w, su, sv, steps):
    """The same matrix through exl3_quantize_matrix_ldlq at K = 2 with a synthetic
    block LDL factor of the input-side Hessian (workloads.ldl_factor, drawn once
    and uploaded outside the timed region): scale search, then 256 spans of 256
    tiles quantized from the last to the first with error feedback."""
    import numpy as np
    import torch
    import workloads
    R, C = m.w.shape
    L, _ = workloads.ldl_factor(C, 2102)
    Ld = torch.from_numpy(L).to(w.device)
    out = ctx.quantize_matrix_ldlq(w, 2, su, sv, Ld, gss=m.gss)
    torch.cuda.synchronize()
    n = max(1, steps // 2)
    ctx.set_timing(True)
    t0 = time.perf_counter()
    for _ in range(n):
        out = ctx.quantize_matrix_ldlq(w, 2, su, sv, Ld, gss=m.gss)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    f1 = ctx.read_timing("fwd1")
    f2 = ctx.read_timing("fwd2")
    f3 = ctx.read_timing("fwd_cost")
    ctx.set_timing(False)
    tiles = (R // 16) * (C // 16)
    return {"workload": "the same 4096x4096 matrix, K=2, golden-section scale, LDLQ over 256 "
                        "spans with a synthetic block LDL factor (off-diagonal N(0, 1/4096))",
            "tiles_per_s": round(tiles * n / dt, 1), "ms_per_step": round(1000.0 * dt / n, 3),
            "mse": out["mse"], "scale": out["scale"],
            "fwd_ms_per_step": round((f1[0] + f2[0] + f3[0]) / n, 3)}


def grid_mode(ctx, w, su, sv, n_tiles, steps):
    """The same matrix at K = 2 with the pages' grid + parabolic scale search
    (19 coarse probes on every other sample tile, 7 fine probes on all of them)
    in place of the golden section."""
    import torch
    import trellis_coded_weight_amd as T
    out = ctx.quantize_matrix_grid(w, 2, su, sv, grid=T.GRID_PAGES)
    torch.cuda.synchronize()
    n = max(1, steps // 2)
    t0 = time.perf_counter()
    for _ in range(n):
        out = ctx.quantize_matrix_grid(w, 2, su, sv, grid=T.GRID_PAGES)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    return {"workload": "the same 4096x4096 matrix, K=2, grid {0.1..1.9 step 0.1 on every other "
                        "sample tile; +-0.075 step 0.025 on all; parabolic; floor 0.01}",
            "tiles_per_s": round(n_tiles * n / dt, 1), "ms_per_step": round(1000.0 * dt / n, 3),
            "scale": out["scale"], "mse": out["mse"]}


def codebook_mode(ctx, w, su, sv, n_tiles):
    """The same matrix at K = 2 with the mcg and 3INST level tables (golden
    section; the kernels are the same, only the table differs)."""
    import torch
    out = {}
    for name in ("mcg", "3inst"):
        ctx.set_codebook_kind(name)
        ctx.quantize_matrix(w, 2, su, sv, gss=(12, 0.5, 2.0))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r = ctx.quantize_matrix(w, 2, su, sv, gss=(12, 0.5, 2.0))
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        out[name] = {"tiles_per_s": round(n_tiles / dt, 1), "scale": r["scale"], "mse": r["mse"]}
    ctx.set_codebook_kind("mul1")
    return out


def channel_mode(ctx, n_tiles, steps):
    """Out-channel RMS normalization on a 4096x4096 bf16 matrix whose rows have
    unequal scale (log-normal spread, 0.2% all-zero rows): the normalization
    kernel alone (mean of 20 launches; HBM-bound: 2 B read and 4 B written per
    element), then normalization + K = 2 quantization with the golden section."""
    import torch
    import workloads
    dev = torch.device("cuda", 0)
    m = workloads.channel_spread(4096, 4096, 1002, 2002)
    w = torch.from_numpy(m.w).to(torch.bfloat16).to(dev)
    su, sv = torch.from_numpy(m.su).to(dev), torch.from_numpy(m.sv).to(dev)
    ctx.channel_normalize(w, su)
    # the kernel's own duration: HIP events around each launch on the library's
    # stream (events around the Python call would add the host's call overhead)
    ctx.set_timing(True)
    for _ in range(20):
        ctx.channel_normalize(w, su)
    total, launches, _ = ctx.read_timing("channel")
    ctx.set_timing(False)
    ms = total / launches
    nbytes = 4096 * 4096 * (2 + 4)
    n = max(1, steps // 2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        w_n, su_f, _ = ctx.channel_normalize(w, su)
        out = ctx.quantize_matrix(w_n, 2, su, sv, gss=m.gss)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / n
    return {"workload": "4096x4096 bf16, row std 0.02*exp(0.5 z), 8 all-zero rows; K=2, "
                        "golden-section scale",
            "normalize_ms": round(ms, 4),
            "normalize_gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "normalize_hbm_frac": round(nbytes / (ms * 1e-3) / 8e12, 4),
            "tiles_per_s": round(n_tiles / dt, 1), "scale": out["scale"], "mse": out["mse"]}


def layer_mode(ctx):
    """One transformer layer's seven matrices (q, k, v, o, gate, up, down; 753,664
    tiles, uploaded before timing) quantized back to back on one stream with the
    golden-section search, once at each of K = 2, 3, 4."""
    import torch
    import workloads
    dev = torch.device("cuda", 0)
    mats = []
    for m in workloads.config(5):
        mats.append((torch.from_numpy(m.w).to(torch.bfloat16).to(dev),
                     torch.from_numpy(m.su).to(dev), torch.from_numpy(m.sv).to(dev), m.gss,
                     m.n_tiles))
    tiles = sum(x[4] for x in mats)
    res = {"workload": "q 4096x4096, k/v 4096x1024, o 4096x4096, gate/up 4096x12288, "
                       "down 12288x4096 bf16 N(0, 0.02^2), back to back, golden-section scale",
           "tiles": tiles, "tiles_per_s_by_K": {}, "s_by_K": {}}
    for K in (2, 3, 4):
        ctx.quantize_matrix(mats[1][0], K, mats[1][1], mats[1][2], gss=mats[1][3])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for w, su, sv, gss, _ in mats:
            ctx.quantize_matrix(w, K, su, sv, gss=gss)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        res["tiles_per_s_by_K"][str(K)] = round(tiles / dt, 1)
        res["s_by_K"][str(K)] = round(dt, 3)
    del mats
    return res


def other_workloads(ctx):
    """The remaining workloads at their own K: the 64x64 fp32 matrix at fixed scale
    (latency, median of 100 calls), the heavy-tailed 4096x4096 at K = 4 and the two
    MLP-shaped matrices at K = 3 (golden-section search; inputs uploaded before timing)."""
    import torch
    import workloads
    dev = torch.device("cuda", 0)
    out = {}
    m = workloads.config(1)[0]
    w = torch.from_numpy(m.w).to(dev)
    su, sv = torch.from_numpy(m.su).to(dev), torch.from_numpy(m.sv).to(dev)
    ts = []
    for _ in range(101):
        t0 = time.perf_counter()
        ctx.quantize_matrix(w, m.K, su, sv, had_block=m.had_block, gss=None, scale=m.fixed_scale)
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    med = sorted(ts[1:])[50]
    out["64x64_fp32_k2_fixed_scale"] = {"median_ms": round(1000 * med, 4),
                                        "tiles_per_s": round(m.n_tiles / med, 1)}
    for n, key, reps in ((3, "4096x4096_heavy_tailed_k4", 2), (4, "mlp_4096x12288_12288x4096_k3", 1)):
        mats = [(torch.from_numpy(x.w).to(torch.bfloat16).to(dev), torch.from_numpy(x.su).to(dev),
                 torch.from_numpy(x.sv).to(dev), x) for x in workloads.config(n)]
        ctx.quantize_matrix(mats[0][0], mats[0][3].K, mats[0][1], mats[0][2], gss=mats[0][3].gss)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            for w, su, sv, x in mats:
                ctx.quantize_matrix(w, x.K, su, sv, gss=x.gss)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / reps
        tiles = sum(x.n_tiles for _, _, _, x in mats)
        out[key] = {"tiles": tiles, "s": round(dt, 3), "tiles_per_s": round(tiles / dt, 1)}
        del mats
    return out


def decode_mode(ctx, out, n_tiles):
    """Decode of the final encode's container (all tiles of the matrix at K = 2):
    20 launches timed with the library's events on its stream; algorithmic bytes
    per tile: 64 B of container read, 1 KiB of binary32 values written (the level
    table, 128 KiB, stays in cache)."""
    import torch
    packed = out["packed"].reshape(-1, 32)
    ctx.decode_tiles(packed, 2, out["scale"])
    torch.cuda.synchronize()
    ctx.set_timing(True)
    for _ in range(20):
        ctx.decode_tiles(packed, 2, out["scale"])
    total, launches, _ = ctx.read_timing("decode")
    ctx.set_timing(False)
    ms = total / launches
    nbytes = n_tiles * (64 + 1024)
    return {"workload": "the final encode's container, %d tiles at K=2" % n_tiles,
            "decode_ms": round(ms, 4),
            "decode_gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "decode_hbm_frac": round(nbytes / (ms * 1e-3) / 8e12, 4)}


def run_steps(ctx, w, su, sv, K, gss, steps):
    import torch
    out = None
    for _ in range(steps):
        out = ctx.quantize_matrix(w, K, su, sv, had_block=128, gss=gss)
    torch.cuda.synchronize()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tiles", type=int, default=8192)
    ap.add_argument("--no-other-k", action="store_true",
                    help="skip the K=3, K=4 and K=1 runs and the mcg / 3INST codebook runs "
                         "on the same matrix")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the transformer-layer run (seven matrices at K = 2, 3, 4) and "
                         "the other workloads (64x64, heavy-tailed K=4, MLP K=3)")
    ap.add_argument("--no-grid", action="store_true",
                    help="skip the grid + parabolic scale-search run on the same matrix and "
                         "the out-channel normalization run")
    ap.add_argument("--no-ldlq", action="store_true",
                    help="skip the LDLQ (error feedback) run on the same matrix")
    ap.add_argument("--no-f16", action="store_true",
                    help="skip the binary16-mode encode of the same matrix")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the forward kernel's HBM bytes per tile from two "
                         "rocprofv3 --pmc counter_collection.csv files and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "kernel to scale HBM byte counters against)")
    args = ap.parse_args()

    if args.summarize_traffic:
        if args.copy_probe_mib <= 0:
            sys.exit("--summarize-traffic needs --copy-probe-mib (the probe size used)")
        print(json.dumps(summarize_traffic(*args.summarize_traffic, args.copy_probe_mib),
                         indent=1))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only (the encoder's tiles are independent; sharding "
              "across GPUs is not implemented); --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    import math

    import numpy as np
    import torch
    import trellis_coded_weight_amd as T
    import workloads

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    m = workloads.config(2)[0]
    K = m.K
    R, C = m.w.shape
    n_tiles = (R // 16) * (C // 16)
    w = torch.from_numpy(m.w).to(torch.bfloat16).to(dev)
    su = torch.from_numpy(m.su).to(dev)
    sv = torch.from_numpy(m.sv).to(dev)
    ctx = T.Context(0)
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    out = run_steps(ctx, w, su, sv, K, m.gss, max(args.warmup, 0))
    # the timed region: per-launch timing off
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out = run_steps(ctx, w, su, sv, K, m.gss, args.steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    value = n_tiles * args.steps / dt
    ms_step = 1000.0 * dt / args.steps
    TR, TC = R // 16, C // 16
    gss_encodes = gss_probes(m.gss[0]) * sample_size(TR, TC)
    encodes_per_s = (n_tiles + gss_encodes) * args.steps / dt

    # the same steps again with every launch bracketed by HIP events on the
    # stream it runs on: per-kernel durations for the roofline
    ctx.set_timing(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    run_steps(ctx, w, su, sv, K, m.gss, args.steps)
    torch.cuda.synchronize()
    dt_timed = time.perf_counter() - t1
    kern = {k: ctx.read_timing(k) for k in ("fwd1", "fwd2", "fwd_cost", "tb1", "tb2",
                                             "regularize", "fwd_side")}
    ctx.set_timing(False)
    roofline = roofline_line(K, kern, encodes_per_s, args.steps)
    roofline["instrumented_ms_per_step"] = round(1000.0 * dt_timed / args.steps, 3)
    stages = {k: {"ms": round(v[0] / args.steps, 3), "launches": v[1] // max(args.steps, 1)}
              for k, v in kern.items()}

    by_k = {"2": round(value, 1)}
    if not args.no_other_k:
        for k2 in (3, 4, 1):
            run_steps(ctx, w, su, sv, k2, m.gss, 1)
            t2 = time.perf_counter()
            run_steps(ctx, w, su, sv, k2, m.gss, max(1, args.steps // 2))
            by_k[str(k2)] = round(n_tiles * max(1, args.steps // 2)
                                  / (time.perf_counter() - t2), 1)

    codebooks = None if args.no_other_k else codebook_mode(ctx, w, su, sv, n_tiles)
    f16 = None if args.no_f16 else f16_mode(ctx, w, su, sv, out["scale"], n_tiles, args.steps)
    ldlq = None if args.no_ldlq else ldlq_mode(ctx, m, w, su, sv, args.steps)
    grid = None if args.no_grid else grid_mode(ctx, w, su, sv, n_tiles, args.steps)
    chan = None if args.no_grid else channel_mode(ctx, n_tiles, args.steps)
    dec = decode_mode(ctx, out, n_tiles)
    layer = None if args.no_layer else layer_mode(ctx)
    others = None if args.no_layer else other_workloads(ctx)

    cpu = None
    if not args.no_cpu_baseline and rank == 0:
        threads = host_threads()
        cpu = cpu_baseline(m, K, out["scale"], n_tiles, threads, args.cpu_tiles)

    # ||W - W_hat||_F / ||W||_F: the error is measured in the regularized domain,
    # whose transform is orthonormal, so its norm is the original domain's
    rel_frob = math.sqrt(out["mse"] * R * C / float(np.sum(np.square(m.w, dtype=np.float64))))
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tiles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0, 0.02^2) bf16 matrix; no model weights)",
        "config": {
            "workload": "4096x4096 bf16 projection, N(0,0.02^2), 128-block Hadamard + random "
                        "signs, K=2 trellis encode + 12-iteration golden-section scale search",
            "rows": R, "cols": C, "K": K, "tiles": n_tiles, "had_block": 128,
            "gss": list(m.gss), "scale_search_tile_encodes": gss_encodes,
        },
        "tile_encodes_per_s": round(encodes_per_s, 1),
        "tiles_per_s_by_K": by_k,
        "codebooks_k2": codebooks,
        "scale": out["scale"],
        "mse": out["mse"],
        "rel_frobenius": rel_frob,
        "stages_ms_per_step": stages,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "f16_mode": f16,
        "ldlq_mode": ldlq,
        "grid_search_mode": grid,
        "channel_norm_mode": chan,
        "decode_mode": dec,
        "layer_mode": layer,
        "other_workloads": others,
    }
    if rank == 0:
        print(json.dumps(line), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()
