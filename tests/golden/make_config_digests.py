"""Write tests/golden/config_digests.json from the oracle alone.

For every matrix of the five workloads (workloads.config) and every K it is
encoded at, this script runs the oracle's whole-matrix path -- regularization,
tile statistics, the golden-section scale search on the tile sample, the final
encode -- and stores what a full GPU run must reproduce bit for bit:

  * the binary32 bits of the chosen scale, the binary64 rms and the search's
    probe trace (scale, objective) in binary64;
  * the SHA-256 of the packed container words (little-endian uint16, tile order
    tr * TC + tc, 16 K words per tile) and of the per-tile squared errors
    (little-endian binary32 bits), and the binary64 mean squared error.

Workloads 1-4 are encoded in full.  Workload 5 (seven projections at K = 2, 3
and 4, 2.4 million tile encodes) stores the exact scale of all 21 runs and the
digests of 1,024 evenly spaced tiles per run (tile i * n // 1024).  With
``--f16`` it also stores the binary16 whole-matrix path's scale on workload 2's
matrix at K = 2 and the digests of 256 evenly spaced tiles.

Nothing here calls the GPU library: the inputs come from ``workloads`` and every
stored value from ``oracle``.  The run takes hours on a few cores, so each
run's scale search and each chunk of its final encode are cached (``--cache``)
and a restarted run resumes where it stopped.

    python tests/golden/make_config_digests.py --threads 8 [--only 2,3] [--f16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "config_digests.json")
CHUNK = 8192
SUBSET_LAYER = 1024
SUBSET_F16 = 256


def strided(n_tiles: int, count: int) -> np.ndarray:
    """count evenly spaced tile indices: i * n_tiles // count."""
    if count >= n_tiles:
        return np.arange(n_tiles, dtype=np.int64)
    return (np.arange(count, dtype=np.int64) * n_tiles) // count


def runs():
    """(key, config number, Matrix, K, subset size or None, binary16 mode) in run order:
    cheap runs first, the two large workload-4 matrices last."""
    out = []
    for n in (1, 2, 3):
        for m in workloads.config(n):
            out.append(("c%d_%s_K%d" % (n, m.name, m.K), n, m, m.K, None, False))
    for m in workloads.config(5):
        for K in (2, 3, 4):
            out.append(("c5_%s_K%d" % (m.name, K), 5, m, K, SUBSET_LAYER, False))
    for m in workloads.config(4):
        out.append(("c4_%s_K%d" % (m.name, m.K), 4, m, m.K, None, False))
    return out


def f16_run():
    m = workloads.config(2)[0]
    return ("f16_c2_%s_K2" % m.name, 2, m, 2, SUBSET_F16, True)


def f32_bits(x) -> str:
    return "0x%08x" % int(np.float32(x).view(np.uint32))


def sha(a: np.ndarray, dtype: str) -> str:
    return hashlib.sha256(np.ascontiguousarray(a, dtype=dtype).tobytes()).hexdigest()


def do_run(spec, cache, threads, log):
    key, n, m, K, subset, f16 = spec
    d = os.path.join(cache, key)
    os.makedirs(d, exist_ok=True)
    R, C = m.w.shape
    n_tiles = m.n_tiles
    gss = m.gss
    qm = oracle.quantize_matrix_f16 if f16 else oracle.quantize_matrix
    enc = oracle.encode_tiles_f16_scaled if f16 else oracle.encode_tiles

    # scale search (cached): the oracle's whole-matrix call with an empty final encode
    t0 = time.time()
    base = qm(m.w, m.su, m.sv, K, had_block=m.had_block, gss=gss, fixed_scale=m.fixed_scale,
              threads=threads, tiles_subset=np.zeros(0, np.int64))
    tiles = base["tiles"]
    scale = np.float32(base["scale"])
    head = {
        "key": key, "config": n, "matrix": m.name, "rows": R, "cols": C, "K": K,
        "dtype": m.dtype, "had_block": m.had_block, "gss": list(gss) if gss else None,
        "fixed_scale": None if gss else float(m.fixed_scale), "binary16_search": f16,
        "codebook": "mul1", "rms": repr(float(base["rms"])), "sample_tiles": len(base["sample"]),
        "scale": float(scale), "scale_bits": f32_bits(scale),
        "trace": [[repr(float(s)), repr(float(f))] for s, f in base["trace"]],
    }
    log("%s: scale %s (%s) after %.0f s" % (key, head["scale"], head["scale_bits"],
                                              time.time() - t0))

    idx = np.arange(n_tiles, dtype=np.int64) if subset is None else strided(n_tiles, subset)
    packed_parts, sse_parts = [], []
    for c0 in range(0, idx.size, CHUNK):
        f = os.path.join(d, "chunk_%07d.npz" % c0)
        sel = idx[c0:c0 + CHUNK]
        if os.path.exists(f):
            z = np.load(f)
            if z["scale_bits"].item() == head["scale_bits"] and z["packed"].shape[0] == sel.size:
                packed_parts.append(z["packed"])
                sse_parts.append(z["sse"])
                continue
        t1 = time.time()
        r = enc(tiles[sel], K, scale, threads=threads)
        np.savez(f + ".tmp.npz", packed=r["packed"], sse=r["sse"],
                 scale_bits=np.array(head["scale_bits"]))
        os.replace(f + ".tmp.npz", f)
        packed_parts.append(r["packed"])
        sse_parts.append(r["sse"])
        log("%s: tiles %d..%d of %d encoded (%.0f tiles/s)"
            % (key, c0, c0 + sel.size - 1, idx.size, sel.size / (time.time() - t1)))
    packed = np.concatenate(packed_parts).astype(np.uint16)
    sse = np.concatenate(sse_parts).astype(np.float32)
    head["tiles"] = "all" if subset is None else {"evenly_spaced": int(idx.size),
                                                  "index": "i * n_tiles // %d" % idx.size}
    head["n_tiles"] = n_tiles
    head["packed_sha256"] = sha(packed, "<u2")
    head["sse_sha256"] = sha(sse, "<f4")
    total = 0.0
    for e in sse.tolist():                    # ascending tile order, binary64
        total += float(e)
    head["sse_sum"] = repr(total)
    head["mse"] = repr(total / (R * C)) if subset is None else None
    # a few raw words, so that a mismatch can be located without the cache
    head["first_tile_packed"] = [int(v) for v in packed[0]]
    head["first_tile_sse_bits"] = f32_bits(sse[0])
    return head


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--threads", type=int, default=oracle.default_threads())
    ap.add_argument("--only", default="", help="comma-separated workload numbers")
    ap.add_argument("--f16", action="store_true", help="also the binary16 whole-matrix run")
    ap.add_argument("--cache", default=os.path.join(os.environ.get("TMPDIR", "/tmp"),
                                                    "exl3_config_digest_cache"))
    ap.add_argument("--out", default=OUT)
    a = ap.parse_args()
    only = {int(s) for s in a.only.split(",") if s}
    specs = [s for s in runs() if not only or s[1] in only]
    if a.f16:
        specs.append(f16_run())

    def log(msg):
        print(time.strftime("%H:%M:%S ") + msg, flush=True)

    doc = {"runs": {}}
    if os.path.exists(a.out):
        with open(a.out) as fh:
            doc = json.load(fh)
    doc["generator"] = "tests/golden/make_config_digests.py (oracle and workloads only)"
    for spec in specs:
        if spec[0] in doc["runs"]:
            log("%s: stored" % spec[0])
            continue
        doc["runs"][spec[0]] = do_run(spec, a.cache, a.threads, log)
        with open(a.out + ".tmp", "w") as fh:
            json.dump(doc, fh, indent=1, sort_keys=True)
        os.replace(a.out + ".tmp", a.out)
    log("done: %d runs in %s" % (len(doc["runs"]), a.out))


if __name__ == "__main__":
    main()
