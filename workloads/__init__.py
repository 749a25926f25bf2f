"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers and converts them to the storage dtype.
It contains none of the encoder's arithmetic, so both the oracle and the GPU
library can be fed from it without sharing method code.

The sources quantize real language-model weights; no model or dataset is used
here.  Matrices of the same shapes and value distributions stand in for them:

  1  one 64x64 fp32 matrix, N(0, 1), 64-point Hadamard, K=2, fixed scale 1.0
  2  4096x4096 bf16, N(0, 0.02^2), K=2, scale search
  3  4096x4096 bf16, Student-t(4) scaled to std 0.02, 0.1% of the columns x10
     (chosen from the same seed, applied before bf16 rounding), K=4, scale search
  4  4096x12288 and 12288x4096 bf16, N(0, 0.015^2), K=3, scale search
  5  one transformer layer's projections (q, k, v, o, gate, up, down), bf16,
     N(0, 0.02^2), each at K=2, 3 and 4, scale search

For the out-channel normalization, ``channel_spread`` draws rows of unequal
scale (log-normal spread of the row std) with a few all-zero rows.

Seeds: weights use PCG64(1000 + config), signs PCG64(2000 + config); matrix m of
the layer set uses PCG64(10000 + m) and PCG64(20000 + m).  Signs are drawn as
2*integers(0, 2) - 1.  bf16 values come from torch's round-to-nearest-even cast.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np

LAYER_SHAPES: List[Tuple[str, int, int]] = [
    ("q_proj", 4096, 4096),
    ("k_proj", 4096, 1024),
    ("v_proj", 4096, 1024),
    ("o_proj", 4096, 4096),
    ("gate_proj", 4096, 12288),
    ("up_proj", 4096, 12288),
    ("down_proj", 12288, 4096),
]


@dataclasses.dataclass
class Matrix:
    name: str
    w: np.ndarray            # float32 values (bf16-exact when dtype == "bf16")
    dtype: str               # "f32" or "bf16"
    su: np.ndarray           # float32 +-1, [rows]
    sv: np.ndarray           # float32 +-1, [cols]
    had_block: int
    K: int
    gss: Optional[Tuple[int, float, float]]
    fixed_scale: float = 1.0

    @property
    def shape(self):
        return self.w.shape

    @property
    def n_tiles(self):
        return (self.w.shape[0] // 16) * (self.w.shape[1] // 16)


GSS_DEFAULT = (12, 0.5, 2.0)


def to_bf16_values(w32: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (RNE, via torch) and return the values as float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(w32, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def signs(rng: np.random.Generator, n: int) -> np.ndarray:
    return (2 * rng.integers(0, 2, n) - 1).astype(np.float32)


def gaussian(rows, cols, std, seed_w, seed_s, bf16=True, had_block=128, K=2,
             gss=GSS_DEFAULT, name="w"):
    rw = np.random.Generator(np.random.PCG64(seed_w))
    w = (rw.standard_normal((rows, cols)) * std).astype(np.float32)
    if bf16:
        w = to_bf16_values(w)
    rs = np.random.Generator(np.random.PCG64(seed_s))
    su = signs(rs, rows)
    sv = signs(rs, cols)
    return Matrix(name, w, "bf16" if bf16 else "f32", su, sv, had_block, K, gss)


def heavy_tailed(rows, cols, seed_w, seed_s, K=4, gss=GSS_DEFAULT, name="w"):
    rw = np.random.Generator(np.random.PCG64(seed_w))
    # Student-t with nu=4 has variance 2; scale to std 0.02
    w = (rw.standard_t(4, size=(rows, cols)) * (0.02 / math.sqrt(2.0))).astype(np.float32)
    n_out = int(round(0.001 * cols))
    cols_out = rw.choice(cols, size=n_out, replace=False)
    w[:, cols_out] *= np.float32(10.0)
    w = to_bf16_values(w)
    rs = np.random.Generator(np.random.PCG64(seed_s))
    return Matrix(name, w, "bf16", signs(rs, rows), signs(rs, cols), 128, K, gss)


def channel_spread(rows, cols, seed_w, seed_s, std=0.02, spread=0.5, dead=0.002, K=2,
                   bf16=True, gss=GSS_DEFAULT, name="w"):
    """Rows (output channels) of unequal scale, as trained projections have.

    Row i is N(0, (std * exp(spread * z_i))^2) with z_i ~ N(0, 1); round(dead *
    rows) rows (at least one when dead > 0), chosen from the same seed, are all
    zero (dead channels).  Signs as for the other workloads."""
    rw = np.random.Generator(np.random.PCG64(seed_w))
    row_std = std * np.exp(spread * rw.standard_normal(rows))
    w = (rw.standard_normal((rows, cols)) * row_std[:, None]).astype(np.float32)
    n_dead = max(1, int(round(dead * rows))) if dead > 0 else 0
    w[rw.choice(rows, size=n_dead, replace=False)] = 0.0
    if bf16:
        w = to_bf16_values(w)
    rs = np.random.Generator(np.random.PCG64(seed_s))
    return Matrix(name, w, "bf16" if bf16 else "f32", signs(rs, rows), signs(rs, cols), 128, K,
                  gss)


def config(n: int) -> List[Matrix]:
    """The matrices of workload n (1..5); for 5, K is left at 2 (callers vary it)."""
    if n == 1:
        m = gaussian(64, 64, 1.0, 1001, 2001, bf16=False, had_block=64, K=2, gss=None,
                     name="c1_64x64")
        return [m]
    if n == 2:
        return [gaussian(4096, 4096, 0.02, 1002, 2002, K=2, name="c2_4096x4096")]
    if n == 3:
        return [heavy_tailed(4096, 4096, 1003, 2003, K=4, name="c3_4096x4096_t4")]
    if n == 4:
        # two matrices of one workload: second one draws from the next seeds
        return [gaussian(4096, 12288, 0.015, 1004, 2004, K=3, name="c4_4096x12288"),
                gaussian(12288, 4096, 0.015, 1014, 2014, K=3, name="c4_12288x4096")]
    if n == 5:
        return [gaussian(r, c, 0.02, 10000 + m, 20000 + m, K=2, name=nm)
                for m, (nm, r, c) in enumerate(LAYER_SHAPES)]
    raise ValueError("workloads are numbered 1..5")


def random_tiles(n: int, seed: int, std: float = 1.0) -> np.ndarray:
    """n tile inputs [n, 256] of i.i.d. N(0, std^2) in float32."""
    r = np.random.Generator(np.random.PCG64(seed))
    return (r.standard_normal((n, 256)) * std).astype(np.float32)


def ldl_factor(cols: int, seed: int, off_std: float = 1.0):
    """A synthetic block LDL factorisation H = L D L^T of an input-side Hessian.

    L [cols, cols] float32: identity 16x16 diagonal blocks, i.i.d.
    N(0, off_std^2 / cols) entries in the blocks below the diagonal, zeros above.
    D [cols/16, 16, 16] float64: symmetric positive definite blocks A A^T / 16 + 0.1 I.
    Drawn directly (no Hessian is factorised), seeded with PCG64(seed)."""
    r = np.random.Generator(np.random.PCG64(seed))
    nb = cols // 16
    L = (r.standard_normal((cols, cols)) * (off_std / math.sqrt(cols))).astype(np.float32)
    blk = np.arange(cols) // 16
    L[blk[:, None] <= blk[None, :]] = 0.0
    L[np.arange(cols), np.arange(cols)] = 1.0
    A = r.standard_normal((nb, 16, 16))
    D = A @ A.transpose(0, 2, 1) / 16.0 + 0.1 * np.eye(16)[None]
    return L, D
