"""Thin ctypes binding of libexl3_gfx950.so (names follow include/exl3.h).

Only argument marshalling happens here: torch tensors give device pointers and
the current HIP stream; every step of the encoder runs in the library's
kernels.  There is no CPU fallback -- if the library or a GPU is missing, the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

from . import build as _build

EXL3_OK = 0
EXL3_EINVAL = -1
EXL3_ENOMEM = -2
EXL3_ENONFINITE = -3
EXL3_EHIP = -4
EXL3_EUNSUPPORTED = -5
EXL3_F32 = 0
EXL3_BF16 = 1
EXL3_ROW_MAJOR = 0
EXL3_TILE_MAJOR = 1

EXPORTED = [
    "exl3_version", "exl3_ctx_create", "exl3_ctx_destroy", "exl3_last_error",
    "exl3_ctx_set_stream", "exl3_set_codebook", "exl3_get_codebook", "exl3_set_codebook_kind",
    "exl3_set_tile_order",
    "exl3_regularize", "exl3_unregularize",
    "exl3_channel_normalize", "exl3_encode_tiles", "exl3_encode_tiles_noalloc",
    "exl3_encode_tiles_f16", "exl3_decode_tiles", "exl3_quantize_matrix",
    "exl3_quantize_matrix_ldlq", "exl3_quantize_matrix_grid", "exl3_quantize_matrix_f16", "exl3_scratch_per_tile",
    "exl3_ctx_set_timing", "exl3_ctx_read_timing",
]
CODEBOOK_KINDS = {"mul1": 0, "mcg": 1, "3inst": 2}
KERNEL_KINDS = {"fwd1": 0, "fwd2": 1, "tb1": 2, "tb2": 3, "regularize": 4, "fwd_side": 5,
                "fwd_cost": 6, "channel": 7, "decode": 8}


class Exl3Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("exl3 error %d: %s" % (code, msg))
        self.code = code
        self.msg = msg


class GSS(ctypes.Structure):
    _fields_ = [("iters", ctypes.c_int), ("lo", ctypes.c_double), ("hi", ctypes.c_double)]


class Grid(ctypes.Structure):
    _fields_ = [("coarse_lo", ctypes.c_double), ("coarse_hi", ctypes.c_double),
                ("coarse_step", ctypes.c_double), ("stride", ctypes.c_int),
                ("fine_radius", ctypes.c_double), ("fine_step", ctypes.c_double),
                ("floor", ctypes.c_double)]


GRID_PAGES = (0.1, 1.9, 0.1, 2, 0.075, 0.025, 0.01)


_lib = None


def library_path() -> str:
    return _build.LIB


def load_library():
    """Load the built library (never builds; raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        raise FileNotFoundError(
            "libexl3_gfx950.so is not built; run __graft_entry__.build() or "
            "python trellis_coded_weight_amd/build.py")
    lib = ctypes.CDLL(_build.LIB)
    vp, i32, i64, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_float, ctypes.c_double, ctypes.c_size_t)
    lib.exl3_version.restype = ctypes.c_char_p
    lib.exl3_version.argtypes = []
    lib.exl3_ctx_create.restype = i32
    lib.exl3_ctx_create.argtypes = [ctypes.POINTER(vp), i32, vp, sz]
    lib.exl3_ctx_destroy.restype = None
    lib.exl3_ctx_destroy.argtypes = [vp]
    lib.exl3_last_error.restype = ctypes.c_char_p
    lib.exl3_last_error.argtypes = [vp]
    lib.exl3_ctx_set_stream.restype = i32
    lib.exl3_ctx_set_stream.argtypes = [vp, vp]
    lib.exl3_set_codebook.restype = i32
    lib.exl3_set_codebook.argtypes = [vp, vp]
    lib.exl3_get_codebook.restype = i32
    lib.exl3_set_codebook_kind.restype = i32
    lib.exl3_set_codebook_kind.argtypes = [vp, i32]
    lib.exl3_get_codebook.argtypes = [vp, vp]
    lib.exl3_set_tile_order.restype = i32
    lib.exl3_set_tile_order.argtypes = [vp, vp]
    lib.exl3_regularize.restype = i32
    lib.exl3_regularize.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp]
    lib.exl3_unregularize.restype = i32
    lib.exl3_unregularize.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.exl3_channel_normalize.restype = i32
    lib.exl3_channel_normalize.argtypes = [vp, vp, i32, i32, i32, vp, f64, vp, vp, vp]
    lib.exl3_encode_tiles.restype = i32
    lib.exl3_encode_tiles.argtypes = [vp, vp, i64, i32, f32, vp, vp, vp]
    lib.exl3_encode_tiles_noalloc.restype = i32
    lib.exl3_encode_tiles_noalloc.argtypes = [vp, vp, i64, i32, f32, vp, vp, vp]
    lib.exl3_encode_tiles_f16.restype = i32
    lib.exl3_encode_tiles_f16.argtypes = [vp, vp, i64, i32, vp, vp, vp]
    lib.exl3_decode_tiles.restype = i32
    lib.exl3_decode_tiles.argtypes = [vp, vp, i64, i32, f32, vp]
    lib.exl3_quantize_matrix.restype = i32
    lib.exl3_quantize_matrix.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp,
                                         ctypes.POINTER(GSS), f32, vp, ctypes.POINTER(f32),
                                         ctypes.POINTER(f64), vp, vp]
    lib.exl3_quantize_matrix_ldlq.restype = i32
    lib.exl3_quantize_matrix_ldlq.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp,
                                              ctypes.POINTER(GSS), f32, vp, vp,
                                              ctypes.POINTER(f32), ctypes.POINTER(f64), vp, vp]
    lib.exl3_quantize_matrix_f16.restype = i32
    lib.exl3_quantize_matrix_f16.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp,
                                             ctypes.POINTER(GSS), f32, vp, ctypes.POINTER(f32),
                                             ctypes.POINTER(f64), vp, vp]
    lib.exl3_quantize_matrix_grid.restype = i32
    lib.exl3_quantize_matrix_grid.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp,
                                              ctypes.POINTER(Grid), vp, ctypes.POINTER(f32),
                                              ctypes.POINTER(f64), vp, vp]
    lib.exl3_scratch_per_tile.restype = sz
    lib.exl3_scratch_per_tile.argtypes = [i32]
    lib.exl3_ctx_set_timing.restype = i32
    lib.exl3_ctx_set_timing.argtypes = [vp, i32]
    lib.exl3_ctx_read_timing.restype = i32
    lib.exl3_ctx_read_timing.argtypes = [vp, i32, ctypes.POINTER(f64), ctypes.POINTER(i64),
                                         ctypes.POINTER(i64)]
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, dtype, shape, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


class Context:
    """One library context (scratch, level table) bound to a device."""

    def __init__(self, device: int = 0, scratch_bytes: int = 0):
        if not torch.cuda.is_available():
            raise RuntimeError("the EXL3 encoder needs a GPU; none is visible")
        self.lib = load_library()
        self.device = torch.device("cuda", device)
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            rc = self.lib.exl3_ctx_create(ctypes.byref(h), device,
                                          ctypes.c_void_p(_stream_handle(self.device)),
                                          scratch_bytes)
        if rc != EXL3_OK:
            raise Exl3Error(rc, "context creation failed")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            self.lib.exl3_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    # -- helpers --
    def _sync_stream(self):
        rc = self.lib.exl3_ctx_set_stream(self.handle,
                                          ctypes.c_void_p(_stream_handle(self.device)))
        self._check(rc)

    def _check(self, rc):
        if rc != EXL3_OK:
            raise Exl3Error(rc, self.lib.exl3_last_error(self.handle).decode())

    def last_error(self) -> str:
        return self.lib.exl3_last_error(self.handle).decode()

    def set_timing(self, enable: bool):
        self._sync_stream()
        self._check(self.lib.exl3_ctx_set_timing(self.handle, 1 if enable else 0))

    def read_timing(self, kind: str):
        """(total_ms, launches, tiles) of the recorded launches of one kernel kind."""
        ms = ctypes.c_double()
        nl = ctypes.c_int64()
        nt = ctypes.c_int64()
        self._check(self.lib.exl3_ctx_read_timing(self.handle, KERNEL_KINDS[kind],
                                                  ctypes.byref(ms), ctypes.byref(nl),
                                                  ctypes.byref(nt)))
        return ms.value, nl.value, nt.value

    # -- API --
    def set_codebook(self, levels_fp16: Optional[torch.Tensor]):
        """levels_fp16: host tensor of 65536 float16 values (None restores mul1)."""
        self._sync_stream()
        if levels_fp16 is None:
            return self._check(self.lib.exl3_set_codebook(self.handle, None))
        lv = levels_fp16.detach().cpu().contiguous().view(torch.int16)
        if lv.numel() != 65536:
            raise ValueError("need 65536 levels")
        self._check(self.lib.exl3_set_codebook(self.handle, ctypes.c_void_p(lv.data_ptr())))

    def set_codebook_kind(self, name: str):
        """Select a procedural codebook by name: "mul1", "mcg" or "3inst"."""
        self._sync_stream()
        self._check(self.lib.exl3_set_codebook_kind(self.handle, CODEBOOK_KINDS[name]))

    def set_tile_order(self, order):
        """Within-tile order of tile-major arrays: position t of a tile holds its
        element order[t] (16 * row + col); None restores the natural order."""
        self._sync_stream()
        if order is None:
            return self._check(self.lib.exl3_set_tile_order(self.handle, None))
        o = torch.as_tensor(order, dtype=torch.int64).cpu()
        if o.numel() != 256 or int(o.min()) < 0 or int(o.max()) > 255:
            raise ValueError("a within-tile order has 256 entries in 0..255")
        buf = o.to(torch.uint8).contiguous()
        self._check(self.lib.exl3_set_tile_order(self.handle, ctypes.c_void_p(buf.data_ptr())))

    def get_codebook(self) -> torch.Tensor:
        out = torch.empty(65536, dtype=torch.int16)
        self._sync_stream()
        self._check(self.lib.exl3_get_codebook(self.handle, ctypes.c_void_p(out.data_ptr())))
        return out.view(torch.float16)

    def regularize(self, w: torch.Tensor, su: torch.Tensor, sv: torch.Tensor,
                   had_block: int = 128, tile_major: bool = True):
        """Returns (w_reg float32, tile_sumsq float32 [tiles], nonfinite int32 [1])."""
        rows, cols = w.shape
        dt = {torch.float32: EXL3_F32, torch.bfloat16: EXL3_BF16}.get(w.dtype)
        if dt is None:
            raise ValueError("w must be float32 or bfloat16")
        w = w.contiguous()
        if tile_major:
            out = torch.empty((rows // 16) * (cols // 16), 256, dtype=torch.float32,
                              device=w.device)
        else:
            out = torch.empty(rows, cols, dtype=torch.float32, device=w.device)
        sums = torch.empty((rows // 16) * (cols // 16), dtype=torch.float32, device=w.device)
        flag = torch.zeros(1, dtype=torch.int32, device=w.device)
        self._sync_stream()
        self._check(self.lib.exl3_regularize(
            self.handle, _ptr(w), dt, rows, cols, had_block, _ptr(su.contiguous()),
            _ptr(sv.contiguous()), _ptr(out), EXL3_TILE_MAJOR if tile_major else EXL3_ROW_MAJOR,
            _ptr(sums), _ptr(flag)))
        return out, sums, flag

    def unregularize(self, w_reg: torch.Tensor, rows: int, cols: int, su: torch.Tensor,
                     sv: torch.Tensor, had_block: int = 128, tile_major: bool = True):
        """Inverse regularization of float32 weights (tile-major [tiles, 256] or row-major
        [rows, cols]) -> row-major float32 [rows, cols]."""
        _need(w_reg, torch.float32, tuple(w_reg.shape), "w_reg")
        if w_reg.numel() != rows * cols:
            raise ValueError("w_reg has %d elements, not %d" % (w_reg.numel(), rows * cols))
        out = torch.empty(rows, cols, dtype=torch.float32, device=w_reg.device)
        self._sync_stream()
        self._check(self.lib.exl3_unregularize(
            self.handle, _ptr(w_reg.contiguous()), EXL3_TILE_MAJOR if tile_major else EXL3_ROW_MAJOR,
            rows, cols, had_block, _ptr(su.contiguous()), _ptr(sv.contiguous()), _ptr(out)))
        return out

    def channel_normalize(self, w: torch.Tensor, su: torch.Tensor, floor: float = 0.1):
        """Out-channel RMS normalization: returns (w_norm float32 [rows, cols],
        su_folded float32 [rows], row_rms float64 [rows])."""
        rows, cols = w.shape
        dt = {torch.float32: EXL3_F32, torch.bfloat16: EXL3_BF16}.get(w.dtype)
        if dt is None:
            raise ValueError("w must be float32 or bfloat16")
        w = w.contiguous()
        out = torch.empty(rows, cols, dtype=torch.float32, device=w.device)
        su_f = torch.empty(rows, dtype=torch.float32, device=w.device)
        rms = torch.empty(rows, dtype=torch.float64, device=w.device)
        self._sync_stream()
        self._check(self.lib.exl3_channel_normalize(
            self.handle, _ptr(w), dt, rows, cols, _ptr(su.contiguous()), float(floor), _ptr(out),
            _ptr(su_f), _ptr(rms)))
        return out, su_f, rms

    def encode_tiles(self, x: torch.Tensor, K: int, scale: float, want_states: bool = True,
                     want_sse: bool = True):
        """x float32 [n, 256] -> (packed int16 [n, 16K], states int16 [n, 256] | None,
        sse float32 [n] | None)."""
        n = x.shape[0]
        _need(x, torch.float32, (n, 256), "x")
        packed = torch.empty(n, 16 * K, dtype=torch.int16, device=x.device)
        states = torch.empty(n, 256, dtype=torch.int16, device=x.device) if want_states else None
        sse = torch.empty(n, dtype=torch.float32, device=x.device) if want_sse else None
        self._sync_stream()
        self._check(self.lib.exl3_encode_tiles(self.handle, _ptr(x), n, K, float(scale),
                                               _ptr(packed), _ptr(states), _ptr(sse)))
        return packed, states, sse

    def encode_tiles_noalloc(self, x: torch.Tensor, K: int, scale: float, packed: torch.Tensor,
                             states: Optional[torch.Tensor] = None,
                             sse: Optional[torch.Tensor] = None) -> None:
        """encode_tiles into caller-allocated outputs through the entry point that
        allocates no device memory (at most 256 tiles per call, 512 at K = 4)."""
        n = x.shape[0]
        _need(x, torch.float32, (n, 256), "x")
        _need(packed, torch.int16, (n, 16 * K), "packed")
        if states is not None:
            _need(states, torch.int16, (n, 256), "states")
        if sse is not None:
            _need(sse, torch.float32, (n,), "sse")
        self._sync_stream()
        self._check(self.lib.exl3_encode_tiles_noalloc(self.handle, _ptr(x), n, K, float(scale),
                                                       _ptr(packed), _ptr(states), _ptr(sse)))

    def encode_tiles_f16(self, x: torch.Tensor, K: int, want_states: bool = True,
                         want_cost: bool = True):
        """x float16 [n, 256] -> (packed int16 [n, 16K], states int16 [n, 256] | None,
        cost float16 [n] | None); binary16 arithmetic throughout."""
        n = x.shape[0]
        _need(x, torch.float16, (n, 256), "x")
        packed = torch.empty(n, 16 * K, dtype=torch.int16, device=x.device)
        states = torch.empty(n, 256, dtype=torch.int16, device=x.device) if want_states else None
        cost = torch.empty(n, dtype=torch.float16, device=x.device) if want_cost else None
        self._sync_stream()
        self._check(self.lib.exl3_encode_tiles_f16(self.handle, _ptr(x), n, K, _ptr(packed),
                                                   _ptr(states), _ptr(cost)))
        return packed, states, cost

    def decode_tiles(self, packed: torch.Tensor, K: int, scale: float) -> torch.Tensor:
        n = packed.shape[0]
        _need(packed, torch.int16, (n, 16 * K), "packed")
        out = torch.empty(n, 256, dtype=torch.float32, device=packed.device)
        self._sync_stream()
        self._check(self.lib.exl3_decode_tiles(self.handle, _ptr(packed), n, K, float(scale),
                                               _ptr(out)))
        return out

    def quantize_matrix(self, w: torch.Tensor, K: int, su: torch.Tensor, sv: torch.Tensor,
                        had_block: int = 128,
                        gss: Optional[Tuple[int, float, float]] = (12, 0.5, 2.0),
                        scale: float = 1.0, want_w_hat: bool = False,
                        want_tile_sse: bool = False):
        """Returns dict(packed int16 [R/16, C/16, 16K], scale, mse, w_hat?, tile_sse?)."""
        rows, cols = w.shape
        dt = {torch.float32: EXL3_F32, torch.bfloat16: EXL3_BF16}.get(w.dtype)
        if dt is None:
            raise ValueError("w must be float32 or bfloat16")
        w = w.contiguous()
        dev = w.device
        packed = torch.empty(rows // 16, cols // 16, 16 * K, dtype=torch.int16, device=dev)
        w_hat = (torch.empty((rows // 16) * (cols // 16), 256, dtype=torch.float32, device=dev)
                 if want_w_hat else None)
        tsse = (torch.empty((rows // 16) * (cols // 16), dtype=torch.float32, device=dev)
                if want_tile_sse else None)
        g = None if gss is None else ctypes.byref(GSS(int(gss[0]), float(gss[1]), float(gss[2])))
        s_out = ctypes.c_float(0.0)
        mse = ctypes.c_double(0.0)
        self._sync_stream()
        self._check(self.lib.exl3_quantize_matrix(
            self.handle, _ptr(w), dt, rows, cols, K, had_block, _ptr(su.contiguous()),
            _ptr(sv.contiguous()), g, float(scale), _ptr(packed), ctypes.byref(s_out),
            ctypes.byref(mse), _ptr(w_hat), _ptr(tsse)))
        return {"packed": packed, "scale": s_out.value, "mse": mse.value, "w_hat": w_hat,
                "tile_sse": tsse}

    def quantize_matrix_f16(self, w: torch.Tensor, K: int, su: torch.Tensor, sv: torch.Tensor,
                            had_block: int = 128,
                            gss: Optional[Tuple[int, float, float]] = (12, 0.5, 2.0),
                            scale: float = 1.0, want_w_hat: bool = False,
                            want_tile_sse: bool = False):
        """Whole-matrix path with the binary16 encoder inside the scale search.
        Returns dict(packed int16 [R/16, C/16, 16K], scale, mse, w_hat?, tile_sse?)."""
        rows, cols = w.shape
        dt = {torch.float32: EXL3_F32, torch.bfloat16: EXL3_BF16}.get(w.dtype)
        if dt is None:
            raise ValueError("w must be float32 or bfloat16")
        w = w.contiguous()
        dev = w.device
        packed = torch.empty(rows // 16, cols // 16, 16 * K, dtype=torch.int16, device=dev)
        w_hat = (torch.empty((rows // 16) * (cols // 16), 256, dtype=torch.float32, device=dev)
                 if want_w_hat else None)
        tsse = (torch.empty((rows // 16) * (cols // 16), dtype=torch.float32, device=dev)
                if want_tile_sse else None)
        g = None if gss is None else ctypes.byref(GSS(int(gss[0]), float(gss[1]), float(gss[2])))
        s_out = ctypes.c_float(0.0)
        mse = ctypes.c_double(0.0)
        self._sync_stream()
        self._check(self.lib.exl3_quantize_matrix_f16(
            self.handle, _ptr(w), dt, rows, cols, K, had_block, _ptr(su.contiguous()),
            _ptr(sv.contiguous()), g, float(scale), _ptr(packed), ctypes.byref(s_out),
            ctypes.byref(mse), _ptr(w_hat), _ptr(tsse)))
        return {"packed": packed, "scale": s_out.value, "mse": mse.value, "w_hat": w_hat,
                "tile_sse": tsse}

    def quantize_matrix_grid(self, w: torch.Tensor, K: int, su: torch.Tensor, sv: torch.Tensor,
                             had_block: int = 128, grid: Tuple = GRID_PAGES,
                             want_w_hat: bool = False, want_tile_sse: bool = False):
        """Whole-matrix path with the grid + parabolic scale search.
        Returns dict(packed int16 [R/16, C/16, 16K], scale, mse, w_hat?, tile_sse?)."""
        rows, cols = w.shape
        dt = {torch.float32: EXL3_F32, torch.bfloat16: EXL3_BF16}.get(w.dtype)
        if dt is None:
            raise ValueError("w must be float32 or bfloat16")
        w = w.contiguous()
        dev = w.device
        packed = torch.empty(rows // 16, cols // 16, 16 * K, dtype=torch.int16, device=dev)
        w_hat = (torch.empty((rows // 16) * (cols // 16), 256, dtype=torch.float32, device=dev)
                 if want_w_hat else None)
        tsse = (torch.empty((rows // 16) * (cols // 16), dtype=torch.float32, device=dev)
                if want_tile_sse else None)
        g = Grid(float(grid[0]), float(grid[1]), float(grid[2]), int(grid[3]), float(grid[4]),
                 float(grid[5]), float(grid[6]))
        s_out = ctypes.c_float(0.0)
        mse = ctypes.c_double(0.0)
        self._sync_stream()
        self._check(self.lib.exl3_quantize_matrix_grid(
            self.handle, _ptr(w), dt, rows, cols, K, had_block, _ptr(su.contiguous()),
            _ptr(sv.contiguous()), ctypes.byref(g), _ptr(packed), ctypes.byref(s_out),
            ctypes.byref(mse), _ptr(w_hat), _ptr(tsse)))
        return {"packed": packed, "scale": s_out.value, "mse": mse.value, "w_hat": w_hat,
                "tile_sse": tsse}

    def quantize_matrix_ldlq(self, w: torch.Tensor, K: int, su: torch.Tensor, sv: torch.Tensor,
                             L: torch.Tensor, had_block: int = 128,
                             gss: Optional[Tuple[int, float, float]] = (12, 0.5, 2.0),
                             scale: float = 1.0, want_w_hat: bool = False,
                             want_tile_err: bool = False):
        """LDLQ whole-matrix path; L float32 [cols, cols] on the device.
        Returns dict(packed int16 [R/16, C/16, 16K], scale, mse, w_hat?, tile_err?)."""
        rows, cols = w.shape
        dt = {torch.float32: EXL3_F32, torch.bfloat16: EXL3_BF16}.get(w.dtype)
        if dt is None:
            raise ValueError("w must be float32 or bfloat16")
        _need(L, torch.float32, (cols, cols), "L")
        w = w.contiguous()
        dev = w.device
        packed = torch.empty(rows // 16, cols // 16, 16 * K, dtype=torch.int16, device=dev)
        w_hat = (torch.empty((rows // 16) * (cols // 16), 256, dtype=torch.float32, device=dev)
                 if want_w_hat else None)
        terr = (torch.empty((rows // 16) * (cols // 16), dtype=torch.float32, device=dev)
                if want_tile_err else None)
        g = None if gss is None else ctypes.byref(GSS(int(gss[0]), float(gss[1]), float(gss[2])))
        s_out = ctypes.c_float(0.0)
        mse = ctypes.c_double(0.0)
        self._sync_stream()
        self._check(self.lib.exl3_quantize_matrix_ldlq(
            self.handle, _ptr(w), dt, rows, cols, K, had_block, _ptr(su.contiguous()),
            _ptr(sv.contiguous()), g, float(scale), _ptr(L), _ptr(packed), ctypes.byref(s_out),
            ctypes.byref(mse), _ptr(w_hat), _ptr(terr)))
        return {"packed": packed, "scale": s_out.value, "mse": mse.value, "w_hat": w_hat,
                "tile_err": terr}


def scratch_per_tile(K: int) -> int:
    return int(load_library().exl3_scratch_per_tile(K))


def version() -> str:
    return load_library().exl3_version().decode()


_DEFAULT_CTX = {}


def quantize_matrix(w: torch.Tensor, K: int, su: torch.Tensor, sv: torch.Tensor,
                    had_block: int = 128,
                    gss: Optional[Tuple[int, float, float]] = (12, 0.5, 2.0),
                    scale: float = 1.0):
    """The whole-matrix path as a tuple: (packed int16 [R/16, C/16, 16K], scale,
    mse), on a context per device kept for the process (its scratch is the
    library's default bound).  Context.quantize_matrix takes the same arguments
    and also returns the optional outputs."""
    dev = w.device.index if w.device.index is not None else torch.cuda.current_device()
    ctx = _DEFAULT_CTX.get(dev)
    if ctx is None:
        ctx = _DEFAULT_CTX[dev] = Context(dev)
    out = ctx.quantize_matrix(w, K, su, sv, had_block=had_block, gss=gss, scale=scale)
    return out["packed"], out["scale"], out["mse"]
