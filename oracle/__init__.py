"""Python face of the CPU oracle (oracle.c) for the fine-grained FP8 linear.

TEST INFRASTRUCTURE. Only tests/, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this module.  It shares no code with
the HIP library and never calls it.

Arrays are numpy: bf16 inputs as ``uint16``, codes as ``uint8``, scales as
``float32``, GEMM results as ``float64``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64

AXIS_ROW, AXIS_COL = 0, 1
BSCALE_BLOCK, BSCALE_TILE = 0, 1


def _p(arr, ptype):
    return arr.ctypes.data_as(ptype)


def _c(arr, dtype):
    """C-contiguous array of `dtype` (no copy when it already is one)."""
    return np.ascontiguousarray(arr, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _check_positive(s, name):
    s = np.asarray(s)
    if s.size and not np.all(s > 0):
        raise ValueError(f"{name}: scales must be positive")


def _declare(L):
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_e4m3_encode.argtypes = [ctypes.c_float]
    L.orc_e4m3_decode.restype = ctypes.c_double
    L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_encode_array.restype = None
    L.orc_e4m3_encode_array.argtypes = [_f32p, _i64, _u8p]
    L.orc_group_scale.restype = None
    L.orc_group_scale.argtypes = [ctypes.c_float, ctypes.c_int, _f32p, _f32p]
    L.orc_amax_floor.restype = ctypes.c_float
    L.orc_quant_tile.restype = ctypes.c_int
    L.orc_quant_tile.argtypes = [_u16p, _i64, _i64, _i64, ctypes.c_int,
                                 ctypes.c_int, _u8p, _i64, _f32p, _i64]
    L.orc_quant_block.restype = ctypes.c_int
    L.orc_quant_block.argtypes = [_u16p, _i64, _i64, _i64, ctypes.c_int,
                                  _u8p, _i64, _u8p, _i64, _f32p, _i64]
    L.orc_quant_tile_grouped_col.restype = ctypes.c_int
    L.orc_quant_tile_grouped_col.argtypes = [_u16p, _i64, _i64, _i64, ctypes.c_int, _i32p, ctypes.c_int,
                                             _u8p, _i64, _f32p, _i64, ctypes.POINTER(ctypes.c_int64)]
    L.orc_requant_col.restype = ctypes.c_int
    L.orc_requant_col.argtypes = [_u8p, _i64, _i64, _i64, _f32p, _i64,
                                  ctypes.c_int, _u8p, _i64, _f32p, _i64]
    L.orc_gemm.restype = ctypes.c_int
    L.orc_gemm.argtypes = [_i64, _i64, _i64, _u8p, _i64, _f32p, _i64,
                           _u8p, _i64, _f32p, ctypes.c_int, _i64, _i64,
                           _f64p, _i64]
    L.orc_gemm_entries.restype = ctypes.c_int
    L.orc_gemm_entries.argtypes = [_i64, _i64, _i64, _u8p, _i64, _f32p,
                                   _i64, _u8p, _i64, _f32p, ctypes.c_int,
                                   _i64, _i64, _i64, _i64p, _i64p, _f64p]
    L.orc_grouped_gemm.restype = ctypes.c_int
    L.orc_grouped_gemm.argtypes = [ctypes.c_int, _i64, _i64, _i32p, _u8p,
                                   _i64, _f32p, _i64, _u8p, _f32p, _f64p,
                                   _i64]
    L.orc_grouped_gemm_entries.restype = ctypes.c_int
    L.orc_grouped_gemm_entries.argtypes = [ctypes.c_int, _i64, _i64, _i32p,
                                           _u8p, _i64, _f32p, _i64, _u8p,
                                           _f32p, _i64, _i64p, _i64p, _f64p]
    L.orc_gemm_limited.restype = ctypes.c_int
    L.orc_gemm_limited.argtypes = [_i64, _i64, _i64, _u8p, _i64, _f32p, _i64,
                                   _u8p, _i64, _f32p, ctypes.c_int, _i64, _i64,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   _f64p, _i64]
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_set_num_threads.restype = None
    L.orc_set_num_threads.argtypes = [ctypes.c_int]
    return L


class Oracle:
    """The oracle library at `path` (default: oracle/liboracle.so, built on
    first use when missing or older than oracle.c)."""

    def __init__(self, path=None):
        if path is None:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        self.path = path
        self.L = _declare(ctypes.CDLL(path))

    # ---- E4M3 ------------------------------------------------------------

    def encode(self, v):
        """E4M3 codes (uint8) of float32 values: nearest, ties to even,
        saturating."""
        v = _c(v, np.float32)
        out = np.empty(v.shape, np.uint8)
        self.L.orc_e4m3_encode_array(_p(v, _f32p), v.size, _p(out, _u8p))
        return out

    def decode_table(self):
        """float64[256]: exact value of every E4M3 code (NaN for 0x7F, 0xFF)."""
        return np.array([self.L.orc_e4m3_decode(c) for c in range(256)],
                        np.float64)

    def group_scale(self, amax, pow2):
        """(s, inv) for one group's amax, as float32 numpy scalars."""
        s = ctypes.c_float()
        inv = ctypes.c_float()
        self.L.orc_group_scale(ctypes.c_float(amax), int(pow2),
                               ctypes.byref(s), ctypes.byref(inv))
        return np.float32(s.value), np.float32(inv.value)

    def amax_floor(self):
        return np.float32(self.L.orc_amax_floor())

    # ---- quantisers --------------------------------------------------------

    def quant_tile(self, x, axis, pow2):
        """Quantise bf16 bits x[rows, cols] in 1x128 (axis 0) or 128x1
        (axis 1) groups.  Returns (q, s): axis 0 gives q[rows, cols],
        s[cols/128, rows]; axis 1 gives q[cols, rows] (transposed) and
        s[rows/128, cols]."""
        x = _c(x, np.uint16)
        rows, cols = x.shape
        if axis == AXIS_ROW:
            q = np.empty((rows, cols), np.uint8)
            s = np.empty((cols // 128, rows), np.float32)
            ldq, lds = cols, rows
        else:
            q = np.empty((cols, rows), np.uint8)
            s = np.empty((rows // 128, cols), np.float32)
            ldq, lds = rows, cols
        _check(self.L.orc_quant_tile(_p(x, _u16p), rows, cols, cols, axis,
                                     int(pow2), _p(q, _u8p), ldq,
                                     _p(s, _f32p), lds), "quant_tile")
        return q, s

    def quant_block(self, w, pow2, transpose=False):
        """Quantise bf16 bits w[rows, cols] in 128x128 blocks.  Returns
        (q[rows, cols], s[ceil(rows/128), cols/128], qt[cols, rows] or
        None)."""
        w = _c(w, np.uint16)
        rows, cols = w.shape
        q = np.empty((rows, cols), np.uint8)
        s = np.empty(((rows + 127) // 128, cols // 128), np.float32)
        qt = np.empty((cols, rows), np.uint8) if transpose else None
        _check(self.L.orc_quant_block(_p(w, _u16p), rows, cols, cols,
                                      int(pow2), _p(q, _u8p), cols,
                                      _p(qt, _u8p) if transpose else None,
                                      rows, _p(s, _f32p), s.shape[1]),
               "quant_block")
        return q, s, qt

    def quant_tile_grouped_col(self, x, offsets, pow2):
        """128x1 groups restarted at each expert boundary (see oracle.h).
        x: bf16 bits [T, C]; offsets int32 [G+1].  Returns (q [C, Tpad],
        s [Tpad/128, C])."""
        x = _c(x, np.uint16)
        offsets = _c(offsets, np.int32)
        T, C = x.shape
        G = offsets.size - 1
        tpad = int(sum((int(offsets[e + 1] - offsets[e]) + 127) // 128 * 128 for e in range(G)))
        q = np.empty((C, max(tpad, 1)), np.uint8)[:, :tpad]
        q = np.ascontiguousarray(q)
        s = np.empty((tpad // 128, C), np.float32)
        tp = ctypes.c_int64(0)
        _check(self.L.orc_quant_tile_grouped_col(_p(x, _u16p), T, C, C, G, _p(offsets, _i32p), int(pow2),
                                                 _p(q, _u8p), max(tpad, 1), _p(s, _f32p), C, ctypes.byref(tp)),
               "quant_tile_grouped_col")
        assert tp.value == tpad
        return q, s

    def requant_col(self, q, s, pow2):
        """Backward re-tiling: codes q[rows, cols] in 1x128 row groups with
        scales s[cols/128, rows] -> (qt[cols, rows], st[rows/128, cols]) in
        128x1 groups, as quant_tile's axis 1 lays them out."""
        q = _c(q, np.uint8)
        s = _c(s, np.float32)
        rows, cols = q.shape
        qt = np.empty((cols, rows), np.uint8)
        st = np.empty((rows // 128, cols), np.float32)
        _check(self.L.orc_requant_col(_p(q, _u8p), rows, cols, cols,
                                      _p(s, _f32p), s.shape[1], int(pow2),
                                      _p(qt, _u8p), rows, _p(st, _f32p), cols),
               "requant_col")
        return qt, st

    # ---- GEMM --------------------------------------------------------------

    def gemm(self, a, sa, b, sb, bscale_kind, sb_s0, sb_s1):
        """fp64 R[M, N] = sum_g sa[g, m] * SB(n, g) * P_g[m, n] for codes
        a[M, K], b[N, K]; SB as in oracle.h."""
        a = _c(a, np.uint8)
        b = _c(b, np.uint8)
        sa = _c(sa, np.float32)
        sb = _c(sb, np.float32)
        M, K = a.shape
        N = b.shape[0]
        d = np.empty((M, N), np.float64)
        _check(self.L.orc_gemm(M, N, K, _p(a, _u8p), K, _p(sa, _f32p),
                               sa.shape[1], _p(b, _u8p), K, _p(sb, _f32p),
                               bscale_kind, sb_s0, sb_s1, _p(d, _f64p), N),
               "gemm")
        return d

    def gemm_limited(self, a, sa, b, sb, bscale_kind, sb_s0, sb_s1, bits, chunk, interval):
        """The GEMM on a model accumulator with `bits` significant bits
        (chunks of `chunk` products added exactly, then the running sum cut
        toward zero): never promoted (interval 0) or promoted to fp64 every
        `interval` elements.  See oracle.h."""
        a = _c(a, np.uint8)
        b = _c(b, np.uint8)
        sa = _c(sa, np.float32)
        sb = _c(sb, np.float32)
        M, K = a.shape
        N = b.shape[0]
        d = np.empty((M, N), np.float64)
        _check(self.L.orc_gemm_limited(M, N, K, _p(a, _u8p), K, _p(sa, _f32p), sa.shape[1], _p(b, _u8p), K,
                                       _p(sb, _f32p), bscale_kind, sb_s0, sb_s1, int(bits), int(chunk),
                                       int(interval), _p(d, _f64p), N), "gemm_limited")
        return d

    def gemm_entries(self, a, sa, b, sb, bscale_kind, sb_s0, sb_s1, mi, ni):
        """R[mi[i], ni[i]] for each i, as gemm() would give them."""
        a = _c(a, np.uint8)
        b = _c(b, np.uint8)
        sa = _c(sa, np.float32)
        sb = _c(sb, np.float32)
        mi = _c(mi, np.int64)
        ni = _c(ni, np.int64)
        M, K = a.shape
        N = b.shape[0]
        out = np.empty(mi.shape, np.float64)
        _check(self.L.orc_gemm_entries(M, N, K, _p(a, _u8p), K, _p(sa, _f32p),
                                       sa.shape[1], _p(b, _u8p), K,
                                       _p(sb, _f32p), bscale_kind, sb_s0,
                                       sb_s1, mi.size, _p(mi, _i64p),
                                       _p(ni, _i64p), _p(out, _f64p)),
               "gemm_entries")
        return out

    def gemm_abs(self, a, sa, b, sb, bscale_kind, sb_s0, sb_s1):
        """R_abs: the same GEMM over the absolute values of the codes (sign
        bits cleared; the scales are positive), the size of the products
        the error bound of FP8-matrix-core partials is taken against."""
        _check_positive(sa, "sa")
        _check_positive(sb, "sb")
        return self.gemm(_c(a, np.uint8) & np.uint8(0x7F), sa, _c(b, np.uint8) & np.uint8(0x7F), sb,
                         bscale_kind, sb_s0, sb_s1)

    def gemm_abs_entries(self, a, sa, b, sb, bscale_kind, sb_s0, sb_s1, mi, ni):
        _check_positive(sa, "sa")
        _check_positive(sb, "sb")
        return self.gemm_entries(_c(a, np.uint8) & np.uint8(0x7F), sa, _c(b, np.uint8) & np.uint8(0x7F), sb,
                                 bscale_kind, sb_s0, sb_s1, mi, ni)

    def grouped_gemm(self, offsets, a, sa, b, sb):
        """Grouped GEMM over experts: a[rows, K] codes, sa[K/128, ld] scales,
        b[G, N, K] codes, sb[G, N/128, K/128] block scales."""
        offsets = _c(offsets, np.int32)
        a = _c(a, np.uint8)
        sa = _c(sa, np.float32)
        b = _c(b, np.uint8)
        sb = _c(sb, np.float32)
        G, N, K = b.shape
        rows = int(offsets[-1])
        d = np.zeros((rows, N), np.float64)
        _check(self.L.orc_grouped_gemm(G, N, K, _p(offsets, _i32p),
                                       _p(a, _u8p), K, _p(sa, _f32p),
                                       sa.shape[1], _p(b, _u8p),
                                       _p(sb, _f32p), _p(d, _f64p), N),
               "grouped_gemm")
        return d

    def grouped_gemm_abs(self, offsets, a, sa, b, sb):
        """grouped_gemm over the absolute values of the codes."""
        _check_positive(sa, "sa")
        _check_positive(sb, "sb")
        return self.grouped_gemm(offsets, _c(a, np.uint8) & np.uint8(0x7F), sa, _c(b, np.uint8) & np.uint8(0x7F), sb)

    def grouped_gemm_entries(self, offsets, a, sa, b, sb, mi, ni):
        offsets = _c(offsets, np.int32)
        a = _c(a, np.uint8)
        sa = _c(sa, np.float32)
        b = _c(b, np.uint8)
        sb = _c(sb, np.float32)
        mi = _c(mi, np.int64)
        ni = _c(ni, np.int64)
        G, N, K = b.shape
        out = np.empty(mi.shape, np.float64)
        _check(self.L.orc_grouped_gemm_entries(G, N, K, _p(offsets, _i32p),
                                               _p(a, _u8p), K, _p(sa, _f32p),
                                               sa.shape[1], _p(b, _u8p),
                                               _p(sb, _f32p), mi.size,
                                               _p(mi, _i64p), _p(ni, _i64p),
                                               _p(out, _f64p)),
               "grouped_gemm_entries")
        return out

    def num_threads(self):
        return int(self.L.orc_num_threads())

    def set_num_threads(self, n):
        """Threads for later calls (n < 1: back to the default)."""
        self.L.orc_set_num_threads(int(n))


_default = None


def default():
    """The Oracle over oracle/liboracle.so."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def encode(v):
    return default().encode(v)


def decode_table():
    return default().decode_table()


def group_scale(amax, pow2):
    return default().group_scale(amax, pow2)


def amax_floor():
    return default().amax_floor()


def quant_tile(x, axis, pow2):
    return default().quant_tile(x, axis, pow2)


def quant_block(w, pow2, transpose=False):
    return default().quant_block(w, pow2, transpose)


def requant_col(q, s, pow2):
    return default().requant_col(q, s, pow2)


def quant_tile_grouped_col(x, offsets, pow2):
    return default().quant_tile_grouped_col(x, offsets, pow2)


def gemm(a, sa, b, sb, bscale_kind, sb_s0, sb_s1):
    return default().gemm(a, sa, b, sb, bscale_kind, sb_s0, sb_s1)


def gemm_entries(a, sa, b, sb, bscale_kind, sb_s0, sb_s1, mi, ni):
    return default().gemm_entries(a, sa, b, sb, bscale_kind, sb_s0, sb_s1,
                                  mi, ni)


def grouped_gemm(offsets, a, sa, b, sb):
    return default().grouped_gemm(offsets, a, sa, b, sb)


def gemm_limited(a, sa, b, sb, bscale_kind, sb_s0, sb_s1, bits, chunk, interval):
    return default().gemm_limited(a, sa, b, sb, bscale_kind, sb_s0, sb_s1, bits, chunk, interval)


def gemm_abs(a, sa, b, sb, bscale_kind, sb_s0, sb_s1):
    return default().gemm_abs(a, sa, b, sb, bscale_kind, sb_s0, sb_s1)


def grouped_gemm_abs(offsets, a, sa, b, sb):
    return default().grouped_gemm_abs(offsets, a, sa, b, sb)


def grouped_gemm_entries(offsets, a, sa, b, sb, mi, ni):
    return default().grouped_gemm_entries(offsets, a, sa, b, sb, mi, ni)


def num_threads():
    return default().num_threads()


# ---- comparator -----------------------------------------------------------------

from .compare import (TOL, bound_ratio, describe, fp8_partials_bound, gate,  # noqa: E402,F401
                      max_rel_err, measure, normwise_err, passes)
