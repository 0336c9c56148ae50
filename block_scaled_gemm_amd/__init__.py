"""Python binding of libfp8bs.so: fine-grained FP8 quantisation and the
block-scaled FP8 GEMM on MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of
libfp8bs.so.  PyTorch provides device memory and the current stream.  There
is no fallback: if the library is missing, every call raises.

Functions carry the C names (see include/fp8bs.h for the full contract):

    fp8_cast_e4m3(x)                                -> q
    fp8_quant_tile(x, axis, scale_mode)             -> (q, s)
    fp8_quant_block(w, scale_mode, transpose=False) -> (q, s, qt)
    fp8_quant_dual(x, scale_mode)                   -> (qr, sr, qc, sc)
    fp8_requant_col(q, s, scale_mode)               -> (qt, st)
    fp8_gemm_blockscaled(a, sa, b, sb, bscale_kind, sb_s0, sb_s1, out_dtype) -> d
    fp8_gemm_blockscaled_noalloc(a, sa, b, sb, bscale_kind, sb_s0, sb_s1, d)  -> d
    fp8_grouped_gemm(offsets, a, sa, b, sb, out_dtype, rows_bound=None)    -> d
    fp8_grouped_gemm_strided(offsets, a, sa, G, N, b, ldb, b_estride, sb, ...) -> d

bf16 inputs are ``torch.bfloat16`` tensors (their bit patterns are what the
library reads); codes are ``torch.uint8``; scales ``torch.float32``.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8bs.so")

AXIS_ROW, AXIS_COL = 0, 1
SCALE_FP32, SCALE_POW2 = 0, 1
OUT_BF16, OUT_F32 = 0, 1
BSCALE_BLOCK, BSCALE_TILE = 0, 1
ACCUM_FP32, ACCUM_MFMA8, ACCUM_MFMA8_POW2 = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 16 << 20  # FP8BS_NOALLOC_SCRATCH_BYTES

_lib = None


class FP8BSError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


def lib():
    """The loaded libfp8bs.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m block_scaled_gemm_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.fp8bs_abi_version.restype = i32
        L.fp8bs_abi_version.argtypes = []
        L.fp8bs_status_string.restype = ctypes.c_char_p
        L.fp8bs_status_string.argtypes = [i32]
        L.fp8_cast_e4m3.restype = i32
        L.fp8_cast_e4m3.argtypes = [vp, i64, vp, vp]
        L.fp8_quant_tile.restype = i32
        L.fp8_quant_tile.argtypes = [vp, i64, i64, i64, i32, i32, vp, i64, vp, i64, vp]
        L.fp8_quant_block.restype = i32
        L.fp8_quant_block.argtypes = [vp, i64, i64, i64, i32, vp, i64, vp, i64, vp, i64, vp]
        L.fp8_quant_dual.restype = i32
        L.fp8_quant_dual.argtypes = [vp, i64, i64, i64, i32, vp, i64, vp, i64, vp, i64, vp, i64, vp]
        L.fp8_requant_col.restype = i32
        L.fp8_requant_col.argtypes = [vp, i64, i64, i64, vp, i64, i32, vp, i64, vp, i64, vp]
        L.fp8_gemm_workspace_bytes.restype = ctypes.c_size_t
        L.fp8_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.fp8_gemm_blockscaled.restype = i32
        L.fp8_gemm_blockscaled.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i32,
                                           i64, i64, vp, i64, i32, i32, vp, ctypes.c_size_t, vp]
        L.fp8_gemm_blockscaled_noalloc.restype = i32
        L.fp8_gemm_blockscaled_noalloc.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i32,
                                                   i64, i64, vp, i64, i32, i32, vp]
        L.fp8_grouped_gemm.restype = i32
        L.fp8_grouped_gemm.argtypes = [i32, i64, i64, i64, vp, vp, i64, vp, i64, vp, vp, vp,
                                       i64, i32, i32, vp]
        L.fp8_grouped_gemm_strided.restype = i32
        L.fp8_grouped_gemm_strided.argtypes = [i32, i64, i64, i64, vp, vp, i64, vp, i64, vp, i64, i64, vp, i32,
                                               i64, i64, i64, vp, i64, i32, i32, vp]
        L.fp8_grouped_col_bound.restype = i64
        L.fp8_grouped_col_bound.argtypes = [i64, i32]
        L.fp8_quant_tile_grouped_col.restype = i32
        L.fp8_quant_tile_grouped_col.argtypes = [vp, i64, i64, i64, i32, vp, i32, vp, i64, vp, i64, vp]
        L.fp8_grouped_gemm_kgrouped.restype = i32
        L.fp8_grouped_gemm_kgrouped.argtypes = [i32, i64, i64, i64, vp, vp, i64, vp, i64, vp, i64, vp, i64, vp,
                                                i64, i64, i32, i32, vp]
        L.fp8_scales_are_pow2.restype = i32
        L.fp8_scales_are_pow2.argtypes = [vp, i64, i64, i64, i64, vp, vp]
        L.fp8_gemm_blockscaled_quant.restype = i32
        L.fp8_gemm_blockscaled_quant.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i32, i64, i64, i32,
                                                 vp, i64, vp, i64, i32, vp]
        _lib = L
    return _lib


def status_string(status):
    return lib().fp8bs_status_string(int(status)).decode()


def abi_version():
    return lib().fp8bs_abi_version()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check(rc, what):
    if rc != 0:
        raise FP8BSError(rc, what)


def _dev(t, name, dtype):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() >= 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")


def _ld(t):
    return t.stride(0) if t.dim() == 2 else t.shape[-1]


# ---- quantisation ------------------------------------------------------------------

def fp8_cast_e4m3(x):
    """E4M3 codes of an fp32 tensor (nearest, ties to even, saturating)."""
    _dev(x, "x", torch.float32)
    x = x.contiguous()
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().fp8_cast_e4m3(_ptr(x), x.numel(), _ptr(q), _stream()), "fp8_cast_e4m3")
    return q


def fp8_quant_tile(x, axis=AXIS_ROW, scale_mode=SCALE_FP32, q=None, s=None):
    """1x128 (axis ROW) or 128x1 (axis COL) group quantisation of bf16 x
    [rows, cols].  ROW: q [rows, cols], s [cols/128, rows].  COL: q [cols,
    rows] (transposed), s [rows/128, cols]."""
    _dev(x, "x", torch.bfloat16)
    rows, cols = x.shape
    if axis == AXIS_ROW:
        qs, ss = (rows, cols), (cols // 128, rows)
    else:
        qs, ss = (cols, rows), (rows // 128, cols)
    if q is None:
        q = torch.empty(qs, dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(ss, dtype=torch.float32, device=x.device)
    _check(lib().fp8_quant_tile(_ptr(x), rows, cols, _ld(x), int(axis), int(scale_mode),
                                _ptr(q), _ld(q), _ptr(s), _ld(s), _stream()), "fp8_quant_tile")
    return q, s


def fp8_quant_block(w, scale_mode=SCALE_FP32, transpose=False, q=None, s=None, qt=None):
    """128x128 block quantisation of bf16 w [rows, cols]: q [rows, cols],
    s [ceil(rows/128), cols/128] and, with transpose=True, qt [cols, rows]."""
    _dev(w, "w", torch.bfloat16)
    rows, cols = w.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty(((rows + 127) // 128, cols // 128), dtype=torch.float32, device=w.device)
    if transpose and qt is None:
        # leading dimension padded to a multiple of 16 bytes, as the ABI requires
        ld = (rows + 15) // 16 * 16
        qt = torch.empty((cols, ld), dtype=torch.uint8, device=w.device)[:, :rows]
    _check(lib().fp8_quant_block(_ptr(w), rows, cols, _ld(w), int(scale_mode), _ptr(q), _ld(q),
                                 _ptr(qt) if transpose else None, _ld(qt) if transpose else 0,
                                 _ptr(s), _ld(s), _stream()), "fp8_quant_block")
    return q, s, qt


def fp8_quant_dual(x, scale_mode=SCALE_FP32):
    """Both groupings of bf16 x [rows, cols] from one read: returns
    (qr, sr, qc, sc) equal to fp8_quant_tile(x, ROW) and fp8_quant_tile(x, COL)."""
    _dev(x, "x", torch.bfloat16)
    rows, cols = x.shape
    qr = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    sr = torch.empty((cols // 128, rows), dtype=torch.float32, device=x.device)
    qc = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    sc = torch.empty((rows // 128, cols), dtype=torch.float32, device=x.device)
    _check(lib().fp8_quant_dual(_ptr(x), rows, cols, _ld(x), int(scale_mode), _ptr(qr), _ld(qr), _ptr(sr),
                                _ld(sr), _ptr(qc), _ld(qc), _ptr(sc), _ld(sc), _stream()), "fp8_quant_dual")
    return qr, sr, qc, sc


def grouped_col_bound(T, G):
    return int(lib().fp8_grouped_col_bound(int(T), int(G)))


def fp8_quant_tile_grouped_col(x, offsets, scale_mode=SCALE_FP32):
    """128x1 groups restarted at every expert boundary of the expert-sorted
    tokens x [T, cols] (offsets: int32 device [G+1]).  Returns q [cols, Kb]
    and s [Kb/128, cols] on the padded token axis, Kb = grouped_col_bound(T, G)
    (bytes past the experts' last group are left as allocated)."""
    _dev(x, "x", torch.bfloat16)
    _dev(offsets, "offsets", torch.int32)
    T, cols = x.shape
    G = offsets.numel() - 1
    kb = grouped_col_bound(T, G)
    q = torch.zeros((cols, kb), dtype=torch.uint8, device=x.device)
    s = torch.ones((kb // 128, cols), dtype=torch.float32, device=x.device)
    _check(lib().fp8_quant_tile_grouped_col(_ptr(x), T, cols, _ld(x), G, _ptr(offsets), int(scale_mode), _ptr(q),
                                            _ld(q), _ptr(s), _ld(s), _stream()), "fp8_quant_tile_grouped_col")
    return q, s


def fp8_requant_col(q, s, scale_mode=SCALE_FP32, qt=None, st=None):
    """Backward re-tiling: codes q [rows, cols] in 1x128 row groups with
    scales s [cols/128, rows] (fp8_quant_tile's ROW output) -> qt [cols, rows]
    and st [rows/128, cols] in 128x1 groups (its COL layout)."""
    _dev(q, "q", torch.uint8)
    _dev(s, "s", torch.float32)
    rows, cols = q.shape
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=q.device)
    if st is None:
        st = torch.empty((rows // 128, cols), dtype=torch.float32, device=q.device)
    _check(lib().fp8_requant_col(_ptr(q), rows, cols, _ld(q), _ptr(s), _ld(s), int(scale_mode),
                                 _ptr(qt), _ld(qt), _ptr(st), _ld(st), _stream()), "fp8_requant_col")
    return qt, st


# ---- GEMM -----------------------------------------------------------------------

def gemm_workspace_bytes(M, N, K):
    return int(lib().fp8_gemm_workspace_bytes(M, N, K))


def scales_are_pow2(s, rows=None, cols=None, ld_r=None, ld_c=None):
    """Whether every scale of s is a positive normal power of two (entry
    (r, c) at s[r*ld_r + c*ld_c]; by default the 2-D tensor s itself).
    Synchronises the stream to read the answer.  Any strides (a view of a
    larger array is checked on its own entries)."""
    if not isinstance(s, torch.Tensor) or not s.is_cuda or s.dtype != torch.float32:
        raise TypeError("s must be a float32 CUDA (HIP) tensor")
    if rows is None:
        rows, cols = s.shape
        ld_r, ld_c = s.stride(0), s.stride(1)
    flag = torch.empty(1, dtype=torch.int32, device=s.device)
    _check(lib().fp8_scales_are_pow2(_ptr(s), int(rows), int(cols), int(ld_r), int(ld_c), _ptr(flag), _stream()),
           "fp8_scales_are_pow2")
    return bool(flag.item())


def _check_pow2_mode(accum, sa, a_rows, sb, bscale_kind, sb_s0, sb_s1, n, groups):
    """With FP8BS_CHECK_POW2 set in the environment, refuse the power-of-two
    MFMA mode on scales that are not powers of two (a debugging aid: it
    synchronises the stream)."""
    if accum != ACCUM_MFMA8_POW2 or not os.environ.get("FP8BS_CHECK_POW2"):
        return
    ok = scales_are_pow2(sa, groups, a_rows, _ld(sa), 1)
    if bscale_kind == BSCALE_BLOCK:
        ok = ok and scales_are_pow2(sb, (n + 127) // 128, groups, sb_s0, sb_s1)
    else:
        ok = ok and scales_are_pow2(sb, groups, n, sb_s0, 1)
    if not ok:
        raise ValueError("ACCUM_MFMA8_POW2 with scales that are not powers of two")


def fp8_gemm_blockscaled(a, sa, b, sb, bscale_kind, sb_s0, sb_s1, out_dtype=OUT_BF16, d=None,
                         workspace=None, accum=ACCUM_FP32):
    """D[m,n] = sum_g sa[g,m] * SB(n,g) * sum_{k in g} dec(a[m,k]) dec(b[n,k]).
    a [M, K] and b [N, K] uint8 codes; sa [K/128, >=M] fp32; sb fp32 read as
    SB(n,g) = sb[(n//128)*sb_s0 + g*sb_s1] (BLOCK) or sb[g*sb_s0 + n] (TILE)."""
    _dev(a, "a", torch.uint8)
    _dev(b, "b", torch.uint8)
    _dev(sa, "sa", torch.float32)
    _dev(sb, "sb", torch.float32)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    _check_pow2_mode(accum, sa, M, sb, bscale_kind, sb_s0, sb_s1, N, K // 128)
    dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
    if d is None:
        d = torch.empty((M, N), dtype=dt, device=a.device)
    need = gemm_workspace_bytes(M, N, K)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=a.device)
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(lib().fp8_gemm_blockscaled(M, N, K, _ptr(a), _ld(a), _ptr(sa), _ld(sa), _ptr(b), _ld(b),
                                      _ptr(sb), int(bscale_kind), int(sb_s0), int(sb_s1), _ptr(d),
                                      _ld(d), int(out_dtype), int(accum),
                                      _ptr(workspace) if workspace is not None else None, ws_bytes,
                                      _stream()), "fp8_gemm_blockscaled")
    return d


def fp8_gemm_blockscaled_noalloc(a, sa, b, sb, bscale_kind, sb_s0, sb_s1, d, out_dtype=OUT_BF16,
                                 accum=ACCUM_FP32):
    """fp8_gemm_blockscaled into a caller-allocated d, with no workspace: the
    library's own per-GPU scratch array holds the split-K partials (shapes
    needing more than NOALLOC_SCRATCH_BYTES are rejected).  Calls that
    overlap on one GPU share that array."""
    _dev(a, "a", torch.uint8)
    _dev(b, "b", torch.uint8)
    _dev(sa, "sa", torch.float32)
    _dev(sb, "sb", torch.float32)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    _dev(d, "d", torch.float32 if out_dtype == OUT_F32 else torch.bfloat16)
    _check(lib().fp8_gemm_blockscaled_noalloc(M, N, K, _ptr(a), _ld(a), _ptr(sa), _ld(sa), _ptr(b), _ld(b),
                                              _ptr(sb), int(bscale_kind), int(sb_s0), int(sb_s1), _ptr(d), _ld(d),
                                              int(out_dtype), int(accum), _stream()),
           "fp8_gemm_blockscaled_noalloc")
    return d


def fp8_gemm_blockscaled_quant(a, sa, b, sb, bscale_kind, sb_s0, sb_s1, scale_mode=SCALE_FP32, q=None, s=None,
                               accum=ACCUM_FP32):
    """The GEMM with its bf16 result quantised 1x128 along n in the
    epilogue: returns (q [M, N] codes, s [N/128, M] scales), equal to
    fp8_quant_tile(fp8_gemm_blockscaled(..., OUT_BF16), AXIS_ROW, scale_mode)."""
    _dev(a, "a", torch.uint8)
    _dev(b, "b", torch.uint8)
    _dev(sa, "sa", torch.float32)
    _dev(sb, "sb", torch.float32)
    M, K = a.shape
    N = b.shape[0]
    if q is None:
        q = torch.empty((M, N), dtype=torch.uint8, device=a.device)
    if s is None:
        s = torch.empty((N // 128, M), dtype=torch.float32, device=a.device)
    _check(lib().fp8_gemm_blockscaled_quant(M, N, K, _ptr(a), _ld(a), _ptr(sa), _ld(sa), _ptr(b), _ld(b), _ptr(sb),
                                            int(bscale_kind), int(sb_s0), int(sb_s1), int(scale_mode), _ptr(q),
                                            _ld(q), _ptr(s), _ld(s), int(accum), _stream()),
           "fp8_gemm_blockscaled_quant")
    return q, s


def fp8_grouped_gemm(offsets, a, sa, b, sb, out_dtype=OUT_BF16, rows_bound=None, d=None,
                     accum=ACCUM_FP32):
    """Grouped block-scaled GEMM: rows offsets[e]..offsets[e+1]-1 of a use
    expert e's codes b[e] [N, K] and block scales sb[e] [N/128, K/128].
    offsets is an int32 device tensor; rows_bound defaults to a.shape[0]."""
    _dev(offsets, "offsets", torch.int32)
    _dev(a, "a", torch.uint8)
    _dev(sa, "sa", torch.float32)
    _dev(b, "b", torch.uint8)
    _dev(sb, "sb", torch.float32)
    G, N, K = b.shape
    if not b.is_contiguous() or not sb.is_contiguous():
        raise ValueError("b and sb must be contiguous [G, N, K] / [G, N/128, K/128]")
    rows = a.shape[0] if rows_bound is None else int(rows_bound)
    if accum == ACCUM_MFMA8_POW2 and os.environ.get("FP8BS_CHECK_POW2"):
        # every expert's block scales as one [G*N/128, K/128] array
        if not (scales_are_pow2(sa, K // 128, rows, _ld(sa), 1) and
                scales_are_pow2(sb, G * ((N + 127) // 128), K // 128, K // 128, 1)):
            raise ValueError("ACCUM_MFMA8_POW2 with scales that are not powers of two")
    dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
    if d is None:
        d = torch.empty((rows, N), dtype=dt, device=a.device)
    _check(lib().fp8_grouped_gemm(G, rows, N, K, _ptr(offsets), _ptr(a), _ld(a), _ptr(sa), _ld(sa),
                                  _ptr(b), _ptr(sb), _ptr(d), _ld(d), int(out_dtype), int(accum), _stream()),
           "fp8_grouped_gemm")
    return d


def fp8_grouped_gemm_strided(offsets, a, sa, G, N, b, ldb, b_estride, sb, bscale_kind, sb_s0, sb_s1, sb_estride,
                             out_dtype=OUT_BF16, rows_bound=None, d=None, accum=ACCUM_FP32):
    """Grouped GEMM with strided per-expert B codes and scales (see
    include/fp8bs.h): rows offsets[e]..offsets[e+1]-1 of a use codes at
    b + e*b_estride (rows ldb apart) and scales at sb + e*sb_estride.  b and
    sb are flat device tensors holding every expert."""
    _dev(offsets, "offsets", torch.int32)
    _dev(a, "a", torch.uint8)
    _dev(sa, "sa", torch.float32)
    _dev(b, "b", torch.uint8)
    _dev(sb, "sb", torch.float32)
    K = a.shape[1]
    rows = a.shape[0] if rows_bound is None else int(rows_bound)
    dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
    if d is None:
        d = torch.empty((rows, N), dtype=dt, device=a.device)
    _check(lib().fp8_grouped_gemm_strided(int(G), rows, int(N), K, _ptr(offsets), _ptr(a), _ld(a), _ptr(sa), _ld(sa),
                                          _ptr(b), int(ldb), int(b_estride), _ptr(sb), int(bscale_kind), int(sb_s0),
                                          int(sb_s1), int(sb_estride), _ptr(d), _ld(d), int(out_dtype), int(accum),
                                          _stream()), "fp8_grouped_gemm_strided")
    return d


def moe_dgrad(offsets, qdy, sdy, qwt, sw, G, out_dtype=OUT_F32, accum=ACCUM_FP32):
    """M-grouped Dgrad of G experts: dX_e = dY_e W_e.  qdy, sdy: the 1x128
    quantisation of the expert-sorted dY [rows, N_w]; qwt, sw: the transposed
    codes [K_w, >=G*N_w] and scales [G*N_w/128, K_w/128] of the stacked
    weights [G*N_w, K_w] from fp8_quant_block(transpose=True)."""
    Kw, Nw = qwt.shape[0], qdy.shape[1]
    return fp8_grouped_gemm_strided(offsets, qdy, sdy, G, Kw, qwt, _ld(qwt), Nw, sw, BSCALE_BLOCK, 1, _ld(sw),
                                    (Nw // 128) * _ld(sw), out_dtype, accum=accum)


def fp8_grouped_gemm_kgrouped(offsets, a, sa, b, sb, out_dtype=OUT_F32, d=None, accum=ACCUM_FP32):
    """K-grouped expert GEMM: D[e] = sum over expert e's padded token groups
    (see include/fp8bs.h).  a [M, K], sa [K/128, M], b [N, K], sb [K/128, N]
    on the padded token axis; returns d [G, M, N]."""
    _dev(offsets, "offsets", torch.int32)
    _dev(a, "a", torch.uint8)
    _dev(sa, "sa", torch.float32)
    _dev(b, "b", torch.uint8)
    _dev(sb, "sb", torch.float32)
    G = offsets.numel() - 1
    M, K = a.shape
    N = b.shape[0]
    dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
    if d is None:
        d = torch.empty((G, M, N), dtype=dt, device=a.device)
    _check(lib().fp8_grouped_gemm_kgrouped(G, M, N, K, _ptr(offsets), _ptr(a), _ld(a), _ptr(sa), _ld(sa), _ptr(b),
                                           _ld(b), _ptr(sb), _ld(sb), _ptr(d), d.stride(1), d.stride(0),
                                           int(out_dtype), int(accum), _stream()), "fp8_grouped_gemm_kgrouped")
    return d


def moe_wgrad(offsets, dy, x, scale_mode=SCALE_FP32, out_dtype=OUT_F32, accum=ACCUM_FP32):
    """K-grouped Wgrad of G experts, dW_e = dY_e^T X_e, from the
    expert-sorted bf16 dY [T, N] and X [T, C]: both quantised in 128x1 groups
    per expert, then summed over each expert's tokens.  Returns [G, N, C]."""
    qdy, sdy = fp8_quant_tile_grouped_col(dy, offsets, scale_mode)
    qx, sx = fp8_quant_tile_grouped_col(x, offsets, scale_mode)
    return fp8_grouped_gemm_kgrouped(offsets, qdy, sdy, qx, sx, out_dtype, accum=accum)


# ---- the three GEMMs of a Linear ---------------------------------------------------

def linear_fprop(qx, sx, qw, sw, out_dtype=OUT_BF16, accum=ACCUM_FP32):
    """Y = X W^T from quant_tile(X, ROW) and quant_block(W)."""
    return fp8_gemm_blockscaled(qx, sx, qw, sw, BSCALE_BLOCK, _ld(sw), 1, out_dtype, accum=accum)


def linear_dgrad(qdy, sdy, qwt, sw, out_dtype=OUT_F32, accum=ACCUM_FP32):
    """dX = dY W from quant_tile(dY, ROW) and the transposed codes qt of
    quant_block(W) (scales of W read transposed)."""
    return fp8_gemm_blockscaled(qdy, sdy, qwt, sw, BSCALE_BLOCK, 1, _ld(sw), out_dtype, accum=accum)


def linear_wgrad(qdyt, sdyt, qxt, sxt, out_dtype=OUT_F32, accum=ACCUM_FP32):
    """dW = dY^T X from quant_tile(dY, COL) and quant_tile(X, COL)."""
    return fp8_gemm_blockscaled(qdyt, sdyt, qxt, sxt, BSCALE_TILE, _ld(sxt), 0, out_dtype, accum=accum)
