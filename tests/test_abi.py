"""The C ABI of libfp8bs.so: it loads, exports every function include/fp8bs.h
declares, and rejects bad arguments on the host before any HIP call (so
these run without a GPU)."""
import ctypes
import os
import re

import pytest

import block_scaled_gemm_amd as bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")

OK, ARG, SHAPE, ALIGN, WORKSPACE, DEVICE, HIP = range(7)
FAKE = 1 << 20  # a 16-byte aligned non-null address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8\w*)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ["fp8_quant_tile", "fp8_quant_block", "fp8_quant_dual", "fp8_requant_col", "fp8_gemm_blockscaled",
              "fp8_grouped_gemm_strided", "fp8_quant_tile_grouped_col", "fp8_grouped_gemm_kgrouped",
              "fp8_gemm_blockscaled_quant", "fp8_gemm_blockscaled_noalloc", "fp8_scales_are_pow2",
              "fp8_grouped_gemm", "fp8_gemm_workspace_bytes", "fp8_cast_e4m3",
              "fp8bs_abi_version", "fp8bs_status_string"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = bs.lib()
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in fp8bs.h but not exported"


def test_only_the_abi_is_exported():
    out = os.popen(f"nm -D --defined-only {bs.LIB_PATH}").read().split("\n")
    names = {l.split()[-1] for l in out if " T " in l}
    assert names, "nm printed nothing"
    assert names <= set(declared_functions()), names - set(declared_functions())


def test_version_and_status_strings():
    assert bs.abi_version() == 5
    for s in range(7):
        assert bs.status_string(s)
    assert "unknown" in bs.status_string(99)


def _tile(**kw):
    a = dict(x=FAKE, rows=256, cols=256, ldx=256, axis=0, mode=0, q=FAKE, ldq=256, s=FAKE, lds=256)
    a.update(kw)
    return bs.lib().fp8_quant_tile(a["x"], a["rows"], a["cols"], a["ldx"], a["axis"], a["mode"],
                                   a["q"], a["ldq"], a["s"], a["lds"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(axis=2), ARG), (dict(mode=3), ARG), (dict(x=None), ARG), (dict(q=None), ARG),
    (dict(s=None), ARG), (dict(rows=-1), ARG), (dict(ldx=128), ARG), (dict(ldq=128), ARG),
    (dict(lds=100), ARG), (dict(cols=200, ldx=256), SHAPE), (dict(axis=1, rows=200), SHAPE),
    (dict(x=FAKE + 2), ALIGN), (dict(q=FAKE + 8), ALIGN), (dict(s=FAKE + 2), ALIGN),
    (dict(ldx=260), ALIGN), (dict(ldq=264), ALIGN),
    (dict(rows=0), OK), (dict(cols=0, ldx=0, ldq=0), OK),
])
def test_quant_tile_validation(kw, want):
    assert _tile(**kw) == want


def _block(**kw):
    a = dict(w=FAKE, rows=256, cols=256, ldw=256, mode=0, q=FAKE, ldq=256, qt=None, ldqt=0, s=FAKE, lds=2)
    a.update(kw)
    return bs.lib().fp8_quant_block(a["w"], a["rows"], a["cols"], a["ldw"], a["mode"], a["q"], a["ldq"],
                                    a["qt"], a["ldqt"], a["s"], a["lds"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(mode=2), ARG), (dict(w=None), ARG), (dict(lds=1), ARG), (dict(qt=FAKE, ldqt=128), ARG),
    (dict(cols=192, ldw=256), SHAPE), (dict(qt=FAKE + 4, ldqt=256), ALIGN),
    (dict(qt=FAKE, ldqt=264), ALIGN), (dict(ldw=260), ALIGN), (dict(rows=0), OK),
])
def test_quant_block_validation(kw, want):
    assert _block(**kw) == want


def _dual(**kw):
    a = dict(x=FAKE, rows=256, cols=384, ldx=384, mode=0, qr=FAKE, ldqr=384, sr=FAKE, ldsr=256, qc=FAKE,
             ldqc=256, sc=FAKE, ldsc=384)
    a.update(kw)
    return bs.lib().fp8_quant_dual(a["x"], a["rows"], a["cols"], a["ldx"], a["mode"], a["qr"], a["ldqr"],
                                   a["sr"], a["ldsr"], a["qc"], a["ldqc"], a["sc"], a["ldsc"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(mode=2), ARG), (dict(x=None), ARG), (dict(qr=None), ARG), (dict(sc=None), ARG), (dict(cols=-128), ARG),
    (dict(ldx=256), ARG), (dict(ldqr=256), ARG), (dict(ldqc=128), ARG), (dict(ldsr=128), ARG), (dict(ldsc=256), ARG),
    (dict(rows=200, ldqc=256, ldsr=256), SHAPE), (dict(cols=200, ldx=384), SHAPE), (dict(x=FAKE + 8), ALIGN),
    (dict(qc=FAKE + 4), ALIGN), (dict(sr=FAKE + 1), ALIGN), (dict(ldx=388), ALIGN), (dict(ldqc=264), ALIGN),
    (dict(rows=0), OK),
])
def test_dual_validation(kw, want):
    assert _dual(**kw) == want


def _requant(**kw):
    a = dict(q=FAKE, rows=256, cols=384, ldq=384, s=FAKE, lds=256, mode=0, qt=FAKE, ldqt=256, st=FAKE, ldst=384)
    a.update(kw)
    return bs.lib().fp8_requant_col(a["q"], a["rows"], a["cols"], a["ldq"], a["s"], a["lds"], a["mode"],
                                    a["qt"], a["ldqt"], a["st"], a["ldst"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(mode=2), ARG), (dict(q=None), ARG), (dict(s=None), ARG), (dict(qt=None), ARG), (dict(st=None), ARG),
    (dict(rows=-128), ARG), (dict(ldq=256), ARG), (dict(lds=128), ARG), (dict(ldqt=128), ARG),
    (dict(ldst=256), ARG), (dict(rows=200, lds=256, ldqt=256), SHAPE), (dict(cols=200, ldq=384), SHAPE),
    (dict(q=FAKE + 8), ALIGN), (dict(qt=FAKE + 4), ALIGN), (dict(s=FAKE + 4), ALIGN), (dict(st=FAKE + 2), ALIGN),
    (dict(ldq=392), ALIGN), (dict(ldqt=264), ALIGN), (dict(lds=258), ALIGN),
    (dict(rows=0), OK), (dict(cols=0, ldq=0, ldst=0), OK),
])
def test_requant_validation(kw, want):
    assert _requant(**kw) == want


def _gemm(**kw):
    a = dict(M=256, N=256, K=512, a=FAKE, lda=512, sa=FAKE, ldsa=256, b=FAKE, ldb=512, sb=FAKE,
             kind=0, s0=4, s1=1, d=FAKE, ldd=256, out=0, acc=0, ws=None, wsb=0)
    a.update(kw)
    return bs.lib().fp8_gemm_blockscaled(a["M"], a["N"], a["K"], a["a"], a["lda"], a["sa"], a["ldsa"],
                                         a["b"], a["ldb"], a["sb"], a["kind"], a["s0"], a["s1"], a["d"],
                                         a["ldd"], a["out"], a["acc"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(kind=2), ARG), (dict(out=2), ARG), (dict(acc=3), ARG), (dict(a=None), ARG), (dict(d=None), ARG),
    (dict(M=-1), ARG), (dict(lda=256), ARG), (dict(ldd=128), ARG), (dict(ldsa=100), ARG),
    (dict(K=500, lda=512, ldb=512), SHAPE), (dict(a=FAKE + 8), ALIGN), (dict(d=FAKE + 4), ALIGN),
    (dict(lda=520), ALIGN), (dict(ldd=258), ALIGN), (dict(sa=FAKE + 1), ALIGN),
    (dict(M=0), OK), (dict(N=0), OK),
    (dict(M=256, N=256, K=65536, lda=65536, ldb=65536), WORKSPACE),
    # code strides: the kernels' per-lane row offsets inside a tile are 32-bit
    # (M = 0 stops after the argument checks, before any device work)
    (dict(lda=(1 << 24) + 16), SHAPE), (dict(ldb=(1 << 24) + 16), SHAPE), (dict(M=0, lda=(1 << 24) + 16), SHAPE),
    (dict(M=0, lda=1 << 24, ldb=1 << 24), OK),
])
def test_gemm_validation(kw, want):
    assert _gemm(**kw) == want


def _gna(**kw):
    a = dict(M=256, N=256, K=512, a=FAKE, lda=512, sa=FAKE, ldsa=256, b=FAKE, ldb=512, sb=FAKE,
             kind=0, s0=4, s1=1, d=FAKE, ldd=256, out=0, acc=0)
    a.update(kw)
    return bs.lib().fp8_gemm_blockscaled_noalloc(a["M"], a["N"], a["K"], a["a"], a["lda"], a["sa"], a["ldsa"],
                                                 a["b"], a["ldb"], a["sb"], a["kind"], a["s0"], a["s1"], a["d"],
                                                 a["ldd"], a["out"], a["acc"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(kind=2), ARG), (dict(out=2), ARG), (dict(acc=3), ARG), (dict(a=None), ARG), (dict(d=None), ARG),
    (dict(M=-1), ARG), (dict(lda=256), ARG), (dict(ldd=128), ARG), (dict(ldsa=100), ARG),
    (dict(K=500, lda=512, ldb=512), SHAPE), (dict(a=FAKE + 8), ALIGN), (dict(d=FAKE + 4), ALIGN),
    (dict(lda=(1 << 24) + 16), SHAPE), (dict(M=0), OK), (dict(N=0), OK),
    # split-K partials above the library's scratch array: 64 splits of a
    # 512 x 256 output (32 MiB) are refused before any device call
    (dict(M=512, N=256, K=65536, lda=65536, ldb=65536, ldsa=512), WORKSPACE),
])
def test_gemm_noalloc_validation(kw, want):
    assert _gna(**kw) == want


def test_noalloc_scratch_covers_the_large_k_workload():
    """The scratch array holds the split-K partials of the 256 x 256 x 65536
    GEMM, and the binding's constant matches the header's."""
    text = open(HEADER).read()
    assert "#define FP8BS_NOALLOC_SCRATCH_BYTES (16LL << 20)" in text
    assert bs.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert 0 < bs.gemm_workspace_bytes(256, 256, 65536) <= bs.NOALLOC_SCRATCH_BYTES
    assert bs.gemm_workspace_bytes(512, 256, 65536) > bs.NOALLOC_SCRATCH_BYTES


def _gq(**kw):
    a = dict(M=256, N=256, K=512, a=FAKE, lda=512, sa=FAKE, ldsa=256, b=FAKE, ldb=512, sb=FAKE, kind=0, s0=4, s1=1,
             mode=0, q=FAKE, ldq=256, s=FAKE, lds=256, acc=0)
    a.update(kw)
    return bs.lib().fp8_gemm_blockscaled_quant(a["M"], a["N"], a["K"], a["a"], a["lda"], a["sa"], a["ldsa"], a["b"],
                                               a["ldb"], a["sb"], a["kind"], a["s0"], a["s1"], a["mode"], a["q"],
                                               a["ldq"], a["s"], a["lds"], a["acc"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(kind=2), ARG), (dict(mode=2), ARG), (dict(acc=3), ARG), (dict(q=None), ARG), (dict(s=None), ARG),
    (dict(ldq=128), ARG), (dict(lds=100), ARG), (dict(N=200, ldq=256), SHAPE), (dict(K=500, lda=512, ldb=512), SHAPE),
    (dict(q=FAKE + 2), ALIGN), (dict(ldq=258), ALIGN), (dict(s=FAKE + 1), ALIGN), (dict(M=0), OK),
    # code strides above the 32-bit per-lane row offsets, as for the plain GEMM
    (dict(lda=(1 << 24) + 16), SHAPE), (dict(ldb=(1 << 24) + 16), SHAPE), (dict(M=0, lda=(1 << 24) + 16), SHAPE),
    (dict(M=0, lda=1 << 24, ldb=1 << 24), OK),
])
def test_gemm_quant_validation(kw, want):
    assert _gq(**kw) == want


def test_workspace_query():
    assert bs.gemm_workspace_bytes(4096, 18432, 7168) == 0
    need = bs.gemm_workspace_bytes(256, 256, 65536)
    assert need >= 2 * 256 * 256 * 4
    assert bs.gemm_workspace_bytes(256, 256, 100) == 0


def _grouped(**kw):
    a = dict(G=4, rows=512, N=256, K=512, off=FAKE, a=FAKE, lda=512, sa=FAKE, ldsa=512, b=FAKE,
             sb=FAKE, d=FAKE, ldd=256, out=0, acc=0)
    a.update(kw)
    return bs.lib().fp8_grouped_gemm(a["G"], a["rows"], a["N"], a["K"], a["off"], a["a"], a["lda"],
                                     a["sa"], a["ldsa"], a["b"], a["sb"], a["d"], a["ldd"], a["out"],
                                     a["acc"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(G=-1), ARG), (dict(acc=-1), ARG), (dict(off=None), ARG), (dict(N=200, ldd=256), SHAPE),
    (dict(K=500, lda=512), SHAPE), (dict(ldsa=100), ARG), (dict(off=FAKE + 2), ALIGN),
    (dict(G=0), OK), (dict(rows=0), OK),
])
def test_grouped_validation(kw, want):
    assert _grouped(**kw) == want


def _gstrided(**kw):
    a = dict(G=4, rows=512, N=200, K=512, off=FAKE, a=FAKE, lda=512, sa=FAKE, ldsa=512, b=FAKE, ldb=512,
             bes=512 * 256, sb=FAKE, kind=0, s0=4, s1=1, ses=8, d=FAKE, ldd=256, out=0, acc=0)
    a.update(kw)
    return bs.lib().fp8_grouped_gemm_strided(a["G"], a["rows"], a["N"], a["K"], a["off"], a["a"], a["lda"], a["sa"],
                                             a["ldsa"], a["b"], a["ldb"], a["bes"], a["sb"], a["kind"], a["s0"],
                                             a["s1"], a["ses"], a["d"], a["ldd"], a["out"], a["acc"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(G=-1), ARG), (dict(kind=2), ARG), (dict(acc=3), ARG), (dict(off=None), ARG), (dict(bes=-16), ARG),
    (dict(ses=-1), ARG), (dict(ldb=256), ARG), (dict(K=500, lda=512, ldb=512), SHAPE), (dict(bes=520), ALIGN),
    (dict(ldb=520), ALIGN), (dict(off=FAKE + 2), ALIGN), (dict(G=0), OK), (dict(N=0), OK),
])
def test_grouped_strided_validation(kw, want):
    assert _gstrided(**kw) == want


def _gcol(**kw):
    a = dict(x=FAKE, T=300, C=256, ldx=256, G=3, off=FAKE, mode=0, q=FAKE, ldq=768, s=FAKE, lds=256)
    a.update(kw)
    return bs.lib().fp8_quant_tile_grouped_col(a["x"], a["T"], a["C"], a["ldx"], a["G"], a["off"], a["mode"],
                                               a["q"], a["ldq"], a["s"], a["lds"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(mode=2), ARG), (dict(T=-1), ARG), (dict(G=-1), ARG), (dict(off=None), ARG), (dict(q=None), ARG),
    (dict(ldx=128), ARG), (dict(lds=100), ARG), (dict(ldq=640), ARG), (dict(x=FAKE + 8), ALIGN),
    (dict(q=FAKE + 4), ALIGN), (dict(ldq=776), ALIGN), (dict(ldx=260), ALIGN), (dict(G=0), OK), (dict(C=0), OK),
])
def test_grouped_col_validation(kw, want):
    assert _gcol(**kw) == want


def test_grouped_col_bound():
    assert bs.grouped_col_bound(300, 3) == 128 * (3 + 3)
    assert bs.grouped_col_bound(0, 0) == 0


def _kgrouped(**kw):
    a = dict(G=3, M=256, N=200, K=768, off=FAKE, a=FAKE, lda=768, sa=FAKE, ldsa=256, b=FAKE, ldb=768, sb=FAKE,
             ldsb=200, d=FAKE, ldd=200, des=256 * 200, out=1, acc=0)
    a.update(kw)
    return bs.lib().fp8_grouped_gemm_kgrouped(a["G"], a["M"], a["N"], a["K"], a["off"], a["a"], a["lda"], a["sa"],
                                              a["ldsa"], a["b"], a["ldb"], a["sb"], a["ldsb"], a["d"], a["ldd"],
                                              a["des"], a["out"], a["acc"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(G=-1), ARG), (dict(acc=3), ARG), (dict(out=2), ARG), (dict(off=None), ARG), (dict(ldsb=100), ARG),
    (dict(des=100), ARG), (dict(lda=640), ARG), (dict(K=700, lda=768, ldb=768), SHAPE), (dict(des=256 * 200 + 2), ALIGN),
    (dict(off=FAKE + 1), ALIGN), (dict(G=0), OK), (dict(M=0, des=0), OK),
])
def test_kgrouped_validation(kw, want):
    assert _kgrouped(**kw) == want


def test_cast_validation():
    L = bs.lib()
    assert L.fp8_cast_e4m3(None, 10, FAKE, None) == ARG
    assert L.fp8_cast_e4m3(FAKE, -1, FAKE, None) == ARG
    assert L.fp8_cast_e4m3(FAKE + 4, 10, FAKE, None) == ALIGN
    assert L.fp8_cast_e4m3(FAKE, 10, FAKE + 2, None) == ALIGN
    assert L.fp8_cast_e4m3(None, 0, None, None) == OK


def test_no_device_is_reported():
    """Valid arguments on a machine without a GPU stop at the device check
    (the fake pointers are never handed to a kernel)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this check is for GPU-less hosts")
    assert _tile() == DEVICE
    assert _gemm() == DEVICE


def test_pow2_check_validation():
    L = bs.lib()
    chk = lambda *a: L.fp8_scales_are_pow2(*a, None)
    assert chk(FAKE, -1, 4, 4, 1, FAKE) == ARG          # negative size
    assert chk(FAKE, 4, 4, -4, 1, FAKE) == ARG          # negative stride
    assert chk(FAKE, 4, 4, 4, 1, None) == ARG           # no flag
    assert chk(None, 4, 4, 4, 1, FAKE) == ARG           # no scales
    assert chk(FAKE + 2, 4, 4, 4, 1, FAKE) == ALIGN     # misaligned scales
    assert chk(FAKE, 4, 4, 4, 1, FAKE + 1) == ALIGN     # misaligned flag
