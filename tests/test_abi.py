"""Host-side tests of libsra's C ABI (no GPU needed, no kernel is launched).

Every call below fails validation, or is a pure host query, so it returns before any HIP call.
Pointers handed to the library are fake (aligned integers); they are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from sparse_rank_adapter_amd import _abi
from sparse_rank_adapter_amd._abi import (SRA_BF16, SRA_ERR_INVALID_ARG, SRA_ERR_UNSUPPORTED,
                                          SRA_ERR_WORKSPACE, SRA_F32, SRA_FMT_CSR, SRA_FMT_ELL,
                                          SRA_FMT_FFI_TILED, SRA_FMT_NM, SRA_FMT_NM_TILED, SRA_GRAD_DX, SRA_OK,
                                          SraSparse)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20  # aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_abi.LIB_PATH):
        pytest.fail("libsra.so is not built (run __graft_entry__.build())")
    return _abi.load()


def header_functions():
    src = open(os.path.join(ROOT, "include", "sra.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sra_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert sorted(_abi.EXPORTS) == declared
    for name in declared:
        assert getattr(lib, name) is not None


def test_version_and_sizes(lib):
    assert lib.sra_abi_version() == 1
    assert lib.sra_nm_meta_words(64, 2, 4) == 2
    assert lib.sra_nm_meta_words(4096, 2, 4) == 128
    assert lib.sra_nm_meta_words(96, 2, 4) == 3
    assert lib.sra_nm_meta_words(16, 2, 4) == 1   # 8 fields, one partly filled word


def nm_desc(rows=64, cols=128, dtype=SRA_BF16, n=2, m=4):
    d = SraSparse()
    d.format, d.dtype, d.rows, d.cols, d.n, d.m = SRA_FMT_NM, dtype, rows, cols, n, m
    d.values, d.meta = FAKE, FAKE
    return d


def ell_desc(rows=64, cols=128, k=8, dtype=SRA_BF16):
    d = SraSparse()
    d.format, d.dtype, d.rows, d.cols, d.k = SRA_FMT_ELL, dtype, rows, cols, k
    d.values, d.index = FAKE, FAKE
    return d


def err(lib):
    return lib.sra_last_error().decode()


@pytest.mark.parametrize("n,m,code", [(1, 4, SRA_ERR_UNSUPPORTED), (1, 8, SRA_ERR_UNSUPPORTED),
                                      (4, 8, SRA_ERR_UNSUPPORTED), (2, 16, SRA_ERR_INVALID_ARG),
                                      (2, 6, SRA_ERR_INVALID_ARG),
                                      (3, 2, SRA_ERR_INVALID_ARG), (0, 4, SRA_ERR_INVALID_ARG)])
def test_compress_rejects_patterns(lib, n, m, code):
    d = SraSparse()
    d.values, d.meta = FAKE, FAKE
    assert lib.sra_compress(FAKE, SRA_BF16, 4, 64, n, m, ctypes.byref(d), None) == code
    assert err(lib)


def test_compress_validation(lib):
    d = SraSparse()
    d.values, d.meta = FAKE, FAKE
    assert lib.sra_compress(FAKE, 7, 4, 64, 2, 4, ctypes.byref(d), None) == SRA_ERR_INVALID_ARG
    assert lib.sra_compress(FAKE, SRA_BF16, 4, 48, 2, 4, ctypes.byref(d), None) == SRA_ERR_UNSUPPORTED
    assert lib.sra_compress(None, SRA_BF16, 4, 64, 2, 4, ctypes.byref(d), None) == SRA_ERR_INVALID_ARG
    assert lib.sra_compress(FAKE + 2, SRA_BF16, 4, 64, 2, 4, ctypes.byref(d), None) == SRA_ERR_INVALID_ARG
    assert "aligned" in err(lib)
    assert lib.sra_compress(FAKE, SRA_BF16, -1, 64, 2, 4, ctypes.byref(d), None) == SRA_ERR_INVALID_ARG
    assert lib.sra_compress(FAKE, SRA_BF16, 4, 64, 2, 4, None, None) == SRA_ERR_INVALID_ARG


def test_double_prune_validation(lib):
    P = SraSparse()
    P.values, P.meta = FAKE, FAKE
    bad = nm_desc(rows=36)               # second prune groups along rows: 36 % 32 != 0
    assert lib.sra_double_prune(ctypes.byref(bad), ctypes.byref(P), None) == SRA_ERR_UNSUPPORTED
    e = ell_desc()
    assert lib.sra_double_prune(ctypes.byref(e), ctypes.byref(P), None) == SRA_ERR_INVALID_ARG
    ok = nm_desc()
    assert lib.sra_double_prune(ctypes.byref(ok), None, None) == SRA_ERR_INVALID_ARG


def test_compress_pair_validation(lib):
    S, P = SraSparse(), SraSparse()
    S.values, S.meta, P.values, P.meta = FAKE, FAKE, FAKE, FAKE
    # both dimensions are grouped: rows 36 is not a multiple of 32
    assert lib.sra_compress_pair(FAKE, SRA_BF16, 36, 64, 2, 4, ctypes.byref(S), ctypes.byref(P), None) == SRA_ERR_UNSUPPORTED
    assert lib.sra_compress_pair(FAKE, SRA_BF16, 64, 48, 2, 4, ctypes.byref(S), ctypes.byref(P), None) == SRA_ERR_UNSUPPORTED
    assert lib.sra_compress_pair(FAKE, SRA_BF16, 64, 64, 2, 4, ctypes.byref(S), None, None) == SRA_ERR_INVALID_ARG
    P.meta = None
    assert lib.sra_compress_pair(FAKE, SRA_BF16, 64, 64, 2, 4, ctypes.byref(S), ctypes.byref(P), None) == SRA_ERR_INVALID_ARG
    assert "P->meta" in err(lib)


def test_ffi_validation(lib):
    d = SraSparse()
    d.values, d.index = FAKE, FAKE
    assert lib.sra_compress_ffi(FAKE, SRA_BF16, 4, 64, 0, ctypes.byref(d), None) == SRA_ERR_INVALID_ARG
    assert lib.sra_compress_ffi(FAKE, SRA_BF16, 4, 64, 65, ctypes.byref(d), None) == SRA_ERR_INVALID_ARG
    assert lib.sra_compress_ffi(FAKE, SRA_BF16, 4, 40000, 8, ctypes.byref(d), None) == SRA_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert lib.sra_ffi_transpose_workspace(4096, 4096, 410, ctypes.byref(n)) == SRA_OK
    assert n.value >= 64 * 4096 * 4
    T_ = SraSparse()
    T_.row_ptr, T_.index, T_.values = FAKE, FAKE, FAKE
    e = ell_desc()
    assert lib.sra_ffi_transpose(ctypes.byref(e), ctypes.byref(T_), FAKE, 16, None) == SRA_ERR_WORKSPACE
    assert lib.sra_ffi_transpose(ctypes.byref(e), ctypes.byref(T_), None, 1 << 30, None) == SRA_ERR_WORKSPACE


def test_ffi_tile_validation(lib):
    eb, ob = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sra_ffi_tile_size(4096, 4096, 4096 * 410, ctypes.byref(eb), ctypes.byref(ob)) == SRA_OK
    lists = 128 * 64
    assert eb.value == (4096 * 410 + 3 * lists) * 4 and ob.value == (lists + 4) * 4
    assert lib.sra_ffi_tile_size(4096, 40000, 10, ctypes.byref(eb), ctypes.byref(ob)) == SRA_ERR_INVALID_ARG
    assert lib.sra_ffi_tile_size(4, 64, 257, ctypes.byref(eb), ctypes.byref(ob)) == SRA_ERR_INVALID_ARG
    out = SraSparse()
    out.values, out.meta = FAKE, FAKE
    assert lib.sra_ffi_tile(ctypes.byref(nm_desc()), ctypes.byref(out), None) == SRA_ERR_INVALID_ARG
    assert lib.sra_ffi_tile(ctypes.byref(ell_desc(dtype=SRA_F32)), ctypes.byref(out), None) == SRA_ERR_UNSUPPORTED
    assert lib.sra_ffi_tile(ctypes.byref(ell_desc()), None, None) == SRA_ERR_INVALID_ARG
    out.meta = None
    assert lib.sra_ffi_tile(ctypes.byref(ell_desc()), ctypes.byref(out), None) == SRA_ERR_INVALID_ARG
    # the tiled products: bf16, reduction a multiple of 64, no product workspace
    t = SraSparse()
    t.format, t.dtype, t.rows, t.cols, t.nnz = SRA_FMT_FFI_TILED, SRA_BF16, 4096, 4096, 1 << 20
    t.values, t.meta = FAKE, FAKE
    n = ctypes.c_size_t()
    assert lib.sra_fwd_workspace(ctypes.byref(t), 4096, 0, ctypes.byref(n)) == SRA_OK and n.value == 0
    assert lib.sra_bwd_workspace(ctypes.byref(t), 4096, 0, SRA_GRAD_DX, ctypes.byref(n)) == SRA_OK and n.value == 0
    t.cols = 4000
    assert lib.sra_fwd_workspace(ctypes.byref(t), 4096, 0, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
    assert lib.sra_bwd_workspace(ctypes.byref(t), 4096, 0, SRA_GRAD_DX, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
    t.cols, t.dtype = 4096, SRA_F32
    assert lib.sra_fwd_workspace(ctypes.byref(t), 4096, 0, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
    # an ELL weight with 128 or more tokens tiles into the workspace: O(nnz), not R x C
    e = ell_desc(rows=4096, cols=4096, k=410)
    assert lib.sra_fwd_workspace(ctypes.byref(e), 4096, 0, ctypes.byref(n)) == SRA_OK
    assert n.value <= (4096 * 410 + 4 * lists) * 4 + 1024 < 4096 * 4096 * 2 // 4


def test_fwd_validation_and_workspace(lib):
    d = nm_desc(rows=4096, cols=1024)
    n = ctypes.c_size_t()
    assert lib.sra_fwd_workspace(ctypes.byref(d), 2048, 16, ctypes.byref(n)) == SRA_OK
    assert n.value >= 2048 * 16 * 4          # room for U when the caller does not keep it
    assert lib.sra_fwd_workspace(ctypes.byref(d), 2048, 257, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
    assert lib.sra_fwd_workspace(ctypes.byref(d), -1, 16, ctypes.byref(n)) == SRA_ERR_INVALID_ARG
    d48 = nm_desc(rows=64, cols=48)           # 2:4 needs K % 32 == 0
    assert lib.sra_fwd_workspace(ctypes.byref(d48), 8, 4, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
    f32 = nm_desc(rows=64, cols=96, dtype=SRA_F32)
    assert lib.sra_fwd_workspace(ctypes.byref(f32), 8, 4, ctypes.byref(n)) == SRA_OK
    csr = SraSparse()
    csr.format, csr.dtype, csr.rows, csr.cols = SRA_FMT_CSR, SRA_BF16, 8, 8
    assert lib.sra_fwd_workspace(ctypes.byref(csr), 8, 4, ctypes.byref(n)) == SRA_ERR_INVALID_ARG
    # workspace too small / missing
    big = ctypes.c_size_t()
    lib.sra_fwd_workspace(ctypes.byref(d), 2048, 16, ctypes.byref(big))
    st = lib.sra_sparse_lora_fwd(ctypes.byref(d), FAKE, 2048, FAKE, FAKE, 16, FAKE, None, FAKE, 16, None)
    assert st == SRA_ERR_WORKSPACE
    st = lib.sra_sparse_lora_fwd(ctypes.byref(d), None, 2048, FAKE, FAKE, 16, FAKE, None, FAKE, big.value, None)
    assert st == SRA_ERR_INVALID_ARG and "X" in err(lib)
    st = lib.sra_sparse_lora_fwd(ctypes.byref(d), FAKE, 2048, None, FAKE, 16, FAKE, None, FAKE, big.value, None)
    assert st == SRA_ERR_INVALID_ARG and "A" in err(lib)


@pytest.mark.parametrize("T", [0, 1, 7, 2048])
@pytest.mark.parametrize("r", [0, 16, 256])
@pytest.mark.parametrize("shape", [(4096, 1024), (1024, 4096), (32, 64), (64, 96)])
def test_workspace_queries_any_size(lib, T, r, shape):
    """Pure host sizing logic: never fails or traps for valid shapes, including T = 0."""
    for dtype in (SRA_BF16, SRA_F32):
        d = nm_desc(rows=shape[0], cols=shape[1], dtype=dtype)
        n = ctypes.c_size_t()
        assert lib.sra_fwd_workspace(ctypes.byref(d), T, r, ctypes.byref(n)) == SRA_OK
        for flags in (1, 2, 4, 7, 15):
            assert lib.sra_bwd_workspace(ctypes.byref(d), T, r, flags, ctypes.byref(n)) == SRA_OK


def test_nm_tile_validation(lib):
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sra_nm_tile_bytes(36864, 9216, 2, 4, ctypes.byref(vb), ctypes.byref(mb)) == SRA_OK
    assert vb.value == 36864 * 9216 and mb.value == 36864 * 9216 // 8   # same bytes as canonical
    assert lib.sra_nm_tile_bytes(100, 96, 2, 4, ctypes.byref(vb), ctypes.byref(mb)) == SRA_OK
    assert vb.value == 7 * 2 * 1024 and mb.value == 7 * 1 * 1024          # padded 16-row tiles
    assert lib.sra_nm_tile_bytes(64, 48, 2, 4, ctypes.byref(vb), ctypes.byref(mb)) == SRA_ERR_UNSUPPORTED
    assert lib.sra_nm_tile_bytes(64, 64, 1, 4, ctypes.byref(vb), ctypes.byref(mb)) == SRA_ERR_UNSUPPORTED
    f32 = nm_desc(rows=64, cols=64, dtype=SRA_F32)
    out = nm_desc(rows=64, cols=64)
    assert lib.sra_nm_tile(ctypes.byref(f32), ctypes.byref(out), None) == SRA_ERR_UNSUPPORTED
    tiled = nm_desc(rows=64, cols=64)
    tiled.format = SRA_FMT_NM_TILED
    assert lib.sra_nm_tile(ctypes.byref(tiled), ctypes.byref(out), None) == SRA_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert lib.sra_fwd_workspace(ctypes.byref(tiled), 16, 64, ctypes.byref(n)) == SRA_OK
    assert lib.sra_fwd_workspace(ctypes.byref(tiled), 17, 64, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
    assert "16 tokens" in err(lib)
    assert lib.sra_bwd_workspace(ctypes.byref(tiled), 16, 64, SRA_GRAD_DX, ctypes.byref(n)) == SRA_OK
    assert lib.sra_bwd_workspace(ctypes.byref(tiled), 17, 64, SRA_GRAD_DX, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
    wide = nm_desc(rows=256, cols=1024)
    wide.format = SRA_FMT_NM_TILED
    assert lib.sra_fwd_workspace(ctypes.byref(wide), 2048, 16, ctypes.byref(n)) == SRA_OK
    assert lib.sra_bwd_workspace(ctypes.byref(wide), 2048, 16, SRA_GRAD_DX, ctypes.byref(n)) == SRA_OK
    tiled.dtype = SRA_F32
    assert lib.sra_fwd_workspace(ctypes.byref(tiled), 16, 64, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED


def test_compress_pair_tiled_validation(lib):
    a, b = nm_desc(rows=256, cols=256), nm_desc(rows=256, cols=256)
    call = lambda dt, R, C, n=2, m=4: lib.sra_compress_pair_tiled(FAKE, dt, R, C, n, m, ctypes.byref(a),
                                                                  ctypes.byref(b), None)
    assert call(SRA_F32, 256, 256) == SRA_ERR_UNSUPPORTED
    assert call(SRA_BF16, 64, 256) == SRA_ERR_UNSUPPORTED and "128" in err(lib)
    assert call(SRA_BF16, 256, 96) == SRA_ERR_UNSUPPORTED
    assert call(SRA_BF16, 256, 256, 1, 4) == SRA_ERR_UNSUPPORTED
    assert lib.sra_compress_pair_tiled(FAKE, SRA_BF16, 256, 256, 2, 4, None, ctypes.byref(b), None) == SRA_ERR_INVALID_ARG


def test_masked_weight_grad_validation(lib):
    d = nm_desc(rows=64, cols=128)
    assert lib.sra_masked_weight_grad(ctypes.byref(d), FAKE, FAKE, 16, None, None) == SRA_ERR_INVALID_ARG
    assert lib.sra_masked_weight_grad(ctypes.byref(d), FAKE, FAKE, -1, FAKE, None) == SRA_ERR_INVALID_ARG
    f32 = nm_desc(rows=64, cols=128, dtype=SRA_F32)
    assert lib.sra_masked_weight_grad(ctypes.byref(f32), FAKE, FAKE, 16, FAKE, None) == SRA_ERR_UNSUPPORTED
    odd = nm_desc(rows=60, cols=128)
    assert lib.sra_masked_weight_grad(ctypes.byref(odd), FAKE, FAKE, 16, FAKE, None) == SRA_ERR_UNSUPPORTED
    tiled = nm_desc(rows=64, cols=128)
    tiled.format = SRA_FMT_NM_TILED
    assert lib.sra_masked_weight_grad(ctypes.byref(tiled), FAKE, FAKE, 16, FAKE, None) == SRA_ERR_INVALID_ARG
    assert lib.sra_masked_weight_grad(None, FAKE, FAKE, 16, FAKE, None) == SRA_ERR_INVALID_ARG


def test_nm_axpby_validation(lib):
    assert lib.sra_nm_axpby(FAKE, 1.0, FAKE, 1.0, FAKE, -1, SRA_BF16, None) == SRA_ERR_INVALID_ARG
    assert lib.sra_nm_axpby(None, 1.0, FAKE, 1.0, FAKE, 8, SRA_BF16, None) == SRA_ERR_INVALID_ARG
    assert lib.sra_nm_axpby(FAKE, 1.0, FAKE, 1.0, FAKE + 2, 8, SRA_BF16, None) == SRA_ERR_INVALID_ARG
    assert lib.sra_nm_axpby(FAKE, 1.0, FAKE, 1.0, FAKE, 8, 7, None) != SRA_OK
    assert lib.sra_nm_axpby(None, 1.0, None, 1.0, None, 0, SRA_BF16, None) == SRA_OK  # nothing to do


def test_nm12_validation(lib):
    """1:2 is accepted by the canonical paths and refused by the streaming layout."""
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sra_nm_tile_bytes(256, 256, 1, 2, ctypes.byref(vb), ctypes.byref(mb)) == SRA_ERR_UNSUPPORTED
    a, b = nm_desc(rows=256, cols=256), nm_desc(rows=256, cols=256)
    assert lib.sra_compress_pair_tiled(FAKE, SRA_BF16, 256, 256, 1, 2, ctypes.byref(a), ctypes.byref(b),
                                       None) == SRA_ERR_UNSUPPORTED
    d12 = nm_desc(rows=4096, cols=1024, n=1, m=2)
    d24 = nm_desc(rows=4096, cols=1024)
    n12, n24 = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sra_fwd_workspace(ctypes.byref(d12), 2048, 16, ctypes.byref(n12)) == SRA_OK
    assert lib.sra_fwd_workspace(ctypes.byref(d24), 2048, 16, ctypes.byref(n24)) == SRA_OK
    assert n12.value >= n24.value + 4096 * 1024 // 32 * 4   # the converted metadata
    assert lib.sra_nm_tile(ctypes.byref(d12), ctypes.byref(a), None) == SRA_ERR_UNSUPPORTED
    assert lib.sra_nm_meta_words(1024, 1, 2) == 1024 // 32


def test_bwd_validation(lib):
    P = nm_desc(rows=1024, cols=4096)
    n = ctypes.c_size_t()
    assert lib.sra_bwd_workspace(ctypes.byref(P), 2048, 16, 7, ctypes.byref(n)) == SRA_OK
    assert lib.sra_bwd_workspace(ctypes.byref(P), 2048, 16, 16, ctypes.byref(n)) == SRA_ERR_INVALID_ARG
    e = ell_desc()
    assert lib.sra_bwd_workspace(ctypes.byref(e), 8, 4, 7, ctypes.byref(n)) == SRA_ERR_INVALID_ARG
    lib.sra_bwd_workspace(ctypes.byref(P), 2048, 16, 7, ctypes.byref(n))
    st = lib.sra_sparse_lora_bwd(ctypes.byref(P), FAKE, FAKE, 2048, FAKE, FAKE, FAKE, 16, 7,
                                 None, FAKE, FAKE, None, FAKE, n.value, None)
    assert st == SRA_ERR_INVALID_ARG and "dX" in err(lib)
    st = lib.sra_sparse_lora_bwd(ctypes.byref(P), FAKE, FAKE, 2048, FAKE, FAKE, FAKE, 16, 7,
                                 FAKE, FAKE, FAKE, None, None, 0, None)
    assert st == SRA_ERR_WORKSPACE


def test_nm28_validation(lib):
    """2:8: bf16 only, 32-column multiples, no pair or streaming forms; products above 16 tokens run
    on the 2:4 kernels (the weight rewritten as 2:4 in the workspace, K % 32), at 16 tokens or fewer
    on the 2:8 decode kernel (K % 32, no workspace), and the expanded-fragment path (the dense-MFMA
    engine above 16 tokens) needs K % 128."""
    d = SraSparse()
    d.values, d.meta = FAKE, FAKE
    assert lib.sra_compress(FAKE, SRA_F32, 64, 64, 2, 8, ctypes.byref(d), None) == SRA_ERR_UNSUPPORTED
    assert lib.sra_compress(FAKE, SRA_BF16, 64, 48, 2, 8, ctypes.byref(d), None) == SRA_ERR_UNSUPPORTED
    P = SraSparse()
    P.values, P.meta = FAKE, FAKE
    assert lib.sra_compress_pair(FAKE, SRA_BF16, 64, 64, 2, 8, ctypes.byref(d), ctypes.byref(P),
                                 None) == SRA_ERR_UNSUPPORTED
    assert lib.sra_nm_meta_words(1024, 2, 8) == 32 and lib.sra_nm_meta_words(40, 2, 8) == 2
    W = nm_desc(rows=256, cols=192, n=2, m=8)
    n = ctypes.c_size_t()
    assert lib.sra_fwd_workspace(ctypes.byref(W), 300, 8, ctypes.byref(n)) == SRA_OK
    assert n.value >= 256 * 96 * 2 + 256 * 6 * 4  # the 2:4 values and metadata
    assert lib.sra_fwd_workspace(ctypes.byref(W), 16, 0, ctypes.byref(n)) == SRA_OK
    assert n.value == 0  # the decode kernel needs no workspace
    assert lib.sra_set_tuning(4, 1) == SRA_OK  # the dense-MFMA engine
    try:
        assert lib.sra_fwd_workspace(ctypes.byref(W), 300, 8, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
        assert "128" in err(lib)
        assert lib.sra_fwd_workspace(ctypes.byref(W), 16, 8, ctypes.byref(n)) == SRA_OK
    finally:
        assert lib.sra_set_tuning(0, 0) == SRA_OK
    W = nm_desc(rows=256, cols=256, n=2, m=8)
    assert lib.sra_fwd_workspace(ctypes.byref(W), 300, 8, ctypes.byref(n)) == SRA_OK
    W.dtype = SRA_F32
    assert lib.sra_fwd_workspace(ctypes.byref(W), 300, 8, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
    # the 2:8 streaming layout: 16-row x 256-column blocks of 2 KB values + 512 B metadata
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sra_nm_tile_bytes(40, 288, 2, 8, ctypes.byref(vb), ctypes.byref(mb)) == SRA_OK
    assert (vb.value, mb.value) == (3 * 2 * 2048, 3 * 2 * 512)
    assert lib.sra_nm_tile_bytes(40, 288, 1, 2, ctypes.byref(vb), ctypes.byref(mb)) == SRA_ERR_UNSUPPORTED
    out = SraSparse()
    out.values, out.meta = FAKE, FAKE
    assert lib.sra_nm_tile(ctypes.byref(nm_desc(rows=256, cols=256, n=1, m=2)), ctypes.byref(out),
                           None) == SRA_ERR_UNSUPPORTED
    # a tiled 2:8 weight: any K % 32 at 16 tokens or fewer (the decode kernel) and above (the
    # weight rewritten as 2:4), K % 128 only for the dense engine above 16 tokens
    Wt = nm_desc(rows=256, cols=96, n=2, m=8)
    Wt.format = SRA_FMT_NM_TILED
    assert lib.sra_fwd_workspace(ctypes.byref(Wt), 16, 8, ctypes.byref(n)) == SRA_OK
    assert lib.sra_fwd_workspace(ctypes.byref(Wt), 300, 8, ctypes.byref(n)) == SRA_OK
    assert n.value >= 256 * 48 * 2 + 256 * 3 * 4


def test_tuning_knobs(lib):
    """sra_set_tuning: validated keys and values; a dense-engine 2:4 product needs K % 128."""
    from sparse_rank_adapter_amd._abi import SRA_TUNE_KEYS
    assert lib.sra_set_tuning(99, 0) == SRA_ERR_INVALID_ARG
    assert lib.sra_set_tuning(SRA_TUNE_KEYS["engine"], 5) == SRA_ERR_INVALID_ARG
    assert lib.sra_set_tuning(SRA_TUNE_KEYS["decode_rows"], 5) == SRA_ERR_INVALID_ARG
    assert lib.sra_set_tuning(SRA_TUNE_KEYS["spmm_splits"], -1) == SRA_ERR_INVALID_ARG
    W = nm_desc(rows=256, cols=192)
    n = ctypes.c_size_t()
    assert lib.sra_fwd_workspace(ctypes.byref(W), 300, 8, ctypes.byref(n)) == SRA_OK
    try:
        assert lib.sra_set_tuning(SRA_TUNE_KEYS["engine"], 1) == SRA_OK
        assert lib.sra_fwd_workspace(ctypes.byref(W), 300, 8, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
        assert lib.sra_fwd_workspace(ctypes.byref(W), 16, 8, ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
    finally:
        assert lib.sra_set_tuning(0, 0) == SRA_OK
    assert lib.sra_fwd_workspace(ctypes.byref(W), 300, 8, ctypes.byref(n)) == SRA_OK


def test_bwd_noalloc_host_checks(lib):
    """The allocation-free backward validates like sra_sparse_lora_bwd and refuses calls whose
    workspace exceeds its fixed array, both before touching the GPU."""
    P = nm_desc(rows=5120, cols=20480)
    st = lib.sra_sparse_lora_bwd_noalloc(ctypes.byref(P), FAKE, FAKE, 8192, None, FAKE, FAKE, 128, 7,
                                         FAKE, FAKE, FAKE, None, None)
    assert st == SRA_ERR_WORKSPACE and "allocation-free" in err(lib)
    st = lib.sra_sparse_lora_bwd_noalloc(ctypes.byref(P), FAKE, FAKE, 8192, None, FAKE, FAKE, 128, 16,
                                         FAKE, FAKE, FAKE, None, None)
    assert st == SRA_ERR_INVALID_ARG
    small = nm_desc(rows=1024, cols=4096)
    st = lib.sra_sparse_lora_bwd_noalloc(ctypes.byref(small), FAKE, FAKE, 2048, FAKE, FAKE, FAKE, 16,
                                         7, None, FAKE, FAKE, None, None)
    assert st == SRA_ERR_INVALID_ARG and "dX" in err(lib)
    assert _abi.SRA_NOALLOC_SCRATCH_BYTES == 64 << 20


def test_ffa_validation(lib):
    """Fixed-fan-in adapter factor: A must be a bf16 ELL matrix over the layer's K."""
    W = nm_desc(rows=1024, cols=4096)
    A = ell_desc(rows=32, cols=4096, k=768)
    n = ctypes.c_size_t()
    assert lib.sra_ffa_fwd_workspace(ctypes.byref(W), 2048, ctypes.byref(A), ctypes.byref(n)) == SRA_OK
    assert n.value >= 32 * 4096 * 2
    bad = ell_desc(rows=32, cols=2048, k=768)
    assert lib.sra_ffa_fwd_workspace(ctypes.byref(W), 2048, ctypes.byref(bad), ctypes.byref(n)) == SRA_ERR_INVALID_ARG
    assert "columns" in err(lib)
    assert lib.sra_ffa_fwd_workspace(ctypes.byref(W), 2048, ctypes.byref(nm_desc(rows=32, cols=4096)),
                                     ctypes.byref(n)) == SRA_ERR_INVALID_ARG
    big = ell_desc(rows=300, cols=4096, k=8)
    assert lib.sra_ffa_fwd_workspace(ctypes.byref(W), 2048, ctypes.byref(big), ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
    f32 = ell_desc(rows=32, cols=4096, k=768, dtype=SRA_F32)
    assert lib.sra_ffa_fwd_workspace(ctypes.byref(W), 2048, ctypes.byref(f32), ctypes.byref(n)) == SRA_ERR_UNSUPPORTED
    lib.sra_ffa_fwd_workspace(ctypes.byref(W), 2048, ctypes.byref(A), ctypes.byref(n))
    st = lib.sra_sparse_lora_fwd_ffa(ctypes.byref(W), FAKE, 2048, ctypes.byref(A), FAKE, FAKE, None,
                                     FAKE, n.value - 256, None)
    assert st == SRA_ERR_WORKSPACE
    P = nm_desc(rows=4096, cols=1024)
    assert lib.sra_ffa_bwd_workspace(ctypes.byref(P), 2048, ctypes.byref(A), 7, ctypes.byref(n)) == SRA_OK
    st = lib.sra_sparse_lora_bwd_ffa(ctypes.byref(P), FAKE, FAKE, 2048, FAKE, ctypes.byref(A), FAKE, 7,
                                     FAKE, None, FAKE, None, FAKE, n.value, None)
    assert st == SRA_ERR_INVALID_ARG and "dA_values" in err(lib)
    st = lib.sra_sparse_lora_bwd_ffa(ctypes.byref(P), FAKE, None, 2048, FAKE, ctypes.byref(A), FAKE, 7,
                                     FAKE, FAKE, FAKE, None, FAKE, n.value, None)
    assert st == SRA_ERR_INVALID_ARG and "X" in err(lib)


def test_binding_fails_loudly_when_library_missing(tmp_path):
    saved = _abi._lib
    _abi._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            _abi.load(str(tmp_path / "libsra.so"))
    finally:
        _abi._lib = saved


def test_long_reduction_tail_split_workspace(lib):
    """The planner splits the reduction of long-C products whose 256 x 256 tiles leave the last
    wave of 256 workgroups at most half full (OPT-13B fc2 forward: 640 tiles), on both layouts, so
    their workspace holds two fp32 partial arrays; the short-C product (fc1 forward, 2560 tiles)
    needs none.  Rank 0, so only the product's share of the workspace counts."""
    n = ctypes.c_size_t()
    T, partials = 8192, 2 * 8192 * 5120 * 4
    for fmt in (SRA_FMT_NM, SRA_FMT_NM_TILED):
        fc2 = nm_desc(rows=5120, cols=20480)
        fc2.format = fmt
        assert lib.sra_fwd_workspace(ctypes.byref(fc2), T, 0, ctypes.byref(n)) == SRA_OK
        assert n.value >= partials
        fc1 = nm_desc(rows=20480, cols=5120)
        fc1.format = fmt
        assert lib.sra_fwd_workspace(ctypes.byref(fc1), T, 0, ctypes.byref(n)) == SRA_OK
        assert n.value < partials
