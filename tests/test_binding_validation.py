"""The Python binding rejects wrong tensor arguments before anything reaches the library.

Runs without a GPU: the device check of the binding is replaced by a contiguity-only check, and
the library is wrapped so that only host-side size queries may be called.  Every case must raise
ValueError (or TypeError) and launch nothing.
"""
import pytest
import torch

from sparse_rank_adapter_amd import _abi, api
from sparse_rank_adapter_amd.api import SparseMatrix
from sparse_rank_adapter_amd._abi import SRA_FMT_CSR, SRA_FMT_ELL, SRA_FMT_FFI_TILED, SRA_FMT_NM

HOST_QUERIES = {"sra_nm_meta_words", "sra_nm_tile_bytes", "sra_fwd_workspace", "sra_bwd_workspace",
                "sra_ffi_transpose_workspace", "sra_last_error", "sra_abi_version"}


class HostOnly:
    """Forwards the library's host-side queries; any other call fails the test."""

    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        if name in HOST_QUERIES:
            return getattr(self._lib, name)

        def refuse(*a, **k):
            raise AssertionError(f"{name} reached the library despite invalid arguments")
        return refuse


@pytest.fixture
def binding(monkeypatch):
    lib = _abi.load()
    monkeypatch.setattr(api, "load", lambda: HostOnly(lib))

    def dev_cpu(t, name="tensor", device=None):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return t
    monkeypatch.setattr(api, "_dev", dev_cpu)
    return api


def nm(rows, cols, dtype=torch.bfloat16):
    return SparseMatrix(SRA_FMT_NM, dtype, rows, cols, torch.zeros(rows, cols // 2, dtype=dtype),
                        meta=torch.zeros(rows, cols // 32, dtype=torch.int32))


T, K, N, R = 64, 128, 96, 8
bf = torch.bfloat16


def good_fwd():
    return dict(Ws=nm(N, K), X=torch.zeros(T, K, dtype=bf), A=torch.zeros(R, K, dtype=bf),
                B=torch.zeros(N, R, dtype=bf))


FWD_BAD = {
    "X too narrow": dict(X=torch.zeros(T, K - 32, dtype=bf)),
    "X wrong dtype": dict(X=torch.zeros(T, K, dtype=torch.float32)),
    "X transposed view": dict(X=torch.zeros(K, T, dtype=bf).t()),
    "A wrong shape": dict(A=torch.zeros(R, K + 32, dtype=bf)),
    "B transposed": dict(B=torch.zeros(R, N, dtype=bf)),
    "B wrong dtype": dict(B=torch.zeros(N, R, dtype=torch.float16)),
    "Y wrong shape": dict(Y=torch.zeros(T, N + 1, dtype=bf)),
    "U bf16": dict(U=torch.zeros(T, R, dtype=bf)),
    "U wrong rank": dict(U=torch.zeros(T, R + 1, dtype=torch.float32)),
    "values too short": dict(Ws=SparseMatrix(SRA_FMT_NM, bf, N, K, torch.zeros(N, K // 4, dtype=bf),
                                             meta=torch.zeros(N, K // 32, dtype=torch.int32))),
    "meta too short": dict(Ws=SparseMatrix(SRA_FMT_NM, bf, N, K, torch.zeros(N, K // 2, dtype=bf),
                                           meta=torch.zeros(N, 1, dtype=torch.int32))),
    "A without B": dict(B=None),
}


@pytest.mark.parametrize("case", sorted(FWD_BAD))
def test_fwd_rejects(binding, case):
    kw = good_fwd()
    kw.update(FWD_BAD[case])
    with pytest.raises((ValueError, TypeError)):
        binding.sparse_lora_fwd(kw.pop("Ws"), **kw)


def good_bwd():
    return dict(P=nm(K, N), dY=torch.zeros(T, N, dtype=bf), X=torch.zeros(T, K, dtype=bf),
                U=torch.zeros(T, R, dtype=torch.float32), A=torch.zeros(R, K, dtype=bf),
                B=torch.zeros(N, R, dtype=bf))


BWD_BAD = {
    "dY wrong width": dict(dY=torch.zeros(T, N + 4, dtype=bf)),
    "dY wrong dtype": dict(dY=torch.zeros(T, N, dtype=torch.float32)),
    "X wrong tokens": dict(X=torch.zeros(T + 1, K, dtype=bf)),
    "X missing for dA": dict(X=None),
    "U wrong tokens": dict(U=torch.zeros(T - 1, R, dtype=torch.float32)),
    "A wrong width": dict(A=torch.zeros(R, N, dtype=bf)),
    "B transposed": dict(B=torch.zeros(R, N, dtype=bf)),
    "dX out wrong shape": dict(out={"dX": torch.zeros(T, N, dtype=bf)}),
    "dA out bf16": dict(out={"dA": torch.zeros(R, K, dtype=bf)}),
    "dB out wrong shape": dict(out={"dB": torch.zeros(R, N, dtype=torch.float32)}),
    "dU out wrong shape": dict(want_du=True, out={"dU": torch.zeros(T, K, dtype=torch.float32)}),
}


@pytest.mark.parametrize("case", sorted(BWD_BAD))
def test_bwd_rejects(binding, case):
    kw = good_bwd()
    kw.update(BWD_BAD[case])
    with pytest.raises((ValueError, TypeError)):
        binding.sparse_lora_bwd(kw.pop("P"), **kw)


def test_compress_out_buffers_checked(binding):
    W = torch.zeros(N, K, dtype=bf)
    with pytest.raises(ValueError):
        binding.compress(W, out=nm(N, K // 2))                  # wrong logical shape
    small = SparseMatrix(SRA_FMT_NM, bf, N, K, torch.zeros(N, K // 4, dtype=bf),
                         meta=torch.zeros(N, K // 32, dtype=torch.int32))
    with pytest.raises(ValueError):
        binding.compress(W, out=small)                           # values buffer too small
    with pytest.raises(ValueError):
        binding.compress(W, out=nm(N, K, torch.float32))         # dtype differs from W
    with pytest.raises(ValueError):
        binding.compress(torch.zeros(N, K, dtype=torch.float16))
    with pytest.raises(ValueError):
        binding.compress_pair(W, out=(nm(N, K), nm(N, K)))       # P must be K x N


def test_double_prune_and_tile_outputs_checked(binding):
    Ws = nm(N, K)
    with pytest.raises(ValueError):
        binding.double_prune(Ws, out=nm(N, K))                   # P is K x N
    with pytest.raises(ValueError):
        binding.nm_tile(Ws, out=nm(N, K))                        # not the streaming format


def test_weight_grad_and_axpby_checked(binding):
    S = nm(N, K)
    with pytest.raises(ValueError):
        binding.masked_weight_grad(S, torch.zeros(T, K, dtype=bf), torch.zeros(T, K, dtype=bf))
    with pytest.raises(ValueError):
        binding.masked_weight_grad(S, torch.zeros(T, N, dtype=bf), torch.zeros(T, K, dtype=bf),
                                   out=torch.zeros(N, K, dtype=bf))
    a = torch.zeros(100, dtype=bf)
    with pytest.raises(ValueError):
        binding.nm_axpby(1.0, a, 1.0, torch.zeros(99, dtype=bf))
    with pytest.raises(ValueError):
        binding.nm_axpby(1.0, a, 1.0, a, out=torch.zeros(100, dtype=torch.float32))


def test_ffi_descriptors_checked(binding):
    ell = SparseMatrix(SRA_FMT_ELL, bf, N, K, torch.zeros(N, 8, dtype=bf),
                       index=torch.zeros(N, 4, dtype=torch.int16), k=8)
    with pytest.raises(ValueError):
        binding.ffi_transpose(ell)                               # index shorter than values
    csr = SparseMatrix(SRA_FMT_CSR, bf, K, N, torch.zeros(N * 8, dtype=bf),
                       index=torch.zeros(N * 8, dtype=torch.int16),
                       row_ptr=torch.zeros(K, dtype=torch.int32), nnz=N * 8)
    with pytest.raises(ValueError):
        binding.sparse_lora_bwd(csr, torch.zeros(T, N, dtype=bf), torch.zeros(T, K, dtype=bf))


def test_ffi_tiled_descriptors_checked(binding):
    nm = SparseMatrix(SRA_FMT_NM, bf, N, K, torch.zeros(N, K // 2, dtype=bf),
                      meta=torch.zeros(N, K // 32, dtype=torch.int32))
    with pytest.raises(ValueError):
        binding.ffi_tile(nm)                                     # not ELL or CSR
    lists = binding.ffi_tile_lists(N, K)
    short = SparseMatrix(SRA_FMT_FFI_TILED, bf, N, K, torch.zeros(64, dtype=torch.int32),
                         meta=torch.zeros(lists, dtype=torch.int32), nnz=64)
    with pytest.raises(ValueError):                              # offsets lack the 4 closing words
        binding.sparse_lora_fwd(short, torch.zeros(T, K, dtype=bf))
    f32 = SparseMatrix(SRA_FMT_FFI_TILED, torch.float32, N, K, torch.zeros(64, dtype=torch.int32),
                       meta=torch.zeros(lists + 4, dtype=torch.int32), nnz=64)
    with pytest.raises(ValueError):                              # bf16 only
        binding.sparse_lora_fwd(f32, torch.zeros(T, K, dtype=torch.float32))
    few = SparseMatrix(SRA_FMT_FFI_TILED, bf, N, K, torch.zeros(16, dtype=torch.int32),
                       meta=torch.zeros(lists + 4, dtype=torch.int32), nnz=64)
    with pytest.raises(ValueError):                              # fewer words than nnz says
        binding.sparse_lora_fwd(few, torch.zeros(T, K, dtype=bf))
