"""Tensor-level binding of libsra: the same calls as include/sra.h, argument marshalling only.

torch supplies device memory and the current stream; every step runs in the library's HIP
kernels.  Nothing here computes a result on the host.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _abi
from ._abi import (SRA_BF16, SRA_DX_NO_ADAPTER, SRA_F32, SRA_FMT_CSR, SRA_FMT_ELL, SRA_FMT_NM,
                   SRA_FMT_NM_TILED,
                   SRA_GRAD_DA, SRA_GRAD_DB, SRA_GRAD_DX, SraSparse, check, load)

_DT = {torch.bfloat16: SRA_BF16, torch.float32: SRA_F32}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"dtype {t.dtype} is not bfloat16 or float32")
    return _DT[t.dtype]


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


@dataclass
class SparseMatrix:
    """Compressed sparse matrix (rows x cols, every row reduced over its cols) and its buffers."""
    fmt: int
    dtype: torch.dtype
    rows: int
    cols: int
    values: torch.Tensor
    meta: torch.Tensor | None = None     # NM: int32 storage of the uint32 words
    index: torch.Tensor | None = None    # ELL / CSR: int16
    row_ptr: torch.Tensor | None = None  # CSR: int32
    n: int = 2
    m: int = 4
    k: int = 0
    nnz: int = 0

    def desc(self) -> SraSparse:
        d = SraSparse()
        d.format, d.dtype, d.rows, d.cols = self.fmt, _DT[self.dtype], self.rows, self.cols
        d.n, d.m, d.k, d.nnz = self.n, self.m, self.k, self.nnz
        d.values = self.values.data_ptr() if self.values is not None else None
        d.meta = self.meta.data_ptr() if self.meta is not None else None
        d.index = self.index.data_ptr() if self.index is not None else None
        d.row_ptr = self.row_ptr.data_ptr() if self.row_ptr is not None else None
        return d

    @property
    def device(self):
        return self.values.device


def meta_words(cols: int, n: int = 2, m: int = 4) -> int:
    return int(load().sra_nm_meta_words(cols, n, m))


def compress(W: torch.Tensor, n: int = 2, m: int = 4, out: SparseMatrix | None = None) -> SparseMatrix:
    """compress(W, N, M): first N:M prune along W's columns (into `out`'s buffers if given)."""
    lib = load()
    _dev(W)
    rows, cols = W.shape
    if out is None:
        vals = torch.empty((rows, cols // m * n), dtype=W.dtype, device=W.device)
        meta = torch.empty((rows, meta_words(cols, n, m)), dtype=torch.int32, device=W.device)
        out = SparseMatrix(SRA_FMT_NM, W.dtype, rows, cols, vals, meta=meta, n=n, m=m)
    d = out.desc()
    check("sra_compress", lib.sra_compress(_p(W), _dt(W), rows, cols, n, m, ctypes.byref(d), _stream(W.device)))
    return out


def double_prune(Ws: SparseMatrix, out: SparseMatrix | None = None) -> SparseMatrix:
    """P = prune_NM(Ws^T): rows = Ws.cols, cols = Ws.rows (into `out`'s buffers if given)."""
    lib = load()
    P = out
    if P is None:
        vals = torch.empty((Ws.cols, Ws.rows // Ws.m * Ws.n), dtype=Ws.dtype, device=Ws.device)
        meta = torch.empty((Ws.cols, meta_words(Ws.rows, Ws.n, Ws.m)), dtype=torch.int32, device=Ws.device)
        P = SparseMatrix(SRA_FMT_NM, Ws.dtype, Ws.cols, Ws.rows, vals, meta=meta, n=Ws.n, m=Ws.m)
    dw, dp = Ws.desc(), P.desc()
    check("sra_double_prune", lib.sra_double_prune(ctypes.byref(dw), ctypes.byref(dp), _stream(Ws.device)))
    return P


def compress_pair(W: torch.Tensor, n: int = 2, m: int = 4, out: tuple | None = None):
    """(compress(W), double_prune(compress(W))) in one pass over W; `out` = (Ws, P) reuses buffers."""
    lib = load()
    _dev(W)
    rows, cols = W.shape
    if out is None:
        Ws = SparseMatrix(SRA_FMT_NM, W.dtype, rows, cols,
                          torch.empty((rows, cols // m * n), dtype=W.dtype, device=W.device),
                          meta=torch.empty((rows, meta_words(cols, n, m)), dtype=torch.int32, device=W.device),
                          n=n, m=m)
        P = SparseMatrix(SRA_FMT_NM, W.dtype, cols, rows,
                         torch.empty((cols, rows // m * n), dtype=W.dtype, device=W.device),
                         meta=torch.empty((cols, meta_words(rows, n, m)), dtype=torch.int32, device=W.device),
                         n=n, m=m)
    else:
        Ws, P = out
    dw, dp = Ws.desc(), P.desc()
    check("sra_compress_pair", lib.sra_compress_pair(_p(W), _dt(W), rows, cols, n, m, ctypes.byref(dw),
                                                     ctypes.byref(dp), _stream(W.device)))
    return Ws, P


def nm_tile(Ws: SparseMatrix, out: SparseMatrix | None = None) -> SparseMatrix:
    """The 2:4 weight Ws in the streaming layout for forwards of at most 16 tokens (sra_nm_tile)."""
    lib = load()
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    check("sra_nm_tile_bytes", lib.sra_nm_tile_bytes(Ws.rows, Ws.cols, Ws.n, Ws.m, ctypes.byref(vb),
                                                     ctypes.byref(mb)))
    if out is None:
        vals = torch.empty(max(1, vb.value // 2), dtype=Ws.dtype, device=Ws.device)
        meta = torch.empty(max(1, mb.value // 4), dtype=torch.int32, device=Ws.device)
        out = SparseMatrix(SRA_FMT_NM_TILED, Ws.dtype, Ws.rows, Ws.cols, vals, meta=meta, n=Ws.n, m=Ws.m)
    dw, do = Ws.desc(), out.desc()
    check("sra_nm_tile", lib.sra_nm_tile(ctypes.byref(dw), ctypes.byref(do), _stream(Ws.device)))
    return out


def tile_bytes(rows: int, cols: int, n: int = 2, m: int = 4) -> tuple:
    """(value bytes, metadata bytes) of the streaming layout of a rows x cols N:M matrix."""
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    check("sra_nm_tile_bytes", load().sra_nm_tile_bytes(rows, cols, n, m, ctypes.byref(vb), ctypes.byref(mb)))
    return vb.value, mb.value


def compress_pair_tiled(W: torch.Tensor, n: int = 2, m: int = 4, out: tuple | None = None):
    """compress_pair with both outputs in the streaming layout (sra_compress_pair_tiled)."""
    lib = load()
    _dev(W)
    rows, cols = W.shape
    if out is None:
        def mk(r, c):
            vb, mb = tile_bytes(r, c, n, m)
            return SparseMatrix(SRA_FMT_NM_TILED, W.dtype, r, c,
                                torch.empty(max(1, vb // 2), dtype=W.dtype, device=W.device),
                                meta=torch.empty(max(1, mb // 4), dtype=torch.int32, device=W.device), n=n, m=m)
        Ws, P = mk(rows, cols), mk(cols, rows)
    else:
        Ws, P = out
    dw, dp = Ws.desc(), P.desc()
    check("sra_compress_pair_tiled", lib.sra_compress_pair_tiled(_p(W), _dt(W), rows, cols, n, m,
                                                                 ctypes.byref(dw), ctypes.byref(dp),
                                                                 _stream(W.device)))
    return Ws, P


def masked_weight_grad(S: SparseMatrix, row_act: torch.Tensor, col_act: torch.Tensor,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """Gradient of S's stored values: out[row][i] = sum_t row_act[t][row] col_act[t][c_i(row)].

    For the forward weight Ws: masked_weight_grad(Ws, dY, X) = (dY^T X) o mask in Ws's value order.
    """
    lib = load()
    _dev(row_act)
    _dev(col_act)
    T = row_act.shape[0]
    if row_act.shape != (T, S.rows) or col_act.shape != (T, S.cols):
        raise ValueError("row_act must be [T, S.rows] and col_act [T, S.cols]")
    if out is None:
        out = torch.empty((S.rows, S.cols // S.m * S.n), dtype=S.dtype, device=S.device)
    d = S.desc()
    check("sra_masked_weight_grad", lib.sra_masked_weight_grad(ctypes.byref(d), _p(row_act), _p(col_act), T,
                                                               _p(out), _stream(S.device)))
    return out


def nm_axpby(beta: float, a: torch.Tensor, gamma: float, b: torch.Tensor,
             out: torch.Tensor | None = None) -> torch.Tensor:
    """out = beta * a + gamma * b on value arrays sharing one N:M pattern (sra_nm_axpby);
    ``out=a`` updates in place."""
    lib = load()
    _dev(a)
    _dev(b)
    if a.shape != b.shape or a.dtype != b.dtype:
        raise ValueError("a and b must have the same shape and dtype")
    if out is None:
        out = torch.empty_like(a)
    check("sra_nm_axpby", lib.sra_nm_axpby(_p(a), float(beta), _p(b), float(gamma), _p(out), a.numel(),
                                           _dt(a), _stream(a.device)))
    return out


def compress_ffi(W: torch.Tensor, k: int) -> SparseMatrix:
    """compress_ffi(W, k): keep the k largest-magnitude entries of every row (ELL, int16 columns)."""
    lib = load()
    _dev(W)
    rows, cols = W.shape
    vals = torch.empty((rows, k), dtype=W.dtype, device=W.device)
    idx = torch.empty((rows, k), dtype=torch.int16, device=W.device)
    out = SparseMatrix(SRA_FMT_ELL, W.dtype, rows, cols, vals, index=idx, k=k)
    d = out.desc()
    check("sra_compress_ffi", lib.sra_compress_ffi(_p(W), _dt(W), rows, cols, k, ctypes.byref(d), _stream(W.device)))
    return out


def ffi_transpose(Ws: SparseMatrix) -> SparseMatrix:
    """Exact transpose of an ELL weight as CSR (rows = Ws.cols)."""
    lib = load()
    nnz = Ws.rows * Ws.k
    nbytes = ctypes.c_size_t()
    check("sra_ffi_transpose_workspace", lib.sra_ffi_transpose_workspace(Ws.rows, Ws.cols, Ws.k, ctypes.byref(nbytes)))
    ws = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=Ws.device)
    row_ptr = torch.empty(Ws.cols + 1, dtype=torch.int32, device=Ws.device)
    idx = torch.empty(max(nnz, 0), dtype=torch.int16, device=Ws.device)
    vals = torch.empty(max(nnz, 0), dtype=Ws.dtype, device=Ws.device)
    T_ = SparseMatrix(SRA_FMT_CSR, Ws.dtype, Ws.cols, Ws.rows, vals, index=idx, row_ptr=row_ptr, nnz=nnz)
    dw, dt = Ws.desc(), T_.desc()
    check("sra_ffi_transpose", lib.sra_ffi_transpose(ctypes.byref(dw), ctypes.byref(dt), _p(ws), nbytes.value, _stream(Ws.device)))
    return T_


def time_next_kernel(which: int, start: torch.cuda.Event, stop: torch.cuda.Event) -> None:
    """Arm the profiling hook: the next launch of kernel class `which` records start/stop."""
    for e in (start, stop):
        if e.cuda_event == 0:  # torch creates events lazily
            e.record()
    check("sra_time_next_kernel", load().sra_time_next_kernel(which, ctypes.c_void_p(start.cuda_event),
                                                              ctypes.c_void_p(stop.cuda_event)))


def bwd_workspace(P: SparseMatrix, T: int, r: int, flags: int = SRA_GRAD_DX | SRA_GRAD_DA | SRA_GRAD_DB) -> int:
    n = ctypes.c_size_t()
    d = P.desc()
    check("sra_bwd_workspace", load().sra_bwd_workspace(ctypes.byref(d), T, r, flags, ctypes.byref(n)))
    return n.value


def fwd_workspace(Ws: SparseMatrix, T: int, r: int) -> int:
    n = ctypes.c_size_t()
    d = Ws.desc()
    check("sra_fwd_workspace", load().sra_fwd_workspace(ctypes.byref(d), T, r, ctypes.byref(n)))
    return n.value


def sparse_lora_fwd(Ws: SparseMatrix, X: torch.Tensor, A: torch.Tensor | None = None,
                    B: torch.Tensor | None = None, Y: torch.Tensor | None = None,
                    U: torch.Tensor | None = None, want_u: bool = True, ws: torch.Tensor | None = None):
    """Y = X Ws^T + (X A^T) B^T.  Returns (Y, U) with U fp32 [T, r] (None when r = 0 or not wanted)."""
    lib = load()
    _dev(X)
    T = X.shape[0]
    r = 0 if A is None else A.shape[0]
    dev = X.device
    if Y is None:
        Y = torch.empty((T, Ws.rows), dtype=X.dtype, device=dev)
    if U is None and want_u and r > 0:
        U = torch.empty((T, r), dtype=torch.float32, device=dev)
    d = Ws.desc()
    nbytes = ctypes.c_size_t()
    check("sra_fwd_workspace", lib.sra_fwd_workspace(ctypes.byref(d), T, r, ctypes.byref(nbytes)))
    if ws is None or ws.numel() < nbytes.value:
        ws = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=dev)
    check("sra_sparse_lora_fwd", lib.sra_sparse_lora_fwd(
        ctypes.byref(d), _p(X), T, _p(A) if r else None, _p(B) if r else None, r, _p(Y),
        _p(U) if r else None, _p(ws), ws.numel(), _stream(dev)))
    return Y, U


def sparse_lora_bwd(P: SparseMatrix, dY: torch.Tensor, X: torch.Tensor | None = None,
                    U: torch.Tensor | None = None, A: torch.Tensor | None = None,
                    B: torch.Tensor | None = None, dx: bool = True, da: bool = True, db: bool = True,
                    dx_adapter: bool = True, want_du: bool = False, ws: torch.Tensor | None = None,
                    out: dict | None = None):
    """Double-pruned backward.  Returns dict with dX, dA, dB (and dU when want_du)."""
    lib = load()
    _dev(dY)
    T = dY.shape[0]
    r = 0 if A is None else A.shape[0]
    dev = dY.device
    K, N = P.rows, P.cols
    flags = (SRA_GRAD_DX if dx else 0) | (SRA_GRAD_DA if da else 0) | (SRA_GRAD_DB if db else 0)
    if not dx_adapter:
        flags |= SRA_DX_NO_ADAPTER
    out = dict(out or {})
    if dx and out.get("dX") is None:
        out["dX"] = torch.empty((T, K), dtype=dY.dtype, device=dev)
    if da and r and out.get("dA") is None:
        out["dA"] = torch.empty((r, K), dtype=torch.float32, device=dev)
    if db and r and out.get("dB") is None:
        out["dB"] = torch.empty((N, r), dtype=torch.float32, device=dev)
    if want_du and r and out.get("dU") is None:
        out["dU"] = torch.empty((T, r), dtype=torch.float32, device=dev)
    d = P.desc()
    nbytes = ctypes.c_size_t()
    check("sra_bwd_workspace", lib.sra_bwd_workspace(ctypes.byref(d), T, r, flags, ctypes.byref(nbytes)))
    if ws is None or ws.numel() < nbytes.value:
        ws = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=dev)
    check("sra_sparse_lora_bwd", lib.sra_sparse_lora_bwd(
        ctypes.byref(d), _p(dY), _p(X), T, _p(U) if r else None, _p(A) if r else None,
        _p(B) if r else None, r, flags, _p(out.get("dX")), _p(out.get("dA")), _p(out.get("dB")),
        _p(out.get("dU")), _p(ws), ws.numel(), _stream(dev)))
    return out
