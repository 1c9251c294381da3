"""Tensor-level binding of libsra: the same calls as include/sra.h, argument marshalling only.

torch supplies device memory and the current stream; every step runs in the library's HIP
kernels.  Nothing here computes a result on the host.
"""
from __future__ import annotations

import ctypes
from contextlib import contextmanager
from dataclasses import dataclass

import torch

from . import _abi
from ._abi import (SRA_BF16, SRA_DX_NO_ADAPTER, SRA_F32, SRA_FMT_CSR, SRA_FMT_ELL, SRA_FMT_NM,
                   SRA_FMT_NM_TILED, SRA_FMT_FFI_TILED,
                   SRA_GRAD_DA, SRA_GRAD_DB, SRA_GRAD_DX, SraSparse, check, load)

_DT = {torch.bfloat16: SRA_BF16, torch.float32: SRA_F32}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise ValueError(f"dtype {t.dtype} is not bfloat16 or float32")
    return _DT[t.dtype]


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str = "tensor", device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _arg(t, name: str, shape: tuple, dtype: torch.dtype, device=None, min_numel: bool = False):
    """Check one tensor argument before anything reaches the library: shape (or, with
    ``min_numel``, at least that many elements), dtype, device and contiguity.  Shape and dtype
    are checked first so that a wrong call is reported the same way with or without a GPU."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if min_numel:
        need = 1
        for d in shape:
            need *= int(d)
        if t.numel() < need:
            raise ValueError(f"{name} holds {t.numel()} elements, needs at least {need}")
    elif tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return _dev(t, name, device)


def _check_sparse(S: "SparseMatrix", name: str):
    """Buffers of a compressed matrix: dtype, device, contiguity and sizes for its format."""
    if S.dtype not in _DT:
        raise ValueError(f"{name}: dtype {S.dtype} is not bfloat16 or float32")
    dev = S.values.device if S.values is not None else None
    if S.fmt == SRA_FMT_NM:
        _arg(S.values, f"{name}.values", (S.rows, S.cols // S.m * S.n), S.dtype, dev)
        _arg(S.meta, f"{name}.meta", (S.rows, meta_words(S.cols, S.n, S.m)), torch.int32, dev,
             min_numel=True)
    elif S.fmt == SRA_FMT_NM_TILED:
        vb, mb = tile_bytes(S.rows, S.cols, S.n, S.m)
        _arg(S.values, f"{name}.values", (vb // S.values.element_size(),), S.dtype, dev, min_numel=True)
        _arg(S.meta, f"{name}.meta", (mb // 4,), torch.int32, dev, min_numel=True)
    elif S.fmt == SRA_FMT_ELL:
        _arg(S.values, f"{name}.values", (S.rows, S.k), S.dtype, dev)
        _arg(S.index, f"{name}.index", (S.rows, S.k), torch.int16, dev)
    elif S.fmt == SRA_FMT_CSR:
        _arg(S.values, f"{name}.values", (S.nnz,), S.dtype, dev, min_numel=True)
        _arg(S.index, f"{name}.index", (S.nnz,), torch.int16, dev, min_numel=True)
        _arg(S.row_ptr, f"{name}.row_ptr", (S.rows + 1,), torch.int32, dev)
    elif S.fmt == SRA_FMT_FFI_TILED:
        if S.dtype != torch.bfloat16:
            raise ValueError(f"{name}: the tiled fixed fan-in format is bfloat16 only")
        _arg(S.values, f"{name}.values", (S.nnz,), torch.int32, dev, min_numel=True)
        _arg(S.meta, f"{name}.meta", (ffi_tile_lists(S.rows, S.cols) + 4,), torch.int32, dev, min_numel=True)
    else:
        raise ValueError(f"{name}: unknown format {S.fmt}")
    return dev


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


def _mat(W, name: str):
    """A dense 2-D input matrix (bf16 or fp32, on the GPU, contiguous); returns its shape."""
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    _dt(W)
    _dev(W, name)
    return tuple(int(x) for x in W.shape)


def _check_out_nm(S: "SparseMatrix", name: str, like: torch.Tensor, rows: int, cols: int, n: int, m: int):
    """An output descriptor in the canonical N:M format of a rows x cols matrix."""
    if S.fmt != SRA_FMT_NM or S.rows != rows or S.cols != cols or (S.n, S.m) != (n, m):
        raise ValueError(f"{name} must describe a canonical {n}:{m} matrix of {rows} x {cols}")
    if S.dtype != like.dtype:
        raise ValueError(f"{name} has dtype {S.dtype}, expected {like.dtype}")
    _check_sparse(S, name)
    if S.values.device != like.device:
        raise ValueError(f"{name} is on {S.values.device}, expected {like.device}")


def _check_out_tiled(S: "SparseMatrix", name: str, like: torch.Tensor, rows: int, cols: int, n: int, m: int):
    """An output descriptor in the streaming layout of a rows x cols matrix."""
    if S.fmt != SRA_FMT_NM_TILED or S.rows != rows or S.cols != cols or (S.n, S.m) != (n, m):
        raise ValueError(f"{name} must describe a streaming-layout {n}:{m} matrix of {rows} x {cols}")
    if S.dtype != like.dtype:
        raise ValueError(f"{name} has dtype {S.dtype}, expected {like.dtype}")
    _check_sparse(S, name)
    if S.values.device != like.device:
        raise ValueError(f"{name} is on {S.values.device}, expected {like.device}")


def compress(W: torch.Tensor, n: int = 2, m: int = 4, out: SparseMatrix | None = None) -> SparseMatrix:
    """compress(W, N, M): first N:M prune along W's columns (into `out`'s buffers if given)."""
    lib = load()
    rows, cols = _mat(W, "W")
    if out is None:
        vals = torch.empty((rows, cols // m * n), dtype=W.dtype, device=W.device)
        meta = torch.empty((rows, meta_words(cols, n, m)), dtype=torch.int32, device=W.device)
        out = SparseMatrix(SRA_FMT_NM, W.dtype, rows, cols, vals, meta=meta, n=n, m=m)
    _check_out_nm(out, "out", W, rows, cols, n, m)
    d = out.desc()
    check("sra_compress", lib.sra_compress(_p(W), _dt(W), rows, cols, n, m, ctypes.byref(d), _stream(W.device)))
    return out


def double_prune(Ws: SparseMatrix, out: SparseMatrix | None = None) -> SparseMatrix:
    """P = prune_NM(Ws^T): rows = Ws.cols, cols = Ws.rows (into `out`'s buffers if given)."""
    lib = load()
    _check_sparse(Ws, "Ws")
    P = out
    if P is None:
        vals = torch.empty((Ws.cols, Ws.rows // Ws.m * Ws.n), dtype=Ws.dtype, device=Ws.device)
        meta = torch.empty((Ws.cols, meta_words(Ws.rows, Ws.n, Ws.m)), dtype=torch.int32, device=Ws.device)
        P = SparseMatrix(SRA_FMT_NM, Ws.dtype, Ws.cols, Ws.rows, vals, meta=meta, n=Ws.n, m=Ws.m)
    _check_out_nm(P, "out", Ws.values, Ws.cols, Ws.rows, Ws.n, Ws.m)
    dw, dp = Ws.desc(), P.desc()
    check("sra_double_prune", lib.sra_double_prune(ctypes.byref(dw), ctypes.byref(dp), _stream(Ws.device)))
    return P


def compress_pair(W: torch.Tensor, n: int = 2, m: int = 4, out: tuple | None = None):
    """(compress(W), double_prune(compress(W))) in one pass over W; `out` = (Ws, P) reuses buffers."""
    lib = load()
    rows, cols = _mat(W, "W")
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
    _check_out_nm(Ws, "out[0]", W, rows, cols, n, m)
    _check_out_nm(P, "out[1]", W, cols, rows, n, m)
    dw, dp = Ws.desc(), P.desc()
    check("sra_compress_pair", lib.sra_compress_pair(_p(W), _dt(W), rows, cols, n, m, ctypes.byref(dw),
                                                     ctypes.byref(dp), _stream(W.device)))
    return Ws, P


def nm_tile(Ws: SparseMatrix, out: SparseMatrix | None = None) -> SparseMatrix:
    """The 2:4 weight Ws in the streaming layout for forwards of at most 16 tokens (sra_nm_tile)."""
    lib = load()
    _check_sparse(Ws, "Ws")
    vb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    check("sra_nm_tile_bytes", lib.sra_nm_tile_bytes(Ws.rows, Ws.cols, Ws.n, Ws.m, ctypes.byref(vb),
                                                     ctypes.byref(mb)))
    if out is None:
        vals = torch.empty(max(1, vb.value // 2), dtype=Ws.dtype, device=Ws.device)
        meta = torch.empty(max(1, mb.value // 4), dtype=torch.int32, device=Ws.device)
        out = SparseMatrix(SRA_FMT_NM_TILED, Ws.dtype, Ws.rows, Ws.cols, vals, meta=meta, n=Ws.n, m=Ws.m)
    _check_out_tiled(out, "out", Ws.values, Ws.rows, Ws.cols, Ws.n, Ws.m)
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
    rows, cols = _mat(W, "W")
    if out is None:
        def mk(r, c):
            vb, mb = tile_bytes(r, c, n, m)
            return SparseMatrix(SRA_FMT_NM_TILED, W.dtype, r, c,
                                torch.empty(max(1, vb // 2), dtype=W.dtype, device=W.device),
                                meta=torch.empty(max(1, mb // 4), dtype=torch.int32, device=W.device), n=n, m=m)
        Ws, P = mk(rows, cols), mk(cols, rows)
    else:
        Ws, P = out
    _check_out_tiled(Ws, "out[0]", W, rows, cols, n, m)
    _check_out_tiled(P, "out[1]", W, cols, rows, n, m)
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
    if S.fmt != SRA_FMT_NM:
        raise ValueError("masked_weight_grad takes a canonical N:M matrix")
    dev = _check_sparse(S, "S")
    if not isinstance(row_act, torch.Tensor) or row_act.dim() != 2:
        raise ValueError("row_act must be a 2-D tensor [T, S.rows]")
    T = row_act.shape[0]
    _arg(row_act, "row_act", (T, S.rows), S.dtype, dev)
    _arg(col_act, "col_act", (T, S.cols), S.dtype, dev)
    if out is None:
        out = torch.empty((S.rows, S.cols // S.m * S.n), dtype=S.dtype, device=S.device)
    _arg(out, "out", (S.rows, S.cols // S.m * S.n), S.dtype, dev)
    d = S.desc()
    check("sra_masked_weight_grad", lib.sra_masked_weight_grad(ctypes.byref(d), _p(row_act), _p(col_act), T,
                                                               _p(out), _stream(S.device)))
    return out


def nm_axpby(beta: float, a: torch.Tensor, gamma: float, b: torch.Tensor,
             out: torch.Tensor | None = None) -> torch.Tensor:
    """out = beta * a + gamma * b on value arrays sharing one N:M pattern (sra_nm_axpby);
    ``out=a`` updates in place."""
    lib = load()
    _dt(a)
    _arg(a, "a", tuple(a.shape), a.dtype)
    _arg(b, "b", tuple(a.shape), a.dtype, a.device)
    if out is None:
        out = torch.empty_like(a)
    _arg(out, "out", tuple(a.shape), a.dtype, a.device)
    check("sra_nm_axpby", lib.sra_nm_axpby(_p(a), float(beta), _p(b), float(gamma), _p(out), a.numel(),
                                           _dt(a), _stream(a.device)))
    return out


def compress_ffi(W: torch.Tensor, k: int) -> SparseMatrix:
    """compress_ffi(W, k): keep the k largest-magnitude entries of every row (ELL, int16 columns)."""
    lib = load()
    rows, cols = _mat(W, "W")
    vals = torch.empty((rows, k), dtype=W.dtype, device=W.device)
    idx = torch.empty((rows, k), dtype=torch.int16, device=W.device)
    out = SparseMatrix(SRA_FMT_ELL, W.dtype, rows, cols, vals, index=idx, k=k)
    d = out.desc()
    check("sra_compress_ffi", lib.sra_compress_ffi(_p(W), _dt(W), rows, cols, k, ctypes.byref(d), _stream(W.device)))
    return out


def ffi_tile_lists(rows: int, cols: int) -> int:
    """Entry lists of the tiled fixed fan-in format: one per 32-row group and 64-column stage."""
    return -(-rows // 32) * -(-cols // 64)


def ffi_tile(S: SparseMatrix) -> SparseMatrix:
    """The products' tiled layout of an ELL weight or of its CSR transpose (bf16): per 32-row group
    and 64-column stage, a list of packed (value, position) words; values are int32 words."""
    lib = load()
    if S.fmt not in (SRA_FMT_ELL, SRA_FMT_CSR):
        raise ValueError("ffi_tile takes an ELL or CSR matrix")
    _check_sparse(S, "S")
    nnz = S.rows * S.k if S.fmt == SRA_FMT_ELL else S.nnz
    eb, ob = ctypes.c_size_t(), ctypes.c_size_t()
    check("sra_ffi_tile_size", lib.sra_ffi_tile_size(S.rows, S.cols, nnz, ctypes.byref(eb), ctypes.byref(ob)))
    ent = torch.empty(max(1, eb.value // 4), dtype=torch.int32, device=S.device)
    offs = torch.empty(ob.value // 4, dtype=torch.int32, device=S.device)
    out = SparseMatrix(SRA_FMT_FFI_TILED, S.dtype, S.rows, S.cols, ent, meta=offs, nnz=eb.value // 4)
    ds, do = S.desc(), out.desc()
    check("sra_ffi_tile", lib.sra_ffi_tile(ctypes.byref(ds), ctypes.byref(do), _stream(S.device)))
    out.nnz = int(do.nnz)
    return out


def ffi_transpose(Ws: SparseMatrix) -> SparseMatrix:
    """Exact transpose of an ELL weight as CSR (rows = Ws.cols)."""
    lib = load()
    if Ws.fmt != SRA_FMT_ELL:
        raise ValueError("ffi_transpose takes an ELL matrix")
    _check_sparse(Ws, "Ws")
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
    dev = _check_sparse(Ws, "Ws")
    N, K, dt = Ws.rows, Ws.cols, Ws.dtype
    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise ValueError("X must be a 2-D tensor [T, K]")
    T = X.shape[0]
    _arg(X, "X", (T, K), dt, dev)
    if (A is None) != (B is None):
        raise ValueError("A and B must both be given or both be None")
    r = 0 if A is None else A.shape[0]
    if r:
        _arg(A, "A", (r, K), dt, dev)
        _arg(B, "B", (N, r), dt, dev)
    if Y is None:
        Y = torch.empty((T, N), dtype=dt, device=dev)
    _arg(Y, "Y", (T, N), dt, dev)
    if U is None and want_u and r > 0:
        U = torch.empty((T, r), dtype=torch.float32, device=dev)
    if U is not None and r:
        _arg(U, "U", (T, r), torch.float32, dev)
    d = Ws.desc()
    nbytes = ctypes.c_size_t()
    check("sra_fwd_workspace", lib.sra_fwd_workspace(ctypes.byref(d), T, r, ctypes.byref(nbytes)))
    if ws is None or ws.numel() < nbytes.value:
        ws = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=dev)
    _arg(ws, "ws", (ws.numel(),), torch.uint8, dev)
    check("sra_sparse_lora_fwd", lib.sra_sparse_lora_fwd(
        ctypes.byref(d), _p(X), T, _p(A) if r else None, _p(B) if r else None, r, _p(Y),
        _p(U) if r else None, _p(ws), ws.numel(), _stream(dev)))
    return Y, U


def sparse_lora_bwd(P: SparseMatrix, dY: torch.Tensor, X: torch.Tensor | None = None,
                    U: torch.Tensor | None = None, A: torch.Tensor | None = None,
                    B: torch.Tensor | None = None, dx: bool = True, da: bool = True, db: bool = True,
                    dx_adapter: bool = True, want_du: bool = False, ws: torch.Tensor | None = None,
                    out: dict | None = None, noalloc: bool = False):
    """Double-pruned backward.  Returns dict with dX, dA, dB (and dU when want_du).

    ``noalloc=True`` calls sra_sparse_lora_bwd_noalloc: no workspace, the library's fixed per-GPU
    array instead (outputs missing from ``out`` are still allocated here by torch)."""
    lib = load()
    dev = _check_sparse(P, "P")
    K, N, dt = P.rows, P.cols, P.dtype
    if not isinstance(dY, torch.Tensor) or dY.dim() != 2:
        raise ValueError("dY must be a 2-D tensor [T, N]")
    T = dY.shape[0]
    _arg(dY, "dY", (T, N), dt, dev)
    if (A is None) != (B is None):
        raise ValueError("A and B must both be given or both be None")
    r = 0 if A is None else A.shape[0]
    if r:
        _arg(A, "A", (r, K), dt, dev)
        _arg(B, "B", (N, r), dt, dev)
    if U is not None and r:
        _arg(U, "U", (T, r), torch.float32, dev)
    # X feeds dA, and U when U is not given
    if X is not None:
        _arg(X, "X", (T, K), dt, dev)
    elif r and (da or (db and U is None) or dt == torch.float32):
        raise ValueError("X is needed for dA, and for dB when U is not given")
    flags = (SRA_GRAD_DX if dx else 0) | (SRA_GRAD_DA if da else 0) | (SRA_GRAD_DB if db else 0)
    if not dx_adapter:
        flags |= SRA_DX_NO_ADAPTER
    out = dict(out or {})
    if dx and out.get("dX") is None:
        out["dX"] = torch.empty((T, K), dtype=dt, device=dev)
    if da and r and out.get("dA") is None:
        out["dA"] = torch.empty((r, K), dtype=torch.float32, device=dev)
    if db and r and out.get("dB") is None:
        out["dB"] = torch.empty((N, r), dtype=torch.float32, device=dev)
    if want_du and r and out.get("dU") is None:
        out["dU"] = torch.empty((T, r), dtype=torch.float32, device=dev)
    for key, shape, odt in (("dX", (T, K), dt), ("dA", (r, K), torch.float32),
                            ("dB", (N, r), torch.float32), ("dU", (T, r), torch.float32)):
        if out.get(key) is not None:
            _arg(out[key], f"out['{key}']", shape, odt, dev)
    d = P.desc()
    if not noalloc:
        nbytes = ctypes.c_size_t()
        check("sra_bwd_workspace", lib.sra_bwd_workspace(ctypes.byref(d), T, r, flags, ctypes.byref(nbytes)))
        if ws is None or ws.numel() < nbytes.value:
            ws = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=dev)
        _arg(ws, "ws", (ws.numel(),), torch.uint8, dev)
    if noalloc:
        check("sra_sparse_lora_bwd_noalloc", lib.sra_sparse_lora_bwd_noalloc(
            ctypes.byref(d), _p(dY), _p(X), T, _p(U) if r else None, _p(A) if r else None,
            _p(B) if r else None, r, flags, _p(out.get("dX")), _p(out.get("dA")), _p(out.get("dB")),
            _p(out.get("dU")), _stream(dev)))
        return out
    check("sra_sparse_lora_bwd", lib.sra_sparse_lora_bwd(
        ctypes.byref(d), _p(dY), _p(X), T, _p(U) if r else None, _p(A) if r else None,
        _p(B) if r else None, r, flags, _p(out.get("dX")), _p(out.get("dA")), _p(out.get("dB")),
        _p(out.get("dU")), _p(ws), ws.numel(), _stream(dev)))
    return out


def _check_ffa_factor(A: SparseMatrix, K: int, dt, dev):
    if not isinstance(A, SparseMatrix) or A.fmt != SRA_FMT_ELL:
        raise ValueError("A must be an ELL SparseMatrix (compress_ffi of the dense factor)")
    if A.cols != K or A.dtype != dt:
        raise ValueError(f"A must be [r, {K}] of dtype {dt}, got [{A.rows}, {A.cols}] {A.dtype}")
    d = _check_sparse(A, "A")
    if d != dev:
        raise ValueError(f"A is on {d}, expected {dev}")
    return A.rows


def sparse_lora_fwd_ffa(Ws: SparseMatrix, X: torch.Tensor, A: SparseMatrix, B: torch.Tensor,
                        Y: torch.Tensor | None = None, U: torch.Tensor | None = None,
                        want_u: bool = True, ws: torch.Tensor | None = None):
    """Y = X Ws^T + (X A_s^T) B^T with a fixed-fan-in adapter factor A (ELL [r, K]).
    Returns (Y, U) with U fp32 [T, r] (None when not wanted)."""
    lib = load()
    dev = _check_sparse(Ws, "Ws")
    N, K, dt = Ws.rows, Ws.cols, Ws.dtype
    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise ValueError("X must be a 2-D tensor [T, K]")
    T = X.shape[0]
    _arg(X, "X", (T, K), dt, dev)
    r = _check_ffa_factor(A, K, dt, dev)
    _arg(B, "B", (N, r), dt, dev)
    if Y is None:
        Y = torch.empty((T, N), dtype=dt, device=dev)
    _arg(Y, "Y", (T, N), dt, dev)
    if U is None and want_u:
        U = torch.empty((T, r), dtype=torch.float32, device=dev)
    if U is not None:
        _arg(U, "U", (T, r), torch.float32, dev)
    dw, da = Ws.desc(), A.desc()
    nbytes = ctypes.c_size_t()
    check("sra_ffa_fwd_workspace", lib.sra_ffa_fwd_workspace(ctypes.byref(dw), T, ctypes.byref(da),
                                                             ctypes.byref(nbytes)))
    if ws is None or ws.numel() < nbytes.value:
        ws = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=dev)
    _arg(ws, "ws", (ws.numel(),), torch.uint8, dev)
    check("sra_sparse_lora_fwd_ffa", lib.sra_sparse_lora_fwd_ffa(
        ctypes.byref(dw), _p(X), T, ctypes.byref(da), _p(B), _p(Y), _p(U), _p(ws), ws.numel(),
        _stream(dev)))
    return Y, U


def sparse_lora_bwd_ffa(P: SparseMatrix, dY: torch.Tensor, X: torch.Tensor | None,
                        U: torch.Tensor | None, A: SparseMatrix, B: torch.Tensor, dx: bool = True,
                        da: bool = True, db: bool = True, dx_adapter: bool = True,
                        want_du: bool = False, ws: torch.Tensor | None = None,
                        out: dict | None = None):
    """Double-pruned backward with a fixed-fan-in adapter factor A (ELL [r, K]).  Returns dict with
    dX, dA_values (fp32 [r, k], A's ELL order), dB (and dU when want_du)."""
    lib = load()
    dev = _check_sparse(P, "P")
    K, N, dt = P.rows, P.cols, P.dtype
    if not isinstance(dY, torch.Tensor) or dY.dim() != 2:
        raise ValueError("dY must be a 2-D tensor [T, N]")
    T = dY.shape[0]
    _arg(dY, "dY", (T, N), dt, dev)
    r = _check_ffa_factor(A, K, dt, dev)
    _arg(B, "B", (N, r), dt, dev)
    if U is not None:
        _arg(U, "U", (T, r), torch.float32, dev)
    if X is not None:
        _arg(X, "X", (T, K), dt, dev)
    elif da or (db and U is None):
        raise ValueError("X is needed for dA, and for dB when U is not given")
    flags = (SRA_GRAD_DX if dx else 0) | (SRA_GRAD_DA if da else 0) | (SRA_GRAD_DB if db else 0)
    if not dx_adapter:
        flags |= SRA_DX_NO_ADAPTER
    out = dict(out or {})
    if dx and out.get("dX") is None:
        out["dX"] = torch.empty((T, K), dtype=dt, device=dev)
    if da and out.get("dA_values") is None:
        out["dA_values"] = torch.empty((r, A.k), dtype=torch.float32, device=dev)
    if db and out.get("dB") is None:
        out["dB"] = torch.empty((N, r), dtype=torch.float32, device=dev)
    if want_du and out.get("dU") is None:
        out["dU"] = torch.empty((T, r), dtype=torch.float32, device=dev)
    for key, shape, odt in (("dX", (T, K), dt), ("dA_values", (r, A.k), torch.float32),
                            ("dB", (N, r), torch.float32), ("dU", (T, r), torch.float32)):
        if out.get(key) is not None:
            _arg(out[key], f"out['{key}']", shape, odt, dev)
    dp, da_ = P.desc(), A.desc()
    nbytes = ctypes.c_size_t()
    check("sra_ffa_bwd_workspace", lib.sra_ffa_bwd_workspace(ctypes.byref(dp), T, ctypes.byref(da_),
                                                             flags, ctypes.byref(nbytes)))
    if ws is None or ws.numel() < nbytes.value:
        ws = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=dev)
    _arg(ws, "ws", (ws.numel(),), torch.uint8, dev)
    check("sra_sparse_lora_bwd_ffa", lib.sra_sparse_lora_bwd_ffa(
        ctypes.byref(dp), _p(dY), _p(X), T, _p(U), ctypes.byref(da_), _p(B), flags,
        _p(out.get("dX")), _p(out.get("dA_values")), _p(out.get("dB")), _p(out.get("dU")), _p(ws),
        ws.numel(), _stream(dev)))
    return out


def ffa_fwd_workspace(Ws: SparseMatrix, T: int, A: SparseMatrix) -> int:
    n = ctypes.c_size_t()
    dw, da = Ws.desc(), A.desc()
    check("sra_ffa_fwd_workspace", load().sra_ffa_fwd_workspace(ctypes.byref(dw), T, ctypes.byref(da),
                                                                ctypes.byref(n)))
    return n.value


def ffa_bwd_workspace(P: SparseMatrix, T: int, A: SparseMatrix,
                      flags: int = SRA_GRAD_DX | SRA_GRAD_DA | SRA_GRAD_DB) -> int:
    n = ctypes.c_size_t()
    dp, da = P.desc(), A.desc()
    check("sra_ffa_bwd_workspace", load().sra_ffa_bwd_workspace(ctypes.byref(dp), T, ctypes.byref(da),
                                                                flags, ctypes.byref(n)))
    return n.value


_ENGINES = {"smfmac": 0, "dense_mfma": 1}


def set_tuning(**knobs) -> None:
    """Tuning knobs of the calling thread (sra_set_tuning): spmm_config, spmm_splits, spmm_fuse,
    engine ("smfmac" or "dense_mfma"), decode_rows, rows_slices, grads_slices."""
    lib = load()
    for k, v in knobs.items():
        if k not in _abi.SRA_TUNE_KEYS:
            raise ValueError(f"unknown tuning knob {k}")
        if k == "engine" and isinstance(v, str):
            v = _ENGINES[v]
        check("sra_set_tuning", lib.sra_set_tuning(_abi.SRA_TUNE_KEYS[k], int(v)))


def reset_tuning() -> None:
    check("sra_set_tuning", load().sra_set_tuning(0, 0))


@contextmanager
def tuned(**knobs):
    """Run a block with the given tuning knobs, then restore every knob to its default."""
    set_tuning(**knobs)
    try:
        yield
    finally:
        reset_tuning()
