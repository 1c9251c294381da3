"""Fixed fan-in (FFI) selection and transpose -- CPU oracle (test infrastructure only).

Source: SQuAsh project update (fixed fan-in sparsity: every output row keeps
the same number of inputs, at arbitrary columns) and SLoPe paperlayer summary
§2.3 (a sparse format is kept for the weight and one for its transpose).

Readings: per row keep the k entries of largest magnitude, ties to the lower
column, exact storage-dtype magnitudes, +0 == -0.  ELL layout: ``vals[rows,k]``
and ``cols[rows,k]`` with columns ascending.  The transpose is the exact one
(no second pruning for FFI): CSR over the columns with ``row_ptr[cols+1]``,
output-row ids ascending inside each column.
"""
from __future__ import annotations

import numpy as np


def select(W: np.ndarray, k: int):
    """compress_ffi(W, k) -> (vals [rows,k], cols [rows,k] int16 ascending)."""
    rows, K = W.shape
    if not (1 <= k <= K) or K > 32767:
        raise ValueError("need 1 <= k <= K <= 32767")
    # descending magnitude; a stable sort keeps equal magnitudes in ascending column order
    order = np.argsort(-np.abs(W), axis=1, kind="stable")
    cols = np.sort(order[:, :k], axis=1)
    vals = np.take_along_axis(W, cols, axis=1)
    return vals, cols.astype(np.int16)


def to_dense(vals: np.ndarray, cols: np.ndarray, K: int) -> np.ndarray:
    rows = vals.shape[0]
    D = np.zeros((rows, K), dtype=vals.dtype)
    np.put_along_axis(D, cols.astype(np.int64), vals, axis=1)
    return D


def transpose(vals: np.ndarray, cols: np.ndarray, K: int):
    """ELL of Ws -> CSR of Ws^T: (row_ptr int32 [K+1], row_ids int16 [nnz], vals [nnz])."""
    rows, k = cols.shape
    r = np.repeat(np.arange(rows), k)
    c = cols.astype(np.int64).ravel()
    order = np.lexsort((r, c))            # by column, then by output row
    counts = np.bincount(c, minlength=K)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return row_ptr, r[order].astype(np.int16), vals.ravel()[order]


def csr_to_dense(row_ptr: np.ndarray, idx: np.ndarray, vals: np.ndarray, ncols: int) -> np.ndarray:
    rows = row_ptr.shape[0] - 1
    D = np.zeros((rows, ncols), dtype=vals.dtype)
    rr = np.repeat(np.arange(rows), np.diff(row_ptr))
    D[rr, idx.astype(np.int64)] = vals
    return D
