"""Forward and backward of the sparse + low-rank linear layer -- CPU oracle (test infrastructure only).

Sources (SLoPe paperlayer summary): §2.2 "Lazy low-rank adapters" -- the
(double-)pruned sparse weight is augmented by a low-rank term of rank r; §1
and §2.1 -- the backward input gradient uses the transposed weight after a
second N:M prune.  The low-rank term is LoRA ("efficient training for the
gpu-poor", section PEFT): a trainable rank-r product added to the frozen or
sparse base weight.

Shapes: X [T,K], Ws/Wdp [N,K] dense (pruned entries are zero), A [r,K],
B [N,r], Y and dY [T,N].  Readings: adapter scale 1, no bias, no activation;
U = X A^T stays unrounded.  Everything is float64; the caller compares after
the device's own output rounding.
"""
from __future__ import annotations

import numpy as np


def forward(X, Ws, A, B):
    """Y = X Ws^T + (X A^T) B^T.  Returns (Y, U) with U = X A^T."""
    U = X @ A.T
    Y = X @ Ws.T + U @ B.T
    return Y, U


def backward(dY, X, Wsub, A, B, U=None, dx_adapter=True, want=("dU", "dB", "dA", "dX")):
    """Gradients of L = sum(dY * Y) for the forward Y = X Wsub^T + (X A^T) B^T.

    For N:M weights ``Wsub`` is the double-pruned weight Wdp (so dX is the
    gradient of the substituted forward, not of the original one); for FFI
    weights it is Ws itself.  Returns dict with dU [T,r], dB [N,r], dA [r,K],
    dX [T,K].  ``dx_adapter=False`` drops the dU A term from dX.  ``want`` limits which are
    computed, so a caller can evaluate a restricted sub-problem cheaply.
    """
    out = {}
    dU = dY @ B
    if "dU" in want:
        out["dU"] = dU
    if "dB" in want:
        out["dB"] = dY.T @ (X @ A.T if U is None else U)
    if "dA" in want:
        out["dA"] = dU.T @ X
    if "dX" in want:
        dX = dY @ Wsub
        out["dX"] = dX + dU @ A if dx_adapter else dX
    return out


def rel_err(got, ref, floor=1e-3):
    """max |got - ref| / (|ref| + floor), the parity metric."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + floor)))


def masked_weight_grad(row_act, col_act, meta, n, m, cols):
    """Gradient of a compressed N:M matrix's stored values -- SLoPe's sparse training backward.

    Source (SLoPe paperlayer summary, §2.1 and §2.3): during sparse pretraining the N:M weight is
    trained with its mask fixed, so only the stored entries receive a gradient, which is the
    dense weight gradient dY^T X restricted to the mask and kept in the compressed value order.

    For a rows x cols matrix pruned along cols with metadata ``meta``:
        Out[row][i] = sum_t row_act[t][row] * col_act[t][c_i(row)]
    where c_i(row) is the column of the row's i-th stored entry (ascending).  For Ws (rows = N
    outputs, cols = K) row_act = dY [T,N] and col_act = X [T,K], so Out = (dY^T X) o mask1 in Ws's
    value order.  Written out as the masked dense product; float64.
    """
    from . import nm as _nm
    G = row_act.T @ col_act                         # rows x cols, dense
    rows = G.shape[0]
    _, stored = _nm.decompress(np.zeros((rows, cols // m * n)), meta, n, m, cols)
    return G[stored].reshape(rows, cols // m * n)


def nm_axpby(beta, a_vals, gamma, b_vals):
    """beta * A + gamma * B for two compressed matrices that share one N:M pattern (same metadata),
    computed on their value arrays -- SLoPe's optimizer-side sparse kernel for weight decay and
    the update step (SLoPe paperlayer summary, §2.3: a sparse addition of two matrices with the
    same pattern; §2.1: the mask stays fixed, so the metadata carries over unchanged).  float64."""
    return beta * np.asarray(a_vals, dtype=np.float64) + gamma * np.asarray(b_vals, dtype=np.float64)


def ffi_adapter_forward(X, Ws, A_vals, A_cols, B):
    """Forward with a fixed-fan-in adapter factor -- SQuAsh's variant (SQuAsh project update, first
    paragraph: one factor of the low-rank product is pruned with fixed fan-in so that a higher rank
    fits the same memory).  The pruned factor is the down-projection A [r,K]: row j keeps exactly k
    inputs, given as ELL values ``A_vals[r,k]`` and ascending columns ``A_cols[r,k]``.  With
    A_s = A_vals scattered to their columns,
        U = X A_s^T,   Y = X Ws^T + U B^T.
    Returns (Y, U).  float64."""
    from . import ffi as _ffi
    A = _ffi.to_dense(np.asarray(A_vals, dtype=np.float64), np.asarray(A_cols), X.shape[1])
    return forward(X, Ws, A, B)


def ffi_adapter_backward(dY, X, Wsub, A_vals, A_cols, B, U=None, dx_adapter=True):
    """Backward of ffi_adapter_forward: dU = dY B, dB = dY^T U, dX = dY Wsub + dU A_s, and the
    gradient of A's stored values only (the fixed fan-in mask is fixed, as the sparse weight's mask
    is in SLoPe §2.1), i.e. the dense dA = dU^T X read at each row's stored columns, in the ELL
    order: ``dA_vals[j][i] = sum_t dU[t][j] X[t][A_cols[j][i]]``.  Returns dict with dU, dB,
    dA_vals, dX.  float64."""
    from . import ffi as _ffi
    A = _ffi.to_dense(np.asarray(A_vals, dtype=np.float64), np.asarray(A_cols), X.shape[1])
    g = backward(dY, X, Wsub, A, B, U, dx_adapter)
    g["dA_vals"] = np.take_along_axis(g.pop("dA"), np.asarray(A_cols).astype(np.int64), axis=1)
    return g
