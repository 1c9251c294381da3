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
