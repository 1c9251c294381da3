"""Seeded synthetic inputs for the sparse + low-rank linear layer.

This module is shared by the CPU oracle (tests, CPU baseline) and the GPU
path (tests, benchmark).  It only draws random numbers and rounds them to the
storage dtype; it holds none of the layer's arithmetic (no pruning, no
products).

Recipe (one PCG64 stream per tensor, spawned from ``SeedSequence(seed)`` in a
fixed order): draws are float64 ``standard_normal`` scaled by the stated
standard deviation, rounded to float32, then (for bf16 workloads) to bfloat16
with round-to-nearest-even.  ``X`` and ``dY`` are N(0, 1); weights and the
adapter factors are N(0, 0.02) (0.02 is the standard deviation).

The workload shapes mirror the layers the pages talk about: an OPT-350M fc1
layer, a 90%-sparse fixed-fan-in layer, the OPT-66B FFN at decode batch sizes
and the OPT-13B MLP (SLoPe paperlayer summary, §3 and §3.1; SQuAsh project
update).  No dataset, model or trained weight is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "draw", "layer_inputs", "ffi_weight", "to_storage"]


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens (rows of X)
    K: int            # input features (reduction dim of the forward)
    N: int            # output features
    r: int            # adapter rank
    dtype: str        # "bf16" or "f32"
    fmt: str          # "nm" (2:4 along K) or "ffi"
    n: int = 2
    m: int = 4
    ffi_k: int = 0
    adapter_k: int = 0   # > 0: the adapter's A keeps this many inputs per row (fixed fan-in)
    decode_T: tuple = field(default_factory=tuple)
    note: str = ""


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", T=8, K=64, N=32, r=4, dtype="f32", fmt="nm",
                         note="tiny fp32 check, fwd + double-pruned bwd"),
    "opt350m_fc1": Workload("opt350m_fc1", T=2048, K=1024, N=4096, r=16, dtype="bf16", fmt="nm",
                            note="OPT-350M fc1, 4 seqs x 512 tokens, 2:4, rank 16, fwd + bwd"),
    "ffi90_4096": Workload("ffi90_4096", T=4096, K=4096, N=4096, r=64, dtype="bf16", fmt="ffi",
                           ffi_k=410, note="fixed fan-in 410/4096 per row, rank 64, fwd + bwd"),
    "opt66b_ffn_decode": Workload("opt66b_ffn_decode", T=16, K=9216, N=36864, r=64, dtype="bf16",
                                  fmt="nm", decode_T=(1, 4, 16),
                                  note="OPT-66B FFN up-projection, 2:4, rank 64, decode T=1,4,16"),
    "squash_opt350m_fc2": Workload("squash_opt350m_fc2", T=2048, K=4096, N=1024, r=32, dtype="bf16",
                                   fmt="nm", adapter_k=768,
                                   note="OPT-350M fc2, 2:4, rank-32 adapter whose A keeps 768 of 4096 "
                                        "inputs per row: the adapter bytes of a dense rank-16 one"),
    "opt13b_fc1": Workload("opt13b_fc1", T=8192, K=5120, N=20480, r=128, dtype="bf16", fmt="nm",
                           note="OPT-13B MLP fc1, 2:4, rank 128"),
    "opt13b_fc2": Workload("opt13b_fc2", T=8192, K=20480, N=5120, r=128, dtype="bf16", fmt="nm",
                           note="OPT-13B MLP fc2, 2:4, rank 128"),
}


def _streams(seed: int, count: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(count)]


def to_storage(x64: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 draws -> float32 -> (bfloat16, RNE).  Returns a CPU tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t


def _normal(rng, shape, sd, dtype, chunk_rows=4096):
    """Normal draws rounded to the storage dtype, generated in row chunks to bound memory."""
    if len(shape) == 2 and shape[0] > chunk_rows:
        parts = []
        for r0 in range(0, shape[0], chunk_rows):
            rows = min(chunk_rows, shape[0] - r0)
            parts.append(to_storage(rng.standard_normal((rows, shape[1])) * sd, dtype))
        return torch.cat(parts, 0)
    return to_storage(rng.standard_normal(shape) * sd, dtype)


def draw(seed: int, specs):
    """specs: ordered list of (name, shape, sd, dtype).  One stream per entry, in order."""
    rngs = _streams(seed, len(specs))
    return {name: _normal(rng, shape, sd, dt) for rng, (name, shape, sd, dt) in zip(rngs, specs)}


def ffi_weight(rng, N: int, K: int, k: int, sd: float, dtype: str):
    """Dense N x K weight with exactly k nonzeros per row at uniformly random distinct columns.

    Returns (W dense storage tensor, sorted column sets int64 [N, k]).  Values that
    round to exactly zero are redrawn so every chosen column holds a nonzero.
    """
    cols = np.empty((N, k), dtype=np.int64)
    for r0 in range(0, N, 1024):
        rows = min(1024, N - r0)
        keys = rng.random((rows, K))
        cols[r0:r0 + rows] = np.sort(np.argpartition(keys, k - 1, axis=1)[:, :k], axis=1)
    vals = to_storage(rng.standard_normal((N, k)) * sd, dtype)
    while True:
        zero = (vals == 0)
        if not bool(zero.any()):
            break
        redraw = to_storage(rng.standard_normal(int(zero.sum())) * sd, dtype)
        vals[zero] = redraw
    W = torch.zeros((N, K), dtype=vals.dtype)
    W.scatter_(1, torch.from_numpy(cols), vals)
    return W, cols


def layer_inputs(wl: Workload, seed: int = 0, T: int | None = None, with_dy: bool = True):
    """Inputs of one layer call: X [T,K], W [N,K] (dense, before pruning), A [r,K], B [N,r], dY [T,N].

    Streams, in order: X, W, A, B, dY.  For the fixed-fan-in workload W already
    holds exactly ``ffi_k`` nonzeros per row and ``ffi_cols`` gives their columns.
    """
    T = wl.T if T is None else T
    rngs = _streams(seed, 5)
    out = {}
    out["X"] = _normal(rngs[0], (T, wl.K), 1.0, wl.dtype)
    if wl.fmt == "ffi":
        out["W"], out["ffi_cols"] = ffi_weight(rngs[1], wl.N, wl.K, wl.ffi_k, 0.02, wl.dtype)
    else:
        out["W"] = _normal(rngs[1], (wl.N, wl.K), 0.02, wl.dtype)
    out["A"] = _normal(rngs[2], (wl.r, wl.K), 0.02, wl.dtype)
    out["B"] = _normal(rngs[3], (wl.N, wl.r), 0.02, wl.dtype)
    if with_dy:
        out["dY"] = _normal(rngs[4], (T, wl.N), 1.0, wl.dtype)
    return out
