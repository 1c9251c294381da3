"""sra_sparse_lora_bwd_noalloc against sra_sparse_lora_bwd (GPU, through the C ABI).

The allocation-free entry point runs the same kernels with the library's fixed per-GPU array as
workspace, so its outputs must equal the workspace entry point's bit for bit.  Two calls in a row,
the second on a smaller problem, so the second sees the first call's leftovers in the array.
"""
import pytest
import torch

import sparse_rank_adapter_amd as sra
from sparse_rank_adapter_amd._abi import SRA_ERR_WORKSPACE, SRA_FMT_NM, SraError
from sra_inputs import Workload, layer_inputs

from _util import bits

pytestmark = pytest.mark.gpu


def _problem(gpu, T, K, N, r, seed):
    wl = Workload("noalloc", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm")
    inp = layer_inputs(wl, seed=seed)
    X, W, A, B, dY = (inp[k].to(gpu) for k in ("X", "W", "A", "B", "dY"))
    S, P = sra.compress_pair(W)
    _, U = sra.sparse_lora_fwd(S, X, A, B)
    return dict(P=P, dY=dY, X=X, U=U, A=A, B=B)


def _same(a, b):
    assert a.keys() == b.keys()
    for k in a:
        assert (bits(a[k]) == bits(b[k])).all(), f"{k} differs between the two entry points"


CASES = [
    # (T, K, N, r, with_u, want_du): the OPT-350M fc1 backward, then a smaller, ragged one
    (2048, 1024, 4096, 16, True, False),
    (300, 256, 512, 8, False, True),
]


def test_noalloc_matches_workspace_entry_point(gpu):
    torch.cuda.synchronize()
    for i, (T, K, N, r, with_u, want_du) in enumerate(CASES):
        print(f"noalloc case {i}: T={T} K={K} N={N} r={r} U={'given' if with_u else 'recomputed'}",
              flush=True)
        p = _problem(gpu, T, K, N, r, seed=10 + i)
        U = p["U"] if with_u else None
        ref = sra.sparse_lora_bwd(p["P"], p["dY"], p["X"], U, p["A"], p["B"], want_du=want_du)
        got = sra.sparse_lora_bwd(p["P"], p["dY"], p["X"], U, p["A"], p["B"], want_du=want_du,
                                  noalloc=True)
        torch.cuda.synchronize()
        _same(ref, got)


def test_noalloc_rejects_oversized_call(gpu):
    # OPT-13B fc1 backward (rank 128, 8192 tokens) needs far more than the fixed array holds
    T, K, N, r = 8192, 5120, 20480, 128
    P = sra.SparseMatrix(SRA_FMT_NM, torch.bfloat16, K, N,
                         torch.empty((K, N // 2), dtype=torch.bfloat16, device=gpu),
                         meta=torch.empty((K, N // 32), dtype=torch.int32, device=gpu))
    dY = torch.empty((T, N), dtype=torch.bfloat16, device=gpu)
    X = torch.empty((T, K), dtype=torch.bfloat16, device=gpu)
    A = torch.empty((r, K), dtype=torch.bfloat16, device=gpu)
    B = torch.empty((N, r), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(SraError) as e:
        sra.sparse_lora_bwd(P, dY, X, None, A, B, noalloc=True)
    assert e.value.status == SRA_ERR_WORKSPACE
