"""GPU parity of the fixed-fan-in adapter factor (SQuAsh's variant) against the oracle.

The adapter's A [r, K] keeps exactly k inputs per row (sra_compress_ffi of a dense factor), B stays
dense; the layer's weight is 2:4 with its double-pruned backward.  Floats: max |gpu - oracle| /
(|oracle| + 1e-3) <= 2e-2 (bf16); the selected columns of A must match the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import sparse_rank_adapter_amd as sra
from oracle import ffi as offi
from oracle import layer as olayer
from oracle import nm as onm
from sra_inputs import WORKLOADS, Workload, layer_inputs
from tests._util import Report, bits, f64

pytestmark = pytest.mark.gpu


def run_squash(wl: Workload, seed=0, T=None, tiled=False):
    inp = layer_inputs(wl, seed=seed, T=T)
    X, W, Afull, B, dY = (inp[k].cuda() for k in ("X", "W", "A", "B", "dY"))
    k = wl.adapter_k
    print(f"squash {wl.name}: T={X.shape[0]} K={wl.K} N={wl.N} r={wl.r} k={k} tiled={tiled}", flush=True)
    A = sra.compress_ffi(Afull, k)
    if tiled:
        S, P = sra.compress_pair_tiled(W)
    else:
        S, P = sra.compress_pair(W)
    Y, U = sra.sparse_lora_fwd_ffa(S, X, A, B)
    g = sra.sparse_lora_bwd_ffa(P, dY, X, U, A, B, want_du=True)
    torch.cuda.synchronize()

    X64, W64, Af64, B64, dY64 = (f64(inp[n]) for n in ("X", "W", "A", "B", "dY"))
    av, ac = offi.select(Af64, k)
    assert np.array_equal(A.index.cpu().numpy(), ac), "A's selected columns differ from the oracle"
    assert np.array_equal(bits(A.values), bits(torch.from_numpy(av.astype(np.float32)).to(torch.bfloat16)))
    v, m, mask1 = onm.compress(W64, 2, 4)
    _, _, _, Wdp = onm.double_prune(v, m, 2, 4, wl.K)
    Yo, Uo = olayer.ffi_adapter_forward(X64, np.where(mask1, W64, 0.0), av, ac, B64)
    go = olayer.ffi_adapter_backward(dY64, X64, Wdp, av, ac, B64)
    rep = Report(torch.bfloat16)
    rep.add("Y", f64(Y), Yo)
    rep.add("U", U.cpu().numpy(), Uo)
    rep.add("dX", f64(g["dX"]), go["dX"])
    rep.add("dU", g["dU"].cpu().numpy(), go["dU"])
    rep.add("dB", g["dB"].cpu().numpy(), go["dB"])
    rep.add("dA_values", g["dA_values"].cpu().numpy(), go["dA_vals"])
    rep.check()
    return dict(S=S, P=P, A=A, X=X, B=B, dY=dY, U=U, Y=Y, g=g)


@pytest.mark.parametrize("T,K,N,r,k", [(300, 512, 256, 24, 40), (64, 256, 128, 8, 256),
                                       (17, 128, 96, 5, 3), (1, 64, 32, 2, 7)])
def test_squash_ragged(gpu, T, K, N, r, k):
    wl = Workload("squash_ragged", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm", adapter_k=k)
    run_squash(wl, seed=T + k)


def test_squash_opt350m_fc2_full(gpu):
    """The benchmark workload in full: rank 32, A keeps 768 of 4096 inputs per row."""
    run_squash(WORKLOADS["squash_opt350m_fc2"])


def test_squash_streaming_layout(gpu):
    wl = Workload("squash_tiled", T=512, K=1024, N=512, r=16, dtype="bf16", fmt="nm", adapter_k=100)
    run_squash(wl, seed=3, tiled=True)


def test_squash_full_fan_in_equals_dense_adapter(gpu):
    """k = K keeps every entry of A: the same kernels as the dense-adapter calls, equal bits."""
    wl = Workload("squash_full", T=256, K=256, N=128, r=16, dtype="bf16", fmt="nm", adapter_k=256)
    inp = layer_inputs(wl, seed=5)
    X, W, Af, B, dY = (inp[k].cuda() for k in ("X", "W", "A", "B", "dY"))
    A = sra.compress_ffi(Af, 256)
    S, P = sra.compress_pair(W)
    Y1, U1 = sra.sparse_lora_fwd_ffa(S, X, A, B)
    Y2, U2 = sra.sparse_lora_fwd(S, X, Af, B)
    g1 = sra.sparse_lora_bwd_ffa(P, dY, X, U1, A, B)
    g2 = sra.sparse_lora_bwd(P, dY, X, U2, Af, B)
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y1), bits(Y2)) and torch.equal(U1, U2)
    assert np.array_equal(bits(g1["dX"]), bits(g2["dX"]))
    assert torch.equal(g1["dB"], g2["dB"]) and torch.equal(g1["dA_values"], g2["dA"])


def test_squash_zero_tokens(gpu):
    wl = Workload("squash_t0", T=64, K=128, N=64, r=4, dtype="bf16", fmt="nm", adapter_k=16)
    inp = layer_inputs(wl, seed=1)
    W, Af, B = (inp[k].cuda() for k in ("W", "A", "B"))
    A = sra.compress_ffi(Af, 16)
    S, P = sra.compress_pair(W)
    X0 = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    dY0 = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    Y, _ = sra.sparse_lora_fwd_ffa(S, X0, A, B)
    g = sra.sparse_lora_bwd_ffa(P, dY0, X0, None, A, B,
                                out={"dA_values": torch.full((4, 16), 7.0, device="cuda"),
                                     "dB": torch.full((64, 4), 7.0, device="cuda")})
    torch.cuda.synchronize()
    assert Y.shape == (0, 64)
    assert not g["dA_values"].any() and not g["dB"].any()
