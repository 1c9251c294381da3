"""1:2 weights on the GPU (SLoPe §2.1 N:M with N = 1, M = 2).  Compression and the double prune are
bit-exact against the oracle (ties included); the layer runs on the 2:4 kernels through the 1:2 ->
2:4 metadata encoding and matches the oracle's 1:2 layer within the float tolerances."""
import numpy as np
import pytest
import torch

import sparse_rank_adapter_amd as sra
from oracle import layer as olayer
from oracle import nm as onm
from sra_inputs import Workload, layer_inputs
from tests._util import Report, bits, f64

pytestmark = pytest.mark.gpu


def u32(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("R,C,ties", [(32, 64, False), (96, 160, False), (64, 256, True), (256, 1024, False)])
def test_compress_and_double_prune_12(gpu, dtype, R, C, ties):
    wl = Workload("nm12", T=1, K=C, N=R, r=0, dtype=dtype, fmt="nm")
    W = layer_inputs(wl, seed=R + C, with_dy=False)["W"]
    if ties:  # a four-value alphabet of magnitudes with both signs: many equal-magnitude pairs
        g = torch.Generator().manual_seed(R)
        W = (torch.randint(1, 5, W.shape, generator=g).float() * 0.25 *
             torch.where(torch.rand(W.shape, generator=g) < 0.5, -1.0, 1.0)).to(W.dtype)
    Wg = W.cuda()
    S = sra.compress(Wg, 1, 2)
    P = sra.double_prune(S)
    S2, P2 = sra.compress_pair(Wg, 1, 2)
    torch.cuda.synchronize()
    v, m, _ = onm.compress(f64(W), 1, 2)
    Pv, Pm, _, _ = onm.double_prune(v, m, 1, 2, C)
    assert np.array_equal(u32(S.meta), m) and np.array_equal(f64(S.values), v)
    assert np.array_equal(u32(P.meta), Pm) and np.array_equal(f64(P.values), Pv)
    for a, b in ((S, S2), (P, P2)):
        assert np.array_equal(bits(a.values), bits(b.values)) and torch.equal(a.meta, b.meta)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,K,N,r", [(300, 640, 384, 16), (5, 96, 64, 8), (129, 256, 160, 40),
                                     (2048, 1024, 4096, 16)])
def test_layer_12(gpu, dtype, T, K, N, r):
    print(f"1:2 layer {dtype} T={T} K={K} N={N} r={r}", flush=True)
    wl = Workload("nm12", T=T, K=K, N=N, r=r, dtype=dtype, fmt="nm")
    inp = layer_inputs(wl, seed=T + K)
    X, W, A, B, dY = (inp[k].cuda() for k in ("X", "W", "A", "B", "dY"))
    S = sra.compress(W, 1, 2)
    Y, U = sra.sparse_lora_fwd(S, X, A, B)
    P = sra.double_prune(S)
    g = sra.sparse_lora_bwd(P, dY, X, U, A, B, want_du=True)
    torch.cuda.synchronize()
    X64, W64, A64, B64, dY64 = (f64(inp[k]) for k in ("X", "W", "A", "B", "dY"))
    v, m, mask1 = onm.compress(W64, 1, 2)
    _, _, _, Wdp = onm.double_prune(v, m, 1, 2, K)
    Yo, Uo = olayer.forward(X64, np.where(mask1, W64, 0.0), A64, B64)
    go = olayer.backward(dY64, X64, Wdp, A64, B64)
    rep = Report(inp["X"].dtype)
    rep.add("Y", f64(Y), Yo)
    rep.add("U", U.cpu().numpy(), Uo)
    for k in ("dX", "dA", "dB", "dU"):
        rep.add(k, f64(g[k]) if g[k].dtype == torch.bfloat16 else g[k].cpu().numpy(), go[k])
    rep.check()


def test_masked_weight_grad_12(gpu):
    wl = Workload("nm12", T=257, K=512, N=192, r=0, dtype="bf16", fmt="nm")
    inp = layer_inputs(wl, seed=9)
    X, W, dY = (inp[k].cuda() for k in ("X", "W", "dY"))
    S = sra.compress(W, 1, 2)
    gW = sra.masked_weight_grad(S, dY, X)
    torch.cuda.synchronize()
    rep = Report(torch.bfloat16)
    rep.add("dWs", f64(gW), olayer.masked_weight_grad(f64(inp["dY"]), f64(inp["X"]), u32(S.meta), 1, 2, 512))
    rep.check()
