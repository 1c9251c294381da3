"""GPU parity of the sparse-training kernels against the oracle: sra_masked_weight_grad (the
stored-value gradient of a 2:4 weight, dWs = (dY^T X) o mask1 in Ws's value order, and the same
product in P's orientation) and sra_nm_axpby (beta A + gamma B on shared-pattern values, the
update step), with the transpose form refreshed after an update.
Floats: max |gpu - oracle| / (|oracle| + 1e-3) <= 2e-2 for bf16, 1e-5 for fp32."""
import numpy as np
import pytest
import torch

import sparse_rank_adapter_amd as sra
from oracle import layer as olayer
from oracle import nm as onm
from sra_inputs import WORKLOADS, Workload, layer_inputs
from tests._util import Report, f64

pytestmark = pytest.mark.gpu


def check_ws_and_p(wl, T=None, seed=0):
    inp = layer_inputs(wl, seed=seed, T=T)
    X, W, dY = (inp[k].cuda() for k in ("X", "W", "dY"))
    S = sra.compress(W)
    with_p = wl.N % 32 == 0  # the second prune groups along N
    P = sra.double_prune(S) if with_p else None
    gW = sra.masked_weight_grad(S, dY, X)
    gP = sra.masked_weight_grad(P, X, dY) if with_p else None
    torch.cuda.synchronize()
    X64, dY64 = f64(inp["X"]), f64(inp["dY"])
    K, N = wl.K, wl.N
    meta = S.meta.cpu().numpy().view(np.uint32)
    rep = Report(torch.bfloat16)
    rep.add("dWs", f64(gW), olayer.masked_weight_grad(dY64, X64, meta, 2, 4, K))
    if with_p:
        pmeta = P.meta.cpu().numpy().view(np.uint32)
        rep.add("dP", f64(gP), olayer.masked_weight_grad(X64, dY64, pmeta, 2, 4, N))
    rep.check()
    # the metadata the kernel read is the oracle's own mask (bit-exact)
    _, m_o, _ = onm.compress(f64(inp["W"]), 2, 4)
    assert np.array_equal(meta, m_o)


@pytest.mark.parametrize("T,K,N", [(37, 96, 40), (1, 64, 8), (300, 640, 384), (129, 160, 136),
                                   (64, 1024, 256), (513, 128, 992), (70, 96, 96)])
def test_masked_weight_grad_ragged(gpu, T, K, N):
    """Ragged tokens (a partial last 32-token stage), row and column tiles off the 64 x 128 grid
    (P's orientation where N allows the second prune)."""
    check_ws_and_p(Workload("wgrad", T=T, K=K, N=N, r=0, dtype="bf16", fmt="nm"), seed=T + K + N)


def test_masked_weight_grad_opt350m_full(gpu):
    check_ws_and_p(WORKLOADS["opt350m_fc1"])


def test_masked_weight_grad_zero_tokens(gpu):
    wl = Workload("wgrad0", T=4, K=64, N=32, r=0, dtype="bf16", fmt="nm")
    inp = layer_inputs(wl, seed=1)
    S = sra.compress(inp["W"].cuda())
    out = torch.full((32, 32), 7.0, dtype=torch.bfloat16, device="cuda")
    empty_r = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    empty_c = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    sra.masked_weight_grad(S, empty_r, empty_c, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 7, 8, 4097, 1 << 20])
def test_nm_axpby(gpu, dtype, n):
    """beta A + gamma B on value arrays (out of place and in place), tails past the 16-byte chunks."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(n)
    a = torch.randn(n, generator=g).to(tdt)
    b = torch.randn(n, generator=g).to(tdt)
    beta, gamma = 0.999, -0.0123
    out = sra.nm_axpby(beta, a.cuda(), gamma, b.cuda())
    ac = a.cuda()
    sra.nm_axpby(beta, ac, gamma, b.cuda(), out=ac)
    torch.cuda.synchronize()
    ref = olayer.nm_axpby(beta, f64(a), gamma, f64(b))
    rep = Report(tdt)
    rep.add("out", f64(out), ref)
    rep.add("in place", f64(ac), ref)
    rep.check()


def test_sparse_sgd_step_and_refresh(gpu):
    """One sparse training update on OPT-350M fc1: dWs from the masked weight gradient, the
    decayed SGD step on Ws's values (metadata untouched), then the transpose form refreshed by the
    double prune of the updated values -- P bit-exact against the oracle's double prune of the
    same values."""
    wl = WORKLOADS["opt350m_fc1"]
    inp = layer_inputs(wl, seed=5)
    X, W, dY = (inp[k].cuda() for k in ("X", "W", "dY"))
    S = sra.compress(W)
    meta0 = S.meta.clone()
    dWs = sra.masked_weight_grad(S, dY, X)
    lr, wd = 1e-3, 0.1
    vals0 = S.values.clone()
    sra.nm_axpby(1.0 - lr * wd, S.values, -lr, dWs, out=S.values)
    P = sra.double_prune(S)
    torch.cuda.synchronize()
    assert torch.equal(S.meta, meta0)
    rep = Report(torch.bfloat16)
    rep.add("Ws values", f64(S.values), olayer.nm_axpby(1.0 - lr * wd, f64(vals0), -lr, f64(dWs)))
    rep.check()
    v = f64(S.values)
    Pv, Pm, _, _ = onm.double_prune(v, S.meta.cpu().numpy().view(np.uint32), 2, 4, wl.K)
    assert np.array_equal(P.meta.cpu().numpy().view(np.uint32), Pm)
    assert np.array_equal(f64(P.values), Pv)
