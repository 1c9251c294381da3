"""Every tile configuration of the 2:4 SpMM (register-staged, LDS-DMA pipelined, eight-wave, with
metadata super-stages, ping-pong), with and without a split of the reduction, against the oracle on
a ragged problem.

Without a split every configuration performs the same SMFMAC sequence per output element, so
results must also be bit-identical to the default plan's.
"""
import numpy as np
import pytest
import torch

import sparse_rank_adapter_amd as sra
from oracle import layer as olayer
from oracle import nm as onm
from sra_inputs import Workload, layer_inputs
from tests._util import Report, bits, f64

pytestmark = pytest.mark.gpu

CFGS = [3, 13, 14, 50, 51, 55, 61, 62]


@pytest.fixture(scope="module")
def problem(gpu):
    # K % 64 == 0 so the pipelined kernels apply; T, N ragged against every tile size
    wl = Workload("cfg", T=300, K=640, N=544, r=24, dtype="bf16", fmt="nm")
    inp = layer_inputs(wl, seed=21)
    X, W, A, B = (inp[k].cuda() for k in ("X", "W", "A", "B"))
    S = sra.compress(W)
    Y0, U0 = sra.sparse_lora_fwd(S, X, A, B)
    torch.cuda.synchronize()
    W64 = f64(inp["W"])
    v, m, mask1 = onm.compress(W64, 2, 4)
    Yo, _ = olayer.forward(f64(inp["X"]), np.where(mask1, W64, 0.0), f64(inp["A"]), f64(inp["B"]))
    return dict(S=S, X=X, A=A, B=B, Y0=Y0, Yo=Yo)


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("cfg", CFGS)
def test_config(problem, cfg, splits):
    with sra.tuned(spmm_config=cfg, spmm_splits=splits):
        Y, _ = sra.sparse_lora_fwd(problem["S"], problem["X"], problem["A"], problem["B"])
        torch.cuda.synchronize()
    rep = Report(torch.bfloat16)
    rep.add("Y", f64(Y), problem["Yo"])
    rep.check()
    if splits == 1:
        assert np.array_equal(bits(Y), bits(problem["Y0"]))


@pytest.mark.parametrize("splits", [2, -2])
def test_super_stage_split(gpu, splits):
    """The 256x256 tile with 4-stage metadata super-stages split over the reduction (two splits of
    8 stages each, fp32 partials summed in a fixed order; -2: only the tiles past the last whole
    wave of 256 split, here all six) on a ragged problem: within tolerance of the oracle, and the
    same bits on a second call."""
    wl = Workload("split", T=300, K=1024, N=544, r=24, dtype="bf16", fmt="nm")
    inp = layer_inputs(wl, seed=22)
    X, W, A, B = (inp[k].cuda() for k in ("X", "W", "A", "B"))
    S = sra.compress(W)
    with sra.tuned(spmm_config=61, spmm_splits=splits):
        Y, _ = sra.sparse_lora_fwd(S, X, A, B)
        Y2, _ = sra.sparse_lora_fwd(S, X, A, B)
        torch.cuda.synchronize()
    W64 = f64(inp["W"])
    _, _, mask1 = onm.compress(W64, 2, 4)
    Yo, _ = olayer.forward(f64(inp["X"]), np.where(mask1, W64, 0.0), f64(inp["A"]), f64(inp["B"]))
    rep = Report(torch.bfloat16)
    rep.add("Y", f64(Y), Yo)
    rep.check()
    assert np.array_equal(bits(Y), bits(Y2))
