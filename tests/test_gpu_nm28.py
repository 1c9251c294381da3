"""2:8 weights and the dense-MFMA engine for 2:4 weights, against the oracle (GPU, through the C ABI).

2:8: compress and double prune must match the oracle bit for bit (values and 3-bit metadata);
the layer's forward and double-pruned backward run rewritten as 2:4 on the SMFMAC kernels above 16
tokens, on the 2:8 decode kernel (fragments expanded to dense in registers) at 16 tokens or fewer,
and on dense MFMA with expanded fragments on the dense engine.  2:4 on
SRA_ENGINE_DENSE_MFMA: the same products as the SMFMAC path through the same pipeline, held to the
same tolerance.  Floats: max |gpu - oracle| / (|oracle| + 1e-3) <= 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

import sparse_rank_adapter_amd as sra
from sparse_rank_adapter_amd._abi import SRA_ERR_UNSUPPORTED, SraError
from oracle import layer as olayer
from oracle import nm as onm
from sra_inputs import WORKLOADS, Workload, layer_inputs
from tests._util import Report, bits, f64, meta_u32, np_bits, tie_heavy

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols,kind", [(64, 64, "gauss"), (96, 160, "ties"), (32, 32, "ties"),
                                            (256, 1024, "gauss"), (4096, 1024, "gauss")])
def test_compress_double_prune_2_8_bit_exact(gpu, rows, cols, kind):
    torch.manual_seed(rows + cols)
    if kind == "gauss":
        W = (torch.randn(rows, cols) * 0.02).to(torch.bfloat16)
    else:
        W = tie_heavy((rows, cols), seed=rows + cols)
    print(f"2:8 compress/double prune {rows}x{cols} {kind}", flush=True)
    S = sra.compress(W.cuda(), 2, 8)
    P = sra.double_prune(S)
    torch.cuda.synchronize()
    W64 = f64(W)
    v, m, mask1 = onm.compress(W64, 2, 8)
    Pv, Pm, mask2, _ = onm.double_prune(v, m, 2, 8, cols)
    assert np.array_equal(meta_u32(S.meta), m)
    assert np.array_equal(bits(S.values), np_bits(v, torch.bfloat16))
    assert np.array_equal(meta_u32(P.meta), Pm)
    assert np.array_equal(bits(P.values), np_bits(Pv, torch.bfloat16))


def test_lemma_2_1_on_gpu_2_8(gpu):
    """The fraction of all entries the GPU's second 2:8 prune removes on the OPT-350M fc1 weight
    (Gaussian, N(0, 0.02)): equal to the oracle's count (the masks are bit-exact), near the
    binomial model's 5.84% and far from the page's printed 3.39%."""
    wl = WORKLOADS["opt350m_fc1"]
    W = layer_inputs(wl, seed=0, T=1, with_dy=False)["W"].cuda()
    S = sra.compress(W, 2, 8)
    P = sra.double_prune(S)
    nz_s = int((S.values != 0).sum())
    nz_p = int((P.values != 0).sum())
    frac = (nz_s - nz_p) / W.numel()
    print(f"2:8 added zeros on the GPU: {frac:.5f}", flush=True)
    assert abs(frac - 0.05840) < 1.5e-3
    assert abs(frac - 0.0339) > 0.02


def run_layer(wl: Workload, n, m, seed=0, streaming=False, rows=None, tile28=False):
    """Forward + backward of an N:M layer against the oracle (sampled token rows optional).
    tile28: both 2:8 weights in their streaming layout (sra_nm_tile)."""
    inp = layer_inputs(wl, seed=seed)
    X, W, A, B, dY = (inp[k].cuda() for k in ("X", "W", "A", "B", "dY"))
    r = wl.r
    print(f"{n}:{m} layer T={wl.T} K={wl.K} N={wl.N} r={r} streaming={streaming}", flush=True)
    if streaming:
        S, P = sra.compress_pair_tiled(W)
    else:
        S = sra.compress(W, n, m)
        P = sra.double_prune(S)
        if tile28:
            S, P = sra.nm_tile(S), sra.nm_tile(P)
    Y, U = sra.sparse_lora_fwd(S, X, A if r else None, B if r else None)
    g = sra.sparse_lora_bwd(P, dY, X, U, A if r else None, B if r else None, want_du=True)
    torch.cuda.synchronize()
    X64, W64, A64, B64, dY64 = (f64(inp[k]) for k in ("X", "W", "A", "B", "dY"))
    rows = np.arange(wl.T) if rows is None else rows
    v, mm, mask1 = onm.compress(W64, n, m)
    _, _, _, Wdp = onm.double_prune(v, mm, n, m, wl.K)
    Yo, Uo = olayer.forward(X64[rows], np.where(mask1, W64, 0.0), A64, B64)
    go = olayer.backward(dY64[rows], X64[rows], Wdp, A64, B64, want=("dX", "dU"))
    rep = Report(torch.bfloat16)
    rep.add("Y", f64(Y[torch.from_numpy(rows).cuda()]), Yo)
    rep.add("dX", f64(g["dX"][torch.from_numpy(rows).cuda()]), go["dX"])
    if r:
        rep.add("U", U.cpu().numpy()[rows], Uo)
        rep.add("dU", g["dU"].cpu().numpy()[rows], go["dU"])
        gf = olayer.backward(dY64, X64, Wdp, A64, B64, want=("dA", "dB"))
        rep.add("dA", g["dA"].cpu().numpy(), gf["dA"])
        rep.add("dB", g["dB"].cpu().numpy(), gf["dB"])
    rep.check()


# K and N multiples of 128; ragged T against every tile; ranks with the adapter fused (<= 16) or
# not; few tokens (the 128x128 tile with a split reduction)
SHAPES = [(300, 256, 384, 24), (77, 128, 640, 5), (130, 384, 256, 1), (5, 512, 256, 8),
          (1030, 2048, 1536, 128), (257, 1024, 512, 0), (700, 1152, 640, 16)]


@pytest.mark.parametrize("engine", ["smfmac", "dense_mfma"])
@pytest.mark.parametrize("T,K,N,r", SHAPES)
def test_layer_2_8(gpu, T, K, N, r, engine):
    """2:8 weights rewritten as 2:4 for the SMFMAC kernels (more than 16 tokens; the default), and
    on the expanded-fragment dense-MFMA kernels."""
    with sra.tuned(engine=engine):
        run_layer(Workload("nm28", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm"), 2, 8, seed=T + K)


# shapes only the 2:4 route takes (K or N a multiple of 32, not of 128)
@pytest.mark.parametrize("T,K,N,r", [(100, 96, 160, 8), (257, 224, 96, 24), (40, 64, 32, 0)])
def test_layer_2_8_as_2_4_shapes(gpu, T, K, N, r):
    run_layer(Workload("nm28s", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm"), 2, 8, seed=T + N)


# The 2:8 decode kernel (T <= 16, forward and dX): K and N multiples of 32 but not of 128 or of
# the 512-column batch, row counts that leave the last workgroup's row tiles partly or wholly
# empty, one to sixteen tokens, ranks 0 to 136 (the epilogue's 32-column rounds, a partial last one)
DECODE_SHAPES = [(1, 96, 160, 8), (3, 608, 352, 0), (16, 1056, 224, 64), (7, 224, 992, 100),
                 (16, 5120, 2080, 16), (12, 160, 96, 136), (16, 256, 384, 16), (5, 512, 256, 8)]


@pytest.mark.parametrize("T,K,N,r", DECODE_SHAPES)
def test_layer_2_8_decode(gpu, T, K, N, r):
    run_layer(Workload("nm28d", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm"), 2, 8, seed=T + K + N)


def tile28_expected(vals, meta, R, C):
    """The 2:8 streaming layout restated from its definition: per (16-row tile t, 256-column batch b)
    block, 2 KB of values (chunk c of lane l = 16q + i: row 16t + i's stored values 64b + 16q + 8c ..
    +7, at element 512c + 8l) and 512 B of metadata (lane l: the row's words 8b + 2q, +1 at word
    2l), zeros past the matrix."""
    nt, nb = -(-R // 16), -(-C // 256)
    tv = np.zeros((nt, nb, 2, 64, 8), np.uint16)
    tm = np.zeros((nt, nb, 64, 2), np.uint32)
    vs, ms = C // 4, C // 32
    for t in range(nt):
        for b in range(nb):
            for l in range(64):
                q, i = divmod(l, 16)
                row = 16 * t + i
                if row >= R:
                    continue
                for c in range(2):
                    c0 = 64 * b + 16 * q + 8 * c
                    if c0 < vs:
                        tv[t, b, c, l] = vals[row, c0:c0 + 8]
                for e in range(2):
                    w = 8 * b + 2 * q + e
                    if w < ms:
                        tm[t, b, l, e] = meta[row, w]
    return tv.ravel(), tm.ravel()


@pytest.mark.parametrize("R,C", [(16, 32), (40, 288), (100, 608), (257, 1056)])
def test_nm_tile_2_8_layout(gpu, R, C):
    torch.manual_seed(R + C)
    W = (torch.randn(R, C) * 0.02).to(torch.bfloat16).cuda()
    S = sra.compress(W, 2, 8)
    Tt = sra.nm_tile(S)
    torch.cuda.synchronize()
    ev, em = tile28_expected(bits(S.values).reshape(R, C // 4).astype(np.uint16), meta_u32(S.meta), R, C)
    assert np.array_equal(bits(Tt.values).astype(np.uint16)[:ev.size], ev)
    assert np.array_equal(meta_u32(Tt.meta).ravel()[:em.size], em)


# both 2:8 weights in the streaming layout: the decode kernel reading its blocks (T <= 16, forward
# and dX) and, above 16 tokens, the blocks rewritten as canonical 2:4 for the SMFMAC kernels (or the
# dense engine's expanded-fragment kernels)
@pytest.mark.parametrize("T,K,N,r", [(1, 96, 160, 8), (16, 1056, 224, 64), (7, 224, 992, 100),
                                     (16, 5120, 2080, 16), (300, 256, 384, 24), (77, 608, 352, 5)])
def test_layer_2_8_tiled(gpu, T, K, N, r):
    run_layer(Workload("nm28t", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm"), 2, 8, seed=T + K, tile28=True)


def test_layer_2_8_tiled_dense_engine(gpu):
    with sra.tuned(engine="dense_mfma"):
        run_layer(Workload("nm28tx", T=130, K=384, N=256, r=8, dtype="bf16", fmt="nm"), 2, 8, seed=3,
                  tile28=True)


@pytest.mark.parametrize("tile28", [False, True])
def test_layer_2_8_decode_128_row_workgroups(gpu, tile28):
    """32768 output rows: the planner's pick is four waves of two row tiles (128-row workgroups, the
    one shape with the adapter prefetch), on the canonical arrays and on the streaming layout."""
    run_layer(Workload("nm28d128", T=4, K=256, N=32768, r=40, dtype="bf16", fmt="nm"), 2, 8, seed=11,
              tile28=tile28)


@pytest.mark.parametrize("rows", [3, 4, 9])
def test_layer_2_8_decode_row_tiles(gpu, rows):
    """Each workgroup shape of the 2:8 decode kernel (48, 64 or 144 weight rows), forced; the
    planner picks 48 for small layers and 144 at the OPT-66B FFN shape."""
    with sra.tuned(decode_rows=rows):
        run_layer(Workload("nm28dr", T=16, K=1568, N=1184, r=40, dtype="bf16", fmt="nm"), 2, 8, seed=rows)


@pytest.mark.parametrize("T", [1, 16])
def test_opt66b_decode_2_8_sampled(gpu, T):
    """The OPT-66B FFN weight (36864 x 9216) at 2:8, forward at decode token counts, on 514 sampled
    output columns (2:8 selection is local to each weight row, so the oracle compresses only those
    rows)."""
    wl = WORKLOADS["opt66b_ffn_decode"]
    inp = layer_inputs(wl, seed=0, T=T, with_dy=False)
    X, A, B = (inp[k].cuda() for k in ("X", "A", "B"))
    print(f"2:8 OPT-66B decode T={T}", flush=True)
    S = sra.compress(inp["W"].cuda(), 2, 8)
    Y, U = sra.sparse_lora_fwd(S, X, A, B)
    torch.cuda.synchronize()
    rng = np.random.default_rng(T)
    cols_n = np.unique(np.concatenate([[0, wl.N - 1], rng.choice(wl.N, 512, replace=False)]))
    W_n = f64(inp["W"][torch.from_numpy(cols_n)])
    _, _, mask1 = onm.compress(W_n, 2, 8)
    X64, A64, B64 = (f64(inp[k]) for k in ("X", "A", "B"))
    Yo, Uo = olayer.forward(X64, np.where(mask1, W_n, 0.0), A64, B64[cols_n])
    rep = Report(torch.bfloat16)
    rep.add("Y", f64(Y[:, torch.from_numpy(cols_n).cuda()]), Yo)
    rep.add("U", U.cpu().numpy(), Uo)
    rep.check()


def test_layer_2_8_opt350m_fc1(gpu):
    wl = WORKLOADS["opt350m_fc1"]
    run_layer(wl, 2, 8, rows=np.arange(0, wl.T, 7))


@pytest.mark.parametrize("T,K,N,r", SHAPES)
def test_layer_2_4_dense_engine(gpu, T, K, N, r):
    with sra.tuned(engine="dense_mfma"):
        run_layer(Workload("nm24x", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm"), 2, 4, seed=T + N)


@pytest.mark.parametrize("T,K,N,r", [(300, 256, 384, 24), (700, 1152, 640, 8), (16, 512, 256, 20)])
def test_layer_2_4_dense_engine_streaming(gpu, T, K, N, r):
    with sra.tuned(engine="dense_mfma"):
        run_layer(Workload("nm24xs", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm"), 2, 4, seed=T,
                  streaming=True)


def test_layer_2_4_dense_engine_tail_split(gpu):
    """The 256x256 tile with the tail split (the last wave's tiles split in two over the
    reduction) on the dense engine: 320 tiles of 256 x 256, the last 64 split."""
    wl = Workload("nm24x_tail", T=10240, K=2048, N=1024, r=8, dtype="bf16", fmt="nm")
    with sra.tuned(engine="dense_mfma"):
        run_layer(wl, 2, 4, seed=5, rows=np.array([0, 1, 255, 4097, 8191, 8192, 8500, 10239]))


def test_dense_engine_matches_smfmac_closely(gpu):
    """Same operands on both engines: the dense engine's Y differs from the SMFMAC one only by fp32
    summation order (both within a few bf16 ulps of each other)."""
    wl = WORKLOADS["opt350m_fc1"]
    inp = layer_inputs(wl, seed=0, with_dy=False)
    X, W, A, B = (inp[k].cuda() for k in ("X", "W", "A", "B"))
    S = sra.compress(W)
    Y1, U1 = sra.sparse_lora_fwd(S, X, A, B)
    with sra.tuned(engine="dense_mfma"):
        Y2, U2 = sra.sparse_lora_fwd(S, X, A, B)
    torch.cuda.synchronize()
    d = (Y1.float() - Y2.float()).abs()
    assert float(d.max()) <= 2 ** -6 * float(Y1.float().abs().max())
    assert torch.allclose(U1, U2, rtol=1e-5, atol=1e-5)


def test_2_8_rejections(gpu):
    W = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(SraError) as e:
        sra.compress(W.float(), 2, 8)
    assert e.value.status == SRA_ERR_UNSUPPORTED
    S = sra.compress(W, 2, 8)
    # Above 16 tokens the expanded-fragment product (dense engine) needs K % 128 == 0; the
    # default route (the weight as 2:4) and the decode kernel (16 tokens or fewer) take this K.
    X = torch.ones(300, 64, dtype=torch.bfloat16, device="cuda")
    with sra.tuned(engine="dense_mfma"):
        with pytest.raises(SraError) as e:
            sra.sparse_lora_fwd(S, X)
    assert e.value.status == SRA_ERR_UNSUPPORTED
    for T in (300, 16):
        Y, _ = sra.sparse_lora_fwd(S, X[:T])
        torch.cuda.synchronize()
        assert Y.shape == (T, 64) and not Y.float().abs().any()
    with pytest.raises(SraError):  # the streaming layout is 2:4 or 2:8
        sra.nm_tile(sra.compress(W, 1, 2))
    with pytest.raises(SraError):
        sra.compress_pair(W, 2, 8)
