"""GPU parity of the layer calls (sparse_lora_fwd / sparse_lora_bwd) against the oracle.

Floats: max |gpu - oracle| / (|oracle| + 1e-3) <= 2e-2 for bf16 and <= 1e-5 for fp32.  Full-size
workloads compare sampled token rows / output columns that the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

import sparse_rank_adapter_amd as sra
from sparse_rank_adapter_amd._abi import SraError
from oracle import ffi as offi
from oracle import layer as olayer
from oracle import nm as onm
from sra_inputs import WORKLOADS, Workload, layer_inputs
from tests._util import Report, bits, f64

pytestmark = pytest.mark.gpu


def nm_oracle_weights(W64, k_groups=None):
    """(Ws, Wdp) dense float64 from the oracle; optionally only for some 4-column groups of K."""
    if k_groups is not None:
        cols = (k_groups[:, None] * 4 + np.arange(4)[None, :]).ravel()
        W64 = W64[:, cols]
    v, m, mask1 = onm.compress(W64, 2, 4)
    Ws = np.where(mask1, W64, 0.0)
    _, _, _, Wdp = onm.double_prune(v, m, 2, 4, W64.shape[1])
    return Ws, Wdp


def run_nm(wl: Workload, T=None, seed=0, rows=None, cols_n=None, k_groups=None, r=None,
           check_bwd=True, flags_adapter=True, tiled=False, streaming=False, same_decode=False):
    """Runs fwd + bwd on the GPU and compares (optionally on sampled token rows, output columns
    of Y / dB and 4-column groups of K for dX / dA).  tiled: the forward also runs on the
    streaming layout of the weight (sra_nm_tile), whose Y must equal the canonical one bit for bit
    when both run the same decode configuration (same_decode: the decode row tiles are forced
    by the caller's tuning).  streaming: forward and
    backward run on the streaming layouts of Ws and P instead of the canonical arrays."""
    inp = layer_inputs(wl, seed=seed, T=T)
    dtype = inp["X"].dtype
    if r is not None and r != wl.r:
        inp["A"], inp["B"] = inp["A"][:r].contiguous(), inp["B"][:, :r].contiguous()
    rr = inp["A"].shape[0]
    X, W, A, B, dY = (inp[k].cuda() for k in ("X", "W", "A", "B", "dY"))
    S = sra.compress(W)
    Sf = sra.nm_tile(S) if streaming else S
    Y, U = sra.sparse_lora_fwd(Sf, X, A if rr else None, B if rr else None)
    Yt = sra.sparse_lora_fwd(sra.nm_tile(S), X, A if rr else None, B if rr else None)[0] if tiled else None
    g = {}
    if check_bwd:
        P = sra.double_prune(S)
        if streaming:
            P = sra.nm_tile(P)
        g = sra.sparse_lora_bwd(P, dY, X, U, A if rr else None, B if rr else None,
                                dx_adapter=flags_adapter, want_du=True)
    torch.cuda.synchronize()

    X64, A64, B64, dY64 = (f64(inp[k]) for k in ("X", "A", "B", "dY"))
    Tn = X64.shape[0]
    rows = np.arange(Tn) if rows is None else rows
    cols_n = np.arange(wl.N) if cols_n is None else cols_n
    # forward: Y[rows][:, cols_n] needs Ws rows cols_n (mask1 is local to each row)
    Ws_n, _ = nm_oracle_weights(f64(inp["W"][torch.from_numpy(cols_n)]))
    Yo, Uo = olayer.forward(X64[rows], Ws_n, A64, B64[cols_n])
    rep = Report(dtype)
    rep.add("Y", f64(Y[rows][:, cols_n]), Yo)
    if tiled:
        # the same decode configuration on both layouts sums in the same order: equal bits; the
        # planner may give the layouts different workgroup shapes (another split of K), then
        # both are held to the tolerance only
        if same_decode:
            assert np.array_equal(bits(Yt), bits(Y)), "streaming-layout Y differs from the canonical Y"
        rep.add("Y (streaming layout)", f64(Yt[rows][:, cols_n]), Yo)
    if rr:
        rep.add("U", U[rows].cpu().numpy(), Uo)
    if not check_bwd:
        rep.check()
        return
    # backward, each output on a restricted problem the oracle solves independently:
    #   dX[rows][:, kcols], dU[rows]  -- token rows and K columns (Wdp columns are local to their
    #                                    4-column groups of K, the second prune to its column)
    #   dB[cols_n]                    -- output columns
    #   dA[:, kcols]                  -- K columns
    if k_groups is None:
        k_groups = np.arange(wl.K // 4)
    kcols = (k_groups[:, None] * 4 + np.arange(4)[None, :]).ravel()
    _, Wdp_k = nm_oracle_weights(f64(inp["W"]), k_groups)
    gx = olayer.backward(dY64[rows], X64[rows][:, kcols], Wdp_k, A64[:, kcols], B64,
                         dx_adapter=flags_adapter, want=("dX", "dU"))
    rep.add("dX", f64(g["dX"][rows][:, kcols]), gx["dX"])
    if rr:
        rep.add("dU", g["dU"][rows].cpu().numpy(), gx["dU"])
        gb = olayer.backward(dY64[:, cols_n], X64, None, A64, B64[cols_n], want=("dB",))
        rep.add("dB", g["dB"][cols_n].cpu().numpy(), gb["dB"])
        ga = olayer.backward(dY64, X64[:, kcols], None, A64[:, kcols], B64, want=("dA",))
        rep.add("dA", g["dA"][:, kcols].cpu().numpy(), ga["dA"])
    rep.check()


def test_tiny_f32_fwd_bwd(gpu):
    """The tiny fp32 check: X 8x64, W 32x64 pruned 2:4, rank 4, seed 0; tolerance 1e-5."""
    wl = WORKLOADS["tiny_f32"]
    run_nm(wl)


@pytest.mark.parametrize("T,K,N,r", [(1, 64, 32, 4), (5, 64, 96, 16), (130, 192, 160, 20),
                                     (257, 128, 64, 0), (64, 256, 256, 32), (300, 64, 32, 8),
                                     (33, 96, 64, 1), (100, 64, 96, 80), (70, 320, 192, 48),
                                     # T <= 16 takes the streaming decode kernel: half 64-column
                                     # steps (K or N % 64 == 32), ragged row tiles, 16 tokens
                                     (3, 96, 96, 24), (16, 160, 224, 8), (1, 32, 32, 0), (16, 512, 64, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_shapes(gpu, T, K, N, r, dtype):
    wl = Workload("ragged", T=T, K=K, N=N, r=r, dtype=dtype, fmt="nm")
    run_nm(wl, seed=T + K)


@pytest.mark.parametrize("cfg", [14, 55])
@pytest.mark.parametrize("T,K,N,r", [(300, 640, 384, 16), (77, 384, 640, 5), (130, 256, 128, 1)])
def test_in_kernel_adapter_rows(gpu, cfg, T, K, N, r):
    """Ranks <= 16 on the 128x64 tiles (32x32 and 16x16x64 forms) and the eight-wave 256x128 tiles:
    U (forward) and dU (backward, with dU^T's parts for dA and the zero columns past T) are
    computed inside the SpMM."""
    wl = Workload("fused", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm")
    with sra.tuned(spmm_config=cfg):
        run_nm(wl, seed=T + r)


@pytest.mark.parametrize("T,K,N,r", [(300, 640, 384, 40), (257, 512, 1024, 128), (520, 1280, 256, 100),
                                     (384, 256, 640, 136), (256, 64, 128, 64), (1030, 2048, 1536, 128)])
def test_adapter_rows_ring(gpu, T, K, N, r):
    """Ranks above 32 with at least 256 tokens and whole 64-column stages take the LDS-ring rows
    kernel for U and dU: ragged last token tile, adapter rows past r, two adapter-column blocks
    (r = 136), a single-stage reduction (K = 64), one to several reduction slices, and dU^T's
    parts with their zero columns past T."""
    wl = Workload("ring", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm")
    run_nm(wl, seed=T + r)


@pytest.mark.parametrize("fr", ["3", "4", "9"])
@pytest.mark.parametrize("T,K,N,r", [(16, 512, 200, 64), (5, 96, 100, 8), (1, 160, 3000, 0),
                                     (3, 1056, 52, 20), (16, 608, 300, 64)])
def test_decode_row_tiles(gpu, fr, T, K, N, r):
    """The decode kernel with 48-, 64- and 144-row workgroups: a ragged last row tile, waves
    without a row tile of their own (48 rows, four waves), half steps and batches past K, and the
    adapter epilogue; on the canonical arrays and on the streaming layout."""
    wl = Workload("decode_tiles", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm")
    with sra.tuned(decode_rows=int(fr)):
        run_nm(wl, seed=N + T, check_bwd=False, tiled=True, same_decode=True)


@pytest.mark.parametrize("T,K,N,r", [(300, 640, 384, 16), (77, 384, 640, 5), (130, 256, 128, 1),
                                     (200, 512, 256, 64), (33, 1024, 512, 0), (16, 512, 256, 20),
                                     (700, 1024, 640, 8), (1900, 1152, 2048, 8)])
def test_streaming_layout_layer(gpu, T, K, N, r):
    """Forward and double-pruned backward on the streaming layouts of Ws and P (any T when K and N
    are multiples of 128): fused and separate adapter rows, ragged tiles, the decode path."""
    wl = Workload("streaming", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm")
    run_nm(wl, seed=T + K + N, streaming=True)


@pytest.mark.parametrize("cfg", ["61", "62"])
@pytest.mark.parametrize("T,K,N,r", [(300, 640, 384, 16), (700, 1152, 640, 8)])
def test_streaming_layout_three_stage_wide(gpu, cfg, T, K, N, r):
    """The 256x256 tile with three stages and 4-stage metadata super-stages (32-byte pieces of the
    streaming layout's metadata blocks; K and N not multiples of 512, so a last super-stage is
    half past the end), also in the ping-pong schedule (62), on both layouts, forward and
    backward."""
    wl = Workload("wide3", T=T, K=K, N=N, r=r, dtype="bf16", fmt="nm")
    with sra.tuned(spmm_config=int(cfg)):
        run_nm(wl, seed=T + K, streaming=True)
        run_nm(wl, seed=T + K, streaming=False)


def test_split_reduction_both_layouts(gpu):
    """The 256x256 tile with its reduction split in two (8-stage aligned splits, fp32 partials
    summed in a fixed order) for the forward (K = 1024) and dX (N = 2048), on the canonical arrays
    and on the streaming layout, whose split starts its metadata at a 512-column batch."""
    wl = Workload("split2", T=300, K=1024, N=2048, r=8, dtype="bf16", fmt="nm")
    with sra.tuned(spmm_config=61, spmm_splits=2):
        run_nm(wl, seed=31, streaming=True)
        run_nm(wl, seed=31, streaming=False)


@pytest.mark.parametrize("T,N,streaming", [(10240, 2048, False), (10240, 2048, True), (10000, 2016, False)])
def test_tail_split(gpu, T, N, streaming):
    """Tail split: of the forward's 320 tiles of 256 x 256 the first 256 run whole (bf16 stores)
    and the last 64 (tokens 8192 on) split over the reduction into fp32 partials that a second
    kernel sums; the backward's tiles are all tail where it splits.  The ragged case ends in
    partial row and token tiles inside the tail.  Sampled token rows on both sides of the
    boundary, every output column."""
    wl = Workload("tail", T=T, K=1024, N=N, r=8, dtype="bf16", fmt="nm")
    rows = np.array([0, 1, 255, 4097, 8191, 8192, 8500, 9983, T - 1])
    with sra.tuned(spmm_config=61, spmm_splits=-2):
        run_nm(wl, seed=41, rows=rows, streaming=streaming)


@pytest.mark.parametrize("name", ["opt350m_fc1", "opt13b_fc2"])
def test_streaming_layout_bit_identical(gpu, name):
    """The streaming-layout SpMM performs the canonical kernels' SMFMAC sequence per output element,
    so Y, U, dX, dU, dA and dB equal the canonical path's bit for bit (where neither splits K)."""
    wl = WORKLOADS[name]
    T = min(wl.T, 2048)
    inp = layer_inputs(wl, seed=3, T=T)
    X, W, A, B, dY = (inp[k].cuda() for k in ("X", "W", "A", "B", "dY"))
    S, P = sra.compress_pair(W)
    out = []
    for Sx, Px in ((S, P), (sra.nm_tile(S), sra.nm_tile(P))):
        Y, U = sra.sparse_lora_fwd(Sx, X, A, B)
        g = sra.sparse_lora_bwd(Px, dY, X, U, A, B, want_du=True)
        out.append((Y, U, g["dX"], g["dU"], g["dA"], g["dB"]))
    torch.cuda.synchronize()
    for a, b, lab in zip(out[0], out[1], ("Y", "U", "dX", "dU", "dA", "dB")):
        assert np.array_equal(bits(a), bits(b)), f"{lab} differs between layouts"


def tile_layout_np(vals, meta, R, C):
    """The streaming layout as the header defines it, written with numpy reshapes: value block
    (t, s) holds in chunk 16q + i the stored values 32s + 8q .. +7 of row 16t + i; metadata block
    (t, b) holds at 64i the words 16b .. 16b + 15 of row 16t + i; zero past the edges."""
    nt, ns, nb = (R + 15) // 16, (C + 63) // 64, (C + 511) // 512
    vp = np.zeros((nt * 16, ns * 32), np.uint16)
    vp[:R, :C // 2] = vals.reshape(R, C // 2)
    mp = np.zeros((nt * 16, nb * 16), np.uint32)
    mp[:R, :C // 32] = meta.reshape(R, C // 32)
    tv = vp.reshape(nt, 16, ns, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    tm = mp.reshape(nt, 16, nb, 16).transpose(0, 2, 1, 3).reshape(-1)
    return tv, tm


@pytest.mark.parametrize("R,C", [(16, 64), (100, 96), (37, 608), (300, 2048), (48, 1056), (4096, 9216)])
def test_nm_tile_layout(gpu, R, C):
    """sra_nm_tile is a pure permutation of the canonical arrays (bit-exact, zero padding)."""
    wl = Workload("tile", T=1, K=C, N=R, r=0, dtype="bf16", fmt="nm")
    W = layer_inputs(wl, seed=R + C, with_dy=False)["W"].cuda()
    S = sra.compress(W)
    St = sra.nm_tile(S)
    torch.cuda.synchronize()
    tv, tm = tile_layout_np(S.values.view(torch.int16).cpu().numpy().view(np.uint16),
                            S.meta.cpu().numpy().view(np.uint32), R, C)
    gv = St.values.view(torch.int16).cpu().numpy().view(np.uint16)
    gm = St.meta.cpu().numpy().view(np.uint32)
    assert gv.size == tv.size and gm.size == tm.size
    assert np.array_equal(gv, tv) and np.array_equal(gm, tm)


@pytest.mark.parametrize("R,C", [(128, 128), (256, 640), (1024, 4096), (384, 1152)])
def test_compress_pair_tiled(gpu, R, C):
    """sra_compress_pair_tiled = sra_nm_tile of sra_compress_pair's outputs, bit for bit (partial
    512-column metadata batches included: their unused words are zero)."""
    wl = Workload("pair_tiled", T=1, K=C, N=R, r=0, dtype="bf16", fmt="nm")
    W = layer_inputs(wl, seed=R * 7 + C, with_dy=False)["W"].cuda()
    S, P = sra.compress_pair(W)
    St, Pt = sra.compress_pair_tiled(W)
    Se, Pe = sra.nm_tile(S), sra.nm_tile(P)
    torch.cuda.synchronize()
    for a, b in ((St, Se), (Pt, Pe)):
        assert (a.rows, a.cols, a.fmt) == (b.rows, b.cols, b.fmt)
        assert torch.equal(a.values.view(torch.int16), b.values.view(torch.int16))
        assert torch.equal(a.meta, b.meta)


def test_nm_tile_rejects_large_t(gpu):
    wl = Workload("tile", T=17, K=96, N=32, r=0, dtype="bf16", fmt="nm")
    inp = layer_inputs(wl, seed=0, with_dy=False)
    St = sra.nm_tile(sra.compress(inp["W"].cuda()))
    with pytest.raises(SraError, match="16 tokens"):
        sra.sparse_lora_fwd(St, inp["X"].cuda(), None, None)


def test_no_adapter_flag(gpu):
    wl = Workload("noad", T=96, K=128, N=64, r=8, dtype="bf16", fmt="nm")
    run_nm(wl, seed=5, flags_adapter=False)


def test_opt350m_fc1_full(gpu):
    run_nm(WORKLOADS["opt350m_fc1"])


@pytest.mark.parametrize("name", ["opt13b_fc1", "opt13b_fc2"])
def test_opt13b_sampled(gpu, name):
    wl = WORKLOADS[name]
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 62, replace=False)]))
    cols_n = np.unique(np.concatenate([[0, wl.N - 1], rng.choice(wl.N, 254, replace=False)]))
    k_groups = np.unique(np.concatenate([[0, wl.K // 4 - 1], rng.choice(wl.K // 4, 30, replace=False)]))
    run_nm(wl, rows=rows, cols_n=cols_n, k_groups=k_groups)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_opt66b_decode_sampled(gpu, T):
    wl = WORKLOADS["opt66b_ffn_decode"]
    rng = np.random.default_rng(T)
    cols_n = np.unique(np.concatenate([[0, wl.N - 1], rng.choice(wl.N, 510, replace=False)]))
    run_nm(wl, T=T, cols_n=cols_n, check_bwd=False, tiled=True)


def test_deterministic_and_t0(gpu):
    wl = Workload("det", T=200, K=256, N=128, r=16, dtype="bf16", fmt="nm")
    inp = layer_inputs(wl, seed=9)
    X, W, A, B, dY = (inp[k].cuda() for k in ("X", "W", "A", "B", "dY"))
    S = sra.compress(W)
    P = sra.double_prune(S)
    outs = []
    for _ in range(2):
        Y, U = sra.sparse_lora_fwd(S, X, A, B)
        g = sra.sparse_lora_bwd(P, dY, X, U, A, B, want_du=True)
        outs.append([Y.clone(), U.clone()] + [g[k].clone() for k in ("dX", "dA", "dB", "dU")])
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
    # T = 0: forward is a no-op, the backward writes zero adapter gradients
    X0, dY0 = X[:0], dY[:0]
    Y0, _ = sra.sparse_lora_fwd(S, X0, A, B)
    g0 = sra.sparse_lora_bwd(P, dY0, X0, None, A, B, out={"dA": torch.full_like(A, 7, dtype=torch.float32),
                                                          "dB": torch.full_like(B, 7, dtype=torch.float32)})
    torch.cuda.synchronize()
    assert Y0.shape == (0, wl.N) and g0["dX"].shape == (0, wl.K)
    assert torch.count_nonzero(g0["dA"]) == 0 and torch.count_nonzero(g0["dB"]) == 0


def test_u_recomputed_when_not_given(gpu):
    wl = Workload("rec", T=70, K=128, N=96, r=12, dtype="bf16", fmt="nm")
    inp = layer_inputs(wl, seed=11)
    X, W, A, B, dY = (inp[k].cuda() for k in ("X", "W", "A", "B", "dY"))
    S = sra.compress(W)
    P = sra.double_prune(S)
    _, U = sra.sparse_lora_fwd(S, X, A, B)
    g1 = sra.sparse_lora_bwd(P, dY, X, U, A, B)
    g2 = sra.sparse_lora_bwd(P, dY, X, None, A, B)
    torch.cuda.synchronize()
    assert np.array_equal(bits(g1["dX"]), bits(g2["dX"]))
    assert torch.equal(g1["dB"], g2["dB"]) and torch.equal(g1["dA"], g2["dA"])


# ----------------------------------------------------------------------------- fixed fan-in

def run_ffi(wl: Workload, T=None, seed=0, rows=None, cols_n=None, kcols=None, tiled=False):
    inp = layer_inputs(wl, seed=seed, T=T)
    dtype = inp["X"].dtype
    X, W, A, B, dY = (inp[k].cuda() for k in ("X", "W", "A", "B", "dY"))
    rr = A.shape[0]
    S = sra.compress_ffi(W, wl.ffi_k)
    ST = sra.ffi_transpose(S)
    if tiled:  # the products' tiled layout of both (sra_ffi_tile)
        S, ST = sra.ffi_tile(S), sra.ffi_tile(ST)
    Y, U = sra.sparse_lora_fwd(S, X, A if rr else None, B if rr else None)
    g = sra.sparse_lora_bwd(ST, dY, X, U, A if rr else None, B if rr else None, want_du=True)
    torch.cuda.synchronize()
    X64, W64, A64, B64, dY64 = (f64(inp[k]) for k in ("X", "W", "A", "B", "dY"))
    rows = np.arange(X64.shape[0]) if rows is None else rows
    cols_n = np.arange(wl.N) if cols_n is None else cols_n
    kcols = np.arange(wl.K) if kcols is None else kcols
    vals, cols = offi.select(W64, wl.ffi_k)
    Ws = offi.to_dense(vals, cols, wl.K)
    Yo, _ = olayer.forward(X64[rows], Ws[cols_n], A64, B64[cols_n])
    rep = Report(dtype)
    rep.add("Y", f64(Y[rows][:, cols_n]), Yo)
    gx = olayer.backward(dY64[rows], X64[rows][:, kcols], Ws[:, kcols], A64[:, kcols], B64,
                         want=("dX", "dU"))
    rep.add("dX", f64(g["dX"][rows][:, kcols]), gx["dX"])
    if rr:
        rep.add("dU", g["dU"][rows].cpu().numpy(), gx["dU"])
        gb = olayer.backward(dY64[:, cols_n], X64, None, A64, B64[cols_n], want=("dB",))
        rep.add("dB", g["dB"][cols_n].cpu().numpy(), gb["dB"])
        ga = olayer.backward(dY64, X64[:, kcols], None, A64[:, kcols], B64, want=("dA",))
        rep.add("dA", g["dA"][:, kcols].cpu().numpy(), ga["dA"])
    rep.check()


# (T >= 128 with the reduction a multiple of 64 runs the densified MFMA path: (257, 192, 320) in
# both directions, (130, 300, 64) in the backward, (300, 640, 200) in the forward)
@pytest.mark.parametrize("T,K,N,k,r", [(3, 37, 5, 7, 2), (130, 300, 64, 17, 16), (64, 512, 200, 64, 0),
                                       (257, 192, 320, 20, 16), (300, 640, 200, 40, 8)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ffi_ragged(gpu, T, K, N, k, r, dtype):
    wl = Workload("ffi_ragged", T=T, K=K, N=N, r=r, dtype=dtype, fmt="ffi", ffi_k=k)
    run_ffi(wl, seed=k)


def test_ffi90_sampled(gpu):
    wl = WORKLOADS["ffi90_4096"]
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 126, replace=False)]))
    cols = np.unique(np.concatenate([[0, wl.N - 1], rng.choice(wl.N, 254, replace=False)]))
    run_ffi(wl, rows=rows, cols_n=cols, kcols=cols)


# the tiled format (K % 64 == 0 and N % 64 == 0): T = 1 and 5 on the four-wave tile, lists of
# up to 256 entries, denser weights on the 1024-entry slots (k = 60 of 128: about 940 per list),
# and lists longer than the slots (k = 250 of 256: about 2000 per list, the rest read from memory)
@pytest.mark.parametrize("T,K,N,k,r", [(1, 64, 64, 5, 4), (5, 128, 192, 9, 4), (257, 192, 320, 20, 16),
                                       (130, 640, 64, 40, 0), (300, 128, 256, 60, 8),
                                       (200, 256, 320, 250, 8)])
def test_ffi_tiled_ragged(gpu, T, K, N, k, r):
    wl = Workload("ffi_tiled", T=T, K=K, N=N, r=r, dtype="bf16", fmt="ffi", ffi_k=k)
    run_ffi(wl, seed=k, tiled=True)


def test_ffi_tiled_wide_and_ffi90(gpu):
    """The tiled format on the 256 x 256 and 256 x 128 tiles: the ragged wide case below, and the
    90% fixed fan-in layer at full size on sampled outputs."""
    wl = Workload("ffi_wide", T=3900, K=3904, N=3968, r=16, dtype="bf16", fmt="ffi", ffi_k=100)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([np.arange(3840, 3900), rng.choice(3840, 60, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(3840, 3968), rng.choice(3840, 64, replace=False)]))
    kcols = np.unique(np.concatenate([np.arange(3840, 3904), rng.choice(3840, 64, replace=False)]))
    run_ffi(wl, seed=4, rows=rows, cols_n=cols, kcols=kcols, tiled=True)
    wl = WORKLOADS["ffi90_4096"]
    rows = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 126, replace=False)]))
    cols = np.unique(np.concatenate([[0, wl.N - 1], rng.choice(wl.N, 254, replace=False)]))
    run_ffi(wl, rows=rows, cols_n=cols, kcols=cols, tiled=True)
    wl = Workload("ffi_mid", T=1500, K=1024, N=2048, r=8, dtype="bf16", fmt="ffi", ffi_k=96)
    run_ffi(wl, seed=9, tiled=True)


def test_ffi_ragged_wide_tiles(gpu):
    """Token and row counts large enough for the densified product's 256 x 256 tiles in both
    directions (forward rows N = 3968, backward rows K = 3904, T = 3900), each with a ragged last
    tile; sampled outputs include every token, row and column of the ragged tails."""
    wl = Workload("ffi_wide", T=3900, K=3904, N=3968, r=16, dtype="bf16", fmt="ffi", ffi_k=100)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([np.arange(3840, 3900), rng.choice(3840, 60, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(3840, 3968), rng.choice(3840, 64, replace=False)]))
    kcols = np.unique(np.concatenate([np.arange(3840, 3904), rng.choice(3840, 64, replace=False)]))
    run_ffi(wl, seed=3, rows=rows, cols_n=cols, kcols=kcols)


@pytest.mark.parametrize("layout", ["canonical", "streaming"])
def test_mlp_chain(gpu, layout):
    """The OPT-13B MLP chain at a reduced size (hidden 256, FFN 1024, rank 16, 300 tokens): fc1
    forward on X, fc2 forward on fc1's bf16 Y, fc2 backward on dY2, fc1 backward on fc2's bf16 dX,
    no activation between the layers.  Each call is held to the tolerance against the oracle fed
    that call's actual GPU inputs (Y1 and dX2 as the GPU produced them), so one-ulp bf16
    differences upstream do not count against the next layer."""
    T, H, F, r = 300, 256, 1024, 16
    w1 = Workload("mlp_fc1", T=T, K=H, N=F, r=r, dtype="bf16", fmt="nm")
    w2 = Workload("mlp_fc2", T=T, K=F, N=H, r=r, dtype="bf16", fmt="nm")
    i1, i2 = layer_inputs(w1, seed=5, with_dy=False), layer_inputs(w2, seed=6)
    X, W1, A1, B1 = (i1[k].cuda() for k in ("X", "W", "A", "B"))
    W2, A2, B2, dY2 = (i2[k].cuda() for k in ("W", "A", "B", "dY"))
    tiled = layout == "streaming"
    S1, P1 = sra.compress_pair_tiled(W1) if tiled else sra.compress_pair(W1)
    S2, P2 = sra.compress_pair_tiled(W2) if tiled else sra.compress_pair(W2)
    Y1, U1 = sra.sparse_lora_fwd(S1, X, A1, B1)
    Y2, U2 = sra.sparse_lora_fwd(S2, Y1, A2, B2)
    g2 = sra.sparse_lora_bwd(P2, dY2, Y1, U2, A2, B2)
    g1 = sra.sparse_lora_bwd(P1, g2["dX"], X, U1, A1, B1)
    torch.cuda.synchronize()

    rep = Report(torch.bfloat16)
    for name, Win, Xin, Ain, Bin, Yg, Ug, dYin, g in (
            ("fc1", W1, X, A1, B1, Y1, U1, g2["dX"], g1),
            ("fc2", W2, Y1, A2, B2, Y2, U2, dY2, g2)):
        W64, X64, A64, B64, dY64 = (f64(t.cpu()) for t in (Win, Xin, Ain, Bin, dYin))
        Ws, Wdp = nm_oracle_weights(W64)
        Yo, Uo = olayer.forward(X64, Ws, A64, B64)
        rep.add(f"{name} Y", f64(Yg), Yo)
        rep.add(f"{name} U", Ug.cpu().numpy(), Uo)
        go = olayer.backward(dY64, X64, Wdp, A64, B64, want=("dX", "dA", "dB"))
        for k in ("dX", "dA", "dB"):
            rep.add(f"{name} {k}", f64(g[k]) if k == "dX" else g[k].cpu().numpy(), go[k])
    rep.check()
