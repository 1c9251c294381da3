"""GPU parity of the format kernels against the oracle: bit-exact values, metadata and indices.

compress (2:4), double_prune and compress_ffi + ffi_transpose, on tie-heavy and Gaussian inputs,
ragged shapes, and the full-size weights of the OPT-350M fc1, OPT-13B MLP, OPT-66B FFN and the
fixed fan-in 4096 x 4096 layer (full-size weights are checked on sampled rows / column groups,
which the oracle computes independently because both prunes are local to their groups).
"""
import numpy as np
import pytest
import torch

import sparse_rank_adapter_amd as sra
from oracle import ffi as offi
from oracle import nm as onm
from sra_inputs import WORKLOADS, Workload, layer_inputs
from tests._util import bits, f64, meta_u32, np_bits, tie_heavy

pytestmark = pytest.mark.gpu


def check_compress(W_cpu, dtype, rows_sample=None):
    Wg = W_cpu.cuda()
    S = sra.compress(Wg)
    torch.cuda.synchronize()
    W64 = f64(W_cpu)
    rows = np.arange(W64.shape[0]) if rows_sample is None else rows_sample
    vals, meta, mask1 = onm.compress(W64[rows], 2, 4)
    assert np.array_equal(bits(S.values[rows]), np_bits(vals, dtype))
    assert np.array_equal(meta_u32(S.meta[rows]), meta)
    return S


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(1, 32), (7, 64), (33, 96), (128, 1024), (300, 160)])
def test_compress_ties(gpu, dtype, shape):
    check_compress(tie_heavy(shape, seed=shape[0], dtype=dtype), dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_compress_gaussian_tiny(gpu, dtype):
    W = layer_inputs(WORKLOADS["tiny_f32"])["W"].to(dtype)
    check_compress(W, dtype)


def check_double_prune(W_cpu, dtype, col_groups=None):
    Wg = W_cpu.cuda()
    S = sra.compress(Wg)
    P = sra.double_prune(S)
    torch.cuda.synchronize()
    assert (P.rows, P.cols) == (W_cpu.shape[1], W_cpu.shape[0])
    W64 = f64(W_cpu)
    if col_groups is None:
        cols = np.arange(W64.shape[1])
    else:
        cols = (col_groups[:, None] * 4 + np.arange(4)[None, :]).ravel()
    sub = W64[:, cols]
    v, m, _ = onm.compress(sub, 2, 4)
    Pv, Pm, mask2, _ = onm.double_prune(v, m, 2, 4, sub.shape[1])
    assert np.array_equal(bits(P.values[cols]), np_bits(Pv, dtype))
    assert np.array_equal(meta_u32(P.meta[cols]), Pm)
    return S, P


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(32, 32), (32, 64), (64, 96), (160, 224), (256, 1024)])
def test_double_prune_ties(gpu, dtype, shape):
    check_double_prune(tie_heavy(shape, seed=7 + shape[1], dtype=dtype), dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(32, 32), (96, 160), (160, 224), (256, 1024)])
def test_compress_pair_matches_two_kernels(gpu, dtype, shape):
    """compress_pair (one pass) is bit-identical to compress then double_prune, and to the oracle."""
    W_cpu = tie_heavy(shape, seed=3 + shape[0], dtype=dtype)
    S, P = check_double_prune(W_cpu, dtype)
    S2, P2 = sra.compress_pair(W_cpu.cuda())
    torch.cuda.synchronize()
    assert (S2.rows, S2.cols, P2.rows, P2.cols) == (S.rows, S.cols, P.rows, P.cols)
    for a, b in ((S2.values, S.values), (P2.values, P.values)):
        assert np.array_equal(bits(a), bits(b))
    for a, b in ((S2.meta, S.meta), (P2.meta, P.meta)):
        assert np.array_equal(meta_u32(a), meta_u32(b))


def test_compress_pair_opt350m_fc1(gpu):
    W = layer_inputs(WORKLOADS["opt350m_fc1"], with_dy=False)["W"]
    S, P = check_double_prune(W, torch.bfloat16, col_groups=np.arange(0, 256, 7))
    S2, P2 = sra.compress_pair(W.cuda())
    torch.cuda.synchronize()
    for a, b in ((S2.values, S.values), (P2.values, P.values)):
        assert np.array_equal(bits(a), bits(b))
    for a, b in ((S2.meta, S.meta), (P2.meta, P.meta)):
        assert np.array_equal(meta_u32(a), meta_u32(b))


@pytest.mark.parametrize("shape", [(8192, 4096), (4224, 8000)])
def test_compress_pair_large_matches_two_kernels(gpu, shape):
    """At 2^25 elements and above the pair kernel stages each W tile through LDS before pruning
    (a ragged shape included): both outputs bit-identical to compress then double_prune, on the
    canonical arrays and, for the 128-aligned shape, in the streaming layout."""
    wl = Workload("pair_large", T=1, K=shape[1], N=shape[0], r=0, dtype="bf16", fmt="nm")
    W = layer_inputs(wl, seed=shape[0] + shape[1], with_dy=False)["W"].cuda()
    S = sra.compress(W)
    P = sra.double_prune(S)
    S2, P2 = sra.compress_pair(W)
    torch.cuda.synchronize()
    for a, b in ((S2.values, S.values), (P2.values, P.values)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for a, b in ((S2.meta, S.meta), (P2.meta, P.meta)):
        assert torch.equal(a, b)
    if shape[0] % 128 == 0 and shape[1] % 128 == 0:
        St, Pt = sra.compress_pair_tiled(W)
        Se, Pe = sra.nm_tile(S), sra.nm_tile(P)
        torch.cuda.synchronize()
        for a, b in ((St, Se), (Pt, Pe)):
            assert torch.equal(a.values.view(torch.int16), b.values.view(torch.int16))
            assert torch.equal(a.meta, b.meta)


def test_double_prune_tiny_f32(gpu):
    check_double_prune(layer_inputs(WORKLOADS["tiny_f32"])["W"], torch.float32)


def test_opt350m_fc1_formats_full(gpu):
    W = layer_inputs(WORKLOADS["opt350m_fc1"], with_dy=False)["W"]
    check_compress(W, torch.bfloat16)
    check_double_prune(W, torch.bfloat16)


@pytest.mark.parametrize("name", ["opt13b_fc1", "opt13b_fc2"])
def test_opt13b_formats_sampled(gpu, name):
    wl = WORKLOADS[name]
    W = layer_inputs(wl, T=1, with_dy=False)["W"]
    rng = np.random.default_rng(1)
    check_compress(W, torch.bfloat16, rows_sample=np.sort(rng.choice(wl.N, 512, replace=False)))
    check_double_prune(W, torch.bfloat16, col_groups=np.sort(rng.choice(wl.K // 4, 48, replace=False)))


def test_opt66b_decode_weight_formats_sampled(gpu):
    wl = WORKLOADS["opt66b_ffn_decode"]
    W = layer_inputs(wl, T=1, with_dy=False)["W"]
    rng = np.random.default_rng(2)
    rows = np.concatenate([[0, wl.N - 1], rng.choice(wl.N, 254, replace=False)])
    check_compress(W, torch.bfloat16, rows_sample=np.unique(rows))


# ----------------------------------------------------------------------------- fixed fan-in

def check_ffi(W_cpu, k, dtype):
    Wg = W_cpu.cuda()
    S = sra.compress_ffi(Wg, k)
    ST = sra.ffi_transpose(S)
    torch.cuda.synchronize()
    W64 = f64(W_cpu)
    vals, cols = offi.select(W64, k)
    assert np.array_equal(S.index.cpu().numpy(), cols)
    assert np.array_equal(bits(S.values), np_bits(vals, dtype))
    rp, ids, tv = offi.transpose(vals, cols, W64.shape[1])
    assert np.array_equal(ST.row_ptr.cpu().numpy(), rp)
    assert np.array_equal(ST.index.cpu().numpy(), ids)
    assert np.array_equal(bits(ST.values), np_bits(tv, dtype))
    return S, ST


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape,k", [((1, 1), 1), ((5, 37), 1), ((5, 37), 37), ((64, 300), 17),
                                     ((130, 1000), 123), ((3, 4096), 410)])
def test_ffi_ties(gpu, dtype, shape, k):
    check_ffi(tie_heavy(shape, seed=k + shape[1], dtype=dtype), k, dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ffi_gaussian(gpu, dtype):
    g = torch.Generator().manual_seed(3)
    W = (torch.randn(200, 2048, generator=g) * 0.02).to(dtype)
    check_ffi(W, 205, dtype)


def ffi_tile_expected(rows_of, cols_of, vbits, R, C):
    """The tiled fixed fan-in layout (documented with sra_ffi_tile) of entries (row, column, value
    bits): per 32-row group and 64-column stage a list of value | offset << 16 words in (row,
    column) order, the offset being the entry's byte in the group's swizzled 32 x 128-byte block,
    padded to four words with 0xffffffff; lists by group, then stage."""
    nst, groups = -(-C // 64), -(-R // 32)
    r = np.asarray(rows_of, dtype=np.int64)
    c = np.asarray(cols_of, dtype=np.int64)
    g, x = r // 32, c // 64
    lid = g * nst + x
    order = np.lexsort((c, r, lid))
    r, c, lid, vb = r[order], c[order], lid[order], np.asarray(vbits, dtype=np.uint32)[order]
    counts = np.bincount(lid, minlength=groups * nst)
    padded = (counts + 3) // 4 * 4
    starts = np.concatenate([[0], np.cumsum(padded)])
    first = np.concatenate([[0], np.cumsum(counts)])[:-1]
    rank = np.arange(lid.size) - first[lid]
    words = np.full(int(starts[-1]), 0xFFFFFFFF, dtype=np.uint32)
    i, cc = r - 32 * (r // 32), c - 64 * (c // 64)
    pos = (i * 128 + (((cc // 8) ^ ((i // 2) % 8)) * 16) + (cc % 8) * 2).astype(np.uint32)
    words[starts[lid] + rank] = vb | (pos << 16)
    offs = np.concatenate([starts[:-1], [starts[-1]] * 4]).astype(np.uint32)
    return words, offs


def check_ffi_tile(S, ST, vals, cols):
    """ffi_tile of the ELL weight and of its CSR transpose against the layout above, built from
    the oracle's selection and transpose."""
    R, C = S.rows, S.cols
    vb = np_bits(vals, torch.bfloat16).astype(np.uint32)
    rows_of = np.repeat(np.arange(R), vals.shape[1])
    for M, (ro, co, bb, RR, CC) in (
            (sra.ffi_tile(S), (rows_of, cols.reshape(-1), vb.reshape(-1), R, C)),
            (sra.ffi_tile(ST), _csr_entries(ST, vals, cols))):
        torch.cuda.synchronize()
        words, offs = ffi_tile_expected(ro, co, bb, RR, CC)
        got_o = M.meta.cpu().numpy().view(np.uint32)
        assert np.array_equal(got_o[:offs.size], offs)
        got_w = M.values.cpu().numpy().view(np.uint32)
        assert M.nnz >= words.size
        assert np.array_equal(got_w[:words.size], words)


def _csr_entries(ST, vals, cols):
    rp, ids, tv = offi.transpose(vals, cols, ST.rows)
    rows_of = np.repeat(np.arange(ST.rows), np.diff(rp))
    return rows_of, ids, np_bits(tv, torch.bfloat16).astype(np.uint32), ST.rows, ST.cols


@pytest.mark.parametrize("shape,k", [((1, 1), 1), ((5, 37), 3), ((64, 300), 17), ((100, 640), 600),
                                     ((300, 200), 20), ((70, 4096), 410)])
def test_ffi_tile_layout(gpu, shape, k):
    W = tie_heavy(shape, seed=k + shape[0], dtype=torch.bfloat16)
    S, ST = check_ffi(W, k, torch.bfloat16)
    vals, cols = offi.select(f64(W), k)
    check_ffi_tile(S, ST, vals, cols)


def test_ffi90_full(gpu):
    wl = WORKLOADS["ffi90_4096"]
    inp = layer_inputs(wl, T=1, with_dy=False)
    S, ST = check_ffi(inp["W"], wl.ffi_k, torch.bfloat16)
    assert np.array_equal(S.index.cpu().numpy().astype(np.int64), inp["ffi_cols"])
