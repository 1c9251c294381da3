"""N:M pruning, compressed format and double pruning -- CPU oracle (test infrastructure only).

Source: SLoPe paperlayer summary.  §2.1 "Double-pruned backward pass": the
weight is N:M pruned once at initialisation with a mask kept fixed; for the
backward pass the pruned weight is transposed and N:M-pruned a second time,
so the reduction dimension of the input-gradient product is N:M structured
too.  §2.3 keeps compressed formats for both the weight and its transpose.

Readings taken where the page is silent:
* the first mask keeps, in each group of M consecutive entries along the
  input (reduction) dim, the N entries of largest magnitude; ties go to the
  lower index; +0 and -0 have equal magnitude.  Magnitudes are compared
  exactly in the storage dtype (inputs arrive as float64 holding exact
  bf16/fp32 values, so ``abs`` in float64 is exact);
* the second prune uses the same N:M, groups along the output dim, and only
  entries kept by the first mask may be kept again, so mask2 is a subset of
  mask1; the same magnitude/lower-index rule ranks them;
* a group of the second prune with fewer than N eligible entries is padded
  with the lowest unused in-group indices holding +0.0, so every stored group
  has exactly N ascending indices.

Compressed format ("nm"): for a rows x cols matrix pruned along cols,
``values[rows, cols*N/M]`` holds the kept entries of each row in ascending
column order; ``meta`` (uint32 words) holds each kept entry's in-group index:
* M <= 4: a 2-bit field per kept entry, fields in kept order, packed
  least-significant first, 16 per word, unused high fields zero
  (``ceil(cols*N/M/16)`` words per row);
* M = 8 (N <= 2): a 3-bit field per kept entry; the N fields of one group share
  one byte (field i at bits 3i, the rest zero), groups in column order, four
  bytes per word least-significant first (``ceil(cols/32)`` words per row).
  This layout is this library's reading: the pages give 2:8 only as a pattern
  (SLoPe §2.1, Lemma 2.1) and no storage format for it.
"""
from __future__ import annotations

import numpy as np

FIELD_BITS = 2
FIELDS_PER_WORD = 16
GROUPS_PER_WORD_M8 = 4    # M = 8: one byte per group


def meta_words_per_row(cols: int, n: int, m: int) -> int:
    if m == 8:
        groups = cols // m
        return (groups + GROUPS_PER_WORD_M8 - 1) // GROUPS_PER_WORD_M8
    fields = cols // m * n
    return (fields + FIELDS_PER_WORD - 1) // FIELDS_PER_WORD


def _check(cols: int, n: int, m: int):
    if not (1 <= n <= m <= 4 or (m == 8 and 1 <= n <= 2)):
        raise ValueError("oracle supports 1 <= n <= m <= 4, and 1:8 / 2:8")
    if cols % m:
        raise ValueError("grouped dimension must be a multiple of m")


def group_ranks(mag: np.ndarray, eligible: np.ndarray | None = None) -> np.ndarray:
    """Rank of every entry inside its group (last axis = in-group position).

    rank[a] = number of entries j of the same group that outrank a, where j
    outranks a iff j is eligible and (|w_j| > |w_a|, or |w_j| == |w_a| and
    j < a).  Ineligible entries never outrank anything.
    """
    m = mag.shape[-1]
    mj = mag[..., :, None]
    ma = mag[..., None, :]
    lower = np.arange(m)[:, None] < np.arange(m)[None, :]
    outranks = (mj > ma) | ((mj == ma) & lower)
    if eligible is not None:
        outranks &= eligible[..., :, None]
    return outranks.sum(axis=-2)


def nm_mask(W: np.ndarray, n: int, m: int, chunk_rows: int = 2048) -> np.ndarray:
    """mask1: keep the n largest-magnitude entries of each m-group along the last axis."""
    rows, cols = W.shape
    _check(cols, n, m)
    out = np.empty((rows, cols), dtype=bool)
    for r0 in range(0, rows, chunk_rows):
        g = np.abs(W[r0:r0 + chunk_rows]).reshape(-1, cols // m, m)
        out[r0:r0 + chunk_rows] = (group_ranks(g) < n).reshape(-1, cols)
    return out


def pack_fields(fields: np.ndarray, n: int = 2, m: int = 4) -> np.ndarray:
    """fields[rows, F] (in-group indices, F = groups * n) -> uint32 words, LSB-first.

    M <= 4: 2-bit fields, 16 per word.  M = 8: 3-bit fields, one byte per group, 4 per word."""
    if m == 8:
        rows, F = fields.shape
        G = F // n
        f = fields.reshape(rows, G, n).astype(np.uint64)
        byte = (f << (np.arange(n, dtype=np.uint64) * 3)).sum(axis=-1)        # [rows, G]
        words = (G + GROUPS_PER_WORD_M8 - 1) // GROUPS_PER_WORD_M8
        padded = np.zeros((rows, words * GROUPS_PER_WORD_M8), dtype=np.uint64)
        padded[:, :G] = byte
        padded = padded.reshape(rows, words, GROUPS_PER_WORD_M8)
        return (padded << (np.arange(GROUPS_PER_WORD_M8, dtype=np.uint64) * 8)).sum(-1).astype(np.uint32)
    rows, F = fields.shape
    words = (F + FIELDS_PER_WORD - 1) // FIELDS_PER_WORD
    padded = np.zeros((rows, words * FIELDS_PER_WORD), dtype=np.uint64)
    padded[:, :F] = fields
    padded = padded.reshape(rows, words, FIELDS_PER_WORD)
    shifts = (np.arange(FIELDS_PER_WORD, dtype=np.uint64) * FIELD_BITS)
    return (padded << shifts).sum(axis=-1).astype(np.uint32)


def unpack_fields(meta: np.ndarray, F: int, n: int = 2, m: int = 4) -> np.ndarray:
    """Inverse of pack_fields: the first F fields of every row."""
    rows, words = meta.shape
    if m == 8:
        G = F // n
        byte = (meta.astype(np.uint64)[..., None] >> (np.arange(GROUPS_PER_WORD_M8, dtype=np.uint64) * 8)) & 255
        byte = byte.reshape(rows, words * GROUPS_PER_WORD_M8)[:, :G]
        f = (byte[..., None] >> (np.arange(n, dtype=np.uint64) * 3)) & 7
        return f.reshape(rows, G * n).astype(np.int64)
    shifts = (np.arange(FIELDS_PER_WORD, dtype=np.uint64) * FIELD_BITS)
    f = (meta.astype(np.uint64)[..., None] >> shifts) & 3
    return f.reshape(rows, words * FIELDS_PER_WORD)[:, :F].astype(np.int64)


def encode(W: np.ndarray, keep: np.ndarray, n: int, m: int, pad_zero: bool = False):
    """Compress a matrix whose kept set has exactly n entries per group.

    ``keep`` marks the stored positions (after any padding).  If ``pad_zero`` is
    given as a boolean array, stored positions flagged there hold +0.0.
    """
    rows, cols = W.shape
    G = cols // m
    kg = keep.reshape(rows, G, m)
    if not np.all(kg.sum(-1) == n):
        raise AssertionError("every group must store exactly n entries")
    vals = W[keep].reshape(rows, G * n).copy()
    if pad_zero is not False:
        vals[pad_zero[keep].reshape(rows, G * n)] = 0.0
    pos = np.nonzero(kg)[2].reshape(rows, G * n)   # ascending in-group positions, row-major order
    return vals, pack_fields(pos, n, m)


def compress(W: np.ndarray, n: int, m: int):
    """compress(W, N, M) -> (values, meta, mask1).  Rows are pruned along columns."""
    mask1 = nm_mask(W, n, m)
    vals, meta = encode(W, mask1, n, m)
    return vals, meta, mask1


def decompress(vals: np.ndarray, meta: np.ndarray, n: int, m: int, cols: int):
    """Canonical arrays -> (dense matrix, stored-position bitmap)."""
    rows = vals.shape[0]
    G = cols // m
    pos = unpack_fields(meta, G * n, n, m).reshape(rows, G, n)
    col = (np.arange(G)[None, :, None] * m + pos).reshape(rows, G * n)
    dense = np.zeros((rows, cols), dtype=vals.dtype)
    stored = np.zeros((rows, cols), dtype=bool)
    r = np.repeat(np.arange(rows), G * n)
    dense[r, col.ravel()] = vals.ravel()
    stored[r, col.ravel()] = True
    return dense, stored


def double_prune(vals: np.ndarray, meta: np.ndarray, n: int, m: int, cols: int):
    """P = prune_NM(Ws^T) from the compressed Ws (rows = outputs, cols = inputs).

    Returns (P_values, P_meta, mask2, Wdp) where P is cols x rows compressed
    along the original rows, ``mask2`` (rows x cols, Ws orientation) marks the
    entries kept by the second prune, and ``Wdp = Ws * mask2``.
    """
    Ws, mask1 = decompress(vals, meta, n, m, cols)
    rows = Ws.shape[0]
    _check(rows, n, m)
    WT = Ws.T                      # cols x rows; groups of m along rows of Ws
    eligT = mask1.T
    G = rows // m
    magg = np.abs(WT).reshape(cols, G, m)
    eg = eligT.reshape(cols, G, m)
    keptT = eg & (group_ranks(magg, eg) < n)
    # padding: lowest unused in-group indices until n are stored
    need = n - keptT.sum(-1, keepdims=True)
    free_rank = np.cumsum(~keptT, axis=-1) - 1      # 0-based order among unused positions
    padT = (~keptT) & (free_rank < need)
    storedT = keptT | padT
    P_vals, P_meta = encode(WT.reshape(cols, rows), storedT.reshape(cols, rows), n, m,
                            pad_zero=padT.reshape(cols, rows))
    mask2 = keptT.reshape(cols, rows).T.copy()
    Wdp = np.where(mask2, Ws, 0.0)
    return P_vals, P_meta, mask2, Wdp
