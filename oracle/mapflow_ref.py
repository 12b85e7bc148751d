"""fp64 reference of MapFlow's compression and fused retrieval (test infrastructure).

Notation: N tokens, block size B, T = ceil(N / B) block rows and columns,
H_s sender heads, H_r receiver heads, H_kv receiver KV heads with
G = H_r / H_kv receiver heads per KV head, d head dimension.

  A[h][i][j]        causal sender attention map of one sender layer
  mass[I][J]        head-averaged block mass (J <= I; zero above the diagonal)
  row_ptr[T+1], col_idx[nnzb], vals[nnzb][H_s][B][B]   Block Sparse Row state
  W[H_r][H_s]       learned head map of one reuse receiver layer
  V[N][H_kv][d]     receiver values;  O[N][H_r][d] attention output

Each step has a per-block-row function (``*_row``) and a whole-map wrapper
that loops over the rows.  ``A`` only needs ``.shape`` and basic slicing that
returns something ``np.asarray`` accepts, so a test can hand in a lazy view of
a map that lives elsewhere and check sampled block rows.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def n_blocks(N: int, B: int) -> int:
    return -(-N // B)


def _span(X: int, B: int, N: int) -> tuple[int, int]:
    return X * B, min(N, (X + 1) * B)


# ---------------------------------------------------------------------------
# 1. block statistics
# ---------------------------------------------------------------------------

def block_mass_row(A, B: int, I: int) -> np.ndarray:
    """mass[I][0..I] of one block row, fp64.

    MapFlow's compressor first computes a statistic per block and then chooses
    blocks (article aitest123.com/news/zaoi86, third section, first component);
    the selection threshold is a cumulative attention probability (paper page,
    highlight 3).  The statistic is therefore the attention probability that
    falls in the block: the plain sum of A over the block's rows and columns,
    averaged over the sender heads with equal weight, because one cached sender
    state serves receivers with different head maps (article, third section,
    second component).  Rows and columns at or beyond N do not exist (partial
    last block).  Only causal blocks J <= I are candidates.
    """
    H, N, _ = A.shape
    r0, r1 = _span(I, B, N)
    slab = np.asarray(A[:, r0:r1, : min(N, (I + 1) * B)], dtype=F64)
    out = np.zeros(I + 1, dtype=F64)
    for J in range(I + 1):
        c0, c1 = _span(J, B, N)
        out[J] = slab[:, :, c0:c1].sum() / H
    return out


def block_mass(A, B: int) -> np.ndarray:
    """mass[T][T] fp64 for the whole map (zeros above the diagonal)."""
    H, N, N2 = A.shape
    assert N == N2
    T = n_blocks(N, B)
    mass = np.zeros((T, T), dtype=F64)
    for I in range(T):
        mass[I, : I + 1] = block_mass_row(A, B, I)
    return mass


# ---------------------------------------------------------------------------
# 2. block-level Top-p
# ---------------------------------------------------------------------------

def topp_row(m, p: float) -> np.ndarray:
    """Kept columns (ascending) of one block row with candidate masses m[0..I].

    Block-level Top-p (paper page, highlight 3): candidates are visited in
    order of decreasing mass (equal masses: lower column first); blocks are
    kept until the kept mass first reaches p times the row's total mass
    (inclusive: the block that reaches it is kept).  p >= 1 keeps every causal
    block.  Nothing is renormalised; dropped mass is lost.  Sums run in fp64:
    the total in column order, the running sum in visiting order.
    """
    m = [float(x) for x in np.asarray(m, dtype=F64)]
    n = len(m)
    p = float(np.float32(p))          # the boundary passes p as fp32
    if p >= 1.0:
        return np.arange(n, dtype=np.int64)
    total = 0.0
    for x in m:
        total += x
    threshold = p * total
    order = sorted(range(n), key=lambda J: (-m[J], J))
    cum = 0.0
    chosen = []
    for J in order:
        chosen.append(J)
        cum += m[J]
        if cum >= threshold:
            break
    return np.array(sorted(chosen), dtype=np.int64)


def decision_masses(mass) -> np.ndarray:
    """Masses as the selection sees them.  The library stores block masses as
    fp32 and takes the Top-p decision on those values, so the decision is
    taken here on the fp64 masses rounded once to fp32 (then widened back)."""
    return np.asarray(mass, dtype=F64).astype(np.float32).astype(F64)


def topp_select(mass, p: float) -> list:
    """Per-row kept columns for a [T][T] mass matrix (decision on fp32 masses)."""
    m32 = decision_masses(mass)
    return [topp_row(m32[I, : I + 1], p) for I in range(m32.shape[0])]


# ---------------------------------------------------------------------------
# 3. Block Sparse Row state
# ---------------------------------------------------------------------------

def bsr_tile(A, B: int, I: int, J: int) -> np.ndarray:
    """vals entry of block (I, J): the [H_s][B][B] tile copied exactly in the
    input dtype, zeros for rows or columns at or beyond N (paper page,
    "Practical Implementation Details": BSR with regular 2-D blocks)."""
    H, N, _ = A.shape
    r0, r1 = _span(I, B, N)
    c0, c1 = _span(J, B, N)
    src = np.asarray(A[:, r0:r1, c0:c1])
    tile = np.zeros((H, B, B), dtype=src.dtype)
    tile[:, : r1 - r0, : c1 - c0] = src
    return tile


def build_bsr(A, B: int, kept: list):
    """row_ptr[T+1], col_idx[nnzb], vals[nnzb][H_s][B][B] of the kept blocks.
    All H_s heads share one pattern; col_idx is ascending within a row."""
    H, N, _ = A.shape
    T = n_blocks(N, B)
    assert len(kept) == T
    counts = np.array([len(k) for k in kept], dtype=np.int64)
    row_ptr = np.zeros(T + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    nnzb = int(row_ptr[-1])
    col_idx = (np.concatenate([np.asarray(k, dtype=np.int64) for k in kept])
               if nnzb else np.zeros(0, dtype=np.int64))
    dtype = np.asarray(A[:1, :1, :1]).dtype
    vals = np.zeros((nnzb, H, B, B), dtype=dtype)
    k = 0
    for I in range(T):
        for J in kept[I]:
            vals[k] = bsr_tile(A, B, I, int(J))
            k += 1
    return row_ptr, col_idx, vals


# ---------------------------------------------------------------------------
# 4. fused head-mapped retrieval
# ---------------------------------------------------------------------------

def retrieve_row(I: int, cols, tiles, W, V, N: int, B: int) -> np.ndarray:
    """O rows of block row I, [rows][H_r][d] fp64, from its kept blocks.

    For a reuse receiver layer, receiver head r's map is a linear combination
    of the sender heads with the learned weights W[r][:] (paper page, "MapFlow
    System Design" item 3 and highlight 2; article, second section: a learned
    linear combination of heads).  The kernel the pages describe reads only the
    kept blocks, mixes heads on chip and multiplies by the receiver's own
    values, accumulating the output (article, third section, third component;
    paper page, highlight 4).  Per kept block (I, J) and receiver head r:

        Ahat[r] = sum_s W[r][s] * tile[s]                      (B x B)
        O[I*B + i][r][:] += sum_c Ahat[r][i][c] * V[J*B + c][g(r)][:]

    with g(r) = r // (H_r / H_kv): consecutive receiver heads share a KV head.
    Rows and columns at or beyond N are skipped.  No bias, no renormalisation.
    """
    W64 = np.asarray(W, dtype=F64)
    H_r, H_s = W64.shape
    V = np.asarray(V)
    H_kv, d = V.shape[1], V.shape[2]
    assert H_r % H_kv == 0
    G = H_r // H_kv
    r0, r1 = _span(I, B, N)
    O = np.zeros((r1 - r0, H_r, d), dtype=F64)
    for J, tile in zip(cols, tiles):
        c0, c1 = _span(int(J), B, N)
        blk = np.asarray(tile, dtype=F64)                  # [H_s][B][B]
        Vblk = np.asarray(V[c0:c1], dtype=F64)             # [cols][H_kv][d]
        for r in range(H_r):
            ahat = np.zeros((B, B), dtype=F64)
            for s in range(H_s):
                ahat += W64[r, s] * blk[s]
            O[:, r, :] += ahat[: r1 - r0, : c1 - c0] @ Vblk[:, r // G, :]
    return O


def retrieve(row_ptr, col_idx, vals, W, V, N: int, B: int) -> np.ndarray:
    """O[N][H_r][d] fp64 for a whole BSR state (loops retrieve_row)."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    T = len(row_ptr) - 1
    assert T == n_blocks(N, B)
    H_r = np.asarray(W).shape[0]
    d = np.asarray(V).shape[2]
    O = np.zeros((N, H_r, d), dtype=F64)
    for I in range(T):
        k0, k1 = int(row_ptr[I]), int(row_ptr[I + 1])
        r0, r1 = _span(I, B, N)
        O[r0:r1] = retrieve_row(I, col_idx[k0:k1], vals[k0:k1], W, V, N, B)
    return O


def compress(A, B: int, p: float):
    """Sender-side compression: block mass -> Top-p -> BSR.
    Returns (mass, kept, row_ptr, col_idx, vals)."""
    mass = block_mass(A, B)
    kept = topp_select(mass, p)
    row_ptr, col_idx, vals = build_bsr(A, B, kept)
    return mass, kept, row_ptr, col_idx, vals


def pipeline_row(A, V, W, B: int, p: float, I: int):
    """Everything for one block row: (mass row, kept columns, tiles, O rows).

    The chain of the steps above restricted to block row I: the row's block
    masses, the Top-p decision on them as fp32 values, the kept tiles and the
    retrieved output rows.  It equals row I of compress() followed by
    retrieve()."""
    N = A.shape[1]
    m = block_mass_row(A, B, I)
    kept = topp_row(decision_masses(m), p)
    tiles = [bsr_tile(A, B, I, int(J)) for J in kept]
    O = retrieve_row(I, kept, tiles, W, V, N, B)
    return m, kept, tiles, O


# ---------------------------------------------------------------------------
# 5. compression from the sender's Q and K (no dense map)
# ---------------------------------------------------------------------------
#
# The article's compressor never lays out the full dense attention matrix: it
# computes the block statistics and then picks blocks (aitest123.com/news/
# zaoi86, third section, first component).  The sender's map is the causal
# softmax of its scores, so with Q = [H_s][N][d], K = [H_ks][N][d] (sender head
# h reads K head h / (H_s / H_ks)), a per-head score scale and the per-row
# log-sum-exp of the scores, every entry is
#     A[h][i][j] = exp(scale[h] * q_h,i . k_h,j - lse[h][i]),   j <= i,
# and both the block masses and the kept tiles follow from Q, K and lse alone.
# The per-row log-sum-exp is the statistic an attention forward keeps anyway.

def _qk(Q, K):
    Q = np.asarray(Q, dtype=F64)
    K = np.asarray(K, dtype=F64)
    H_s, N, d = Q.shape
    H_ks = K.shape[0]
    assert K.shape[1:] == (N, d) and H_s % H_ks == 0
    return Q, K, H_s // H_ks


def row_lse(Q, K, scale, rows=None) -> np.ndarray:
    """lse[h][i] = log sum_{j <= i} exp(scale[h] * q_h,i . k_h,j), fp64, for the
    rows ``rows`` (default: all N).  The maximum is subtracted before the
    exponentials (exact in real arithmetic)."""
    Q, K, G = _qk(Q, K)
    sc = np.asarray(scale, dtype=F64)
    H_s, N, _ = Q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((H_s, len(rows)), dtype=F64)
    keys = np.arange(N)
    for h in range(H_s):
        s = sc[h] * (Q[h, rows] @ K[h // G].T)
        s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
        m = s.max(axis=1)
        out[h] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


class QKMap:
    """The sender's causal map A[H_s][N][N] as a lazy view computed from Q, K,
    the score scale and the row log-sum-exp; indexing with three slices
    (heads, rows, columns) returns an fp64 array, zero above the diagonal.
    The step functions above (block mass, tiles) accept it in place of A."""

    def __init__(self, Q, K, scale, lse):
        self.Q, self.K, self.G = _qk(Q, K)
        self.scale = np.asarray(scale, dtype=F64)
        self.lse = np.asarray(lse, dtype=F64)
        H_s, N, _ = self.Q.shape
        assert self.lse.shape == (H_s, N) and self.scale.shape == (H_s,)
        self.shape = (H_s, N, N)
        self.dtype = np.dtype(F64)

    def __getitem__(self, idx):
        hs, rs, cs = idx
        H_s, N, _ = self.shape
        heads = np.arange(H_s)[hs]
        rows = np.arange(N)[rs]
        cols = np.arange(N)[cs]
        out = np.empty((len(heads), len(rows), len(cols)), dtype=F64)
        for a, h in enumerate(heads):
            s = self.scale[h] * (self.Q[h, rows] @ self.K[h // self.G, cols].T)
            p = np.exp(s - self.lse[h, rows][:, None])
            out[a] = np.where(cols[None, :] <= rows[:, None], p, 0.0)
        return out


def compress_qk(Q, K, scale, B: int, p: float, lse=None):
    """Compression without a dense map: (lse, mass, kept, row_ptr, col_idx,
    vals) from Q, K and the scale; ``lse`` defaults to the exact row_lse."""
    lse = row_lse(Q, K, scale) if lse is None else np.asarray(lse, dtype=F64)
    A = QKMap(Q, K, scale, lse)
    mass, kept, row_ptr, col_idx, vals = compress(A, B, p)
    return lse, mass, kept, row_ptr, col_idx, vals


# ---------------------------------------------------------------------------
# 6. retrieval over a packed batch of sequences
# ---------------------------------------------------------------------------

# The pages' serving integration runs under chunked prefill and paged KV caches
# (paper page, "Practical Implementation Details").  A packed batch carries S
# sequences back to back: sequence s holds tokens cu_seqlens[s] ..
# cu_seqlens[s+1]-1 of V and O and block rows cu_rows[s] .. cu_rows[s+1]-1 of a
# row_ptr that numbers the rows of all sequences in turn; col_idx is local to
# each sequence; kept block k's tiles sit in page block_table[k] of a pool
# (page k without a table).  Each sequence is retrieved on its own: nothing
# crosses a sequence boundary.

def retrieve_varlen(cu_seqlens, cu_rows, row_ptr, col_idx, pool, W, V, B: int,
                    block_table=None) -> np.ndarray:
    """O[total][H_r][d] fp64: retrieve() for every sequence of a packed batch."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cr = np.asarray(cu_rows, dtype=np.int64)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    V = np.asarray(V)
    H_r = np.asarray(W).shape[0]
    O = np.zeros((V.shape[0], H_r, V.shape[2]), dtype=F64)
    for s in range(len(cu) - 1):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        g0, g1 = int(cr[s]), int(cr[s + 1])
        N = t1 - t0
        if N == 0:
            continue
        assert g1 - g0 == n_blocks(N, B)
        k0, k1 = int(row_ptr[g0]), int(row_ptr[g1])
        ks = np.arange(k0, k1)
        pages = ks if block_table is None else np.asarray(block_table, dtype=np.int64)[ks]
        O[t0:t1] = retrieve(row_ptr[g0:g1 + 1] - k0, col_idx[k0:k1], np.asarray(pool)[pages],
                            W, V[t0:t1], N, B)
    return O
