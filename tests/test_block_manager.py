"""Block Manager (host side, no GPU): the library's manager against the plain
Python model in oracle/block_manager_ref.py, call for call.

Pins of the model itself: the published FNV-1a 64-bit test vectors, the
chained prefix hash written out byte by byte, and hand-worked scenarios (LRU
order, held rows, capacity errors, rows already cached).
"""
from __future__ import annotations

import numpy as np
import pytest

import cross_model_sparse_amd as mf
from oracle import block_manager_ref as ref


# ---- the hash ------------------------------------------------------------------

def test_fnv1a64_published_vectors():
    # test vectors of the FNV-1a 64-bit function (offset basis for the empty input)
    assert ref.fnv1a64(b"") == 0xCBF29CE484222325
    assert ref.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert ref.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_chain_is_fnv_over_parent_then_tokens():
    parent, chunk = 0x0123456789ABCDEF, [7, -1, 65536]
    data = bytes([0xEF, 0xCD, 0xAB, 0x89, 0x67, 0x45, 0x23, 0x01,
                  7, 0, 0, 0, 0xFF, 0xFF, 0xFF, 0xFF, 0, 0, 1, 0])
    assert ref.chain(parent, chunk) == ref.fnv1a64(data)


@pytest.mark.parametrize("B,n,seed", [(1, 5, 0), (4, 23, 99), (64, 300, 2**63 + 5)])
def test_library_prefix_hashes_match_the_model(B, n, seed):
    rng = np.random.default_rng(n)
    tok = rng.integers(-2**31, 2**31, size=n, dtype=np.int64).astype(np.int32)
    got = mf.prefix_hashes(tok, B, seed)
    assert [int(x) for x in got] == ref.prefix_hashes(tok.tolist(), B, seed)


def test_prefix_hashes_carry_the_preceding_context():
    a = np.arange(12, dtype=np.int32)
    b = a.copy()
    b[0] = 99                                    # only the first chunk differs
    ha, hb = mf.prefix_hashes(a, 4), mf.prefix_hashes(b, 4)
    assert all(x != y for x, y in zip(ha, hb))  # every later key changes too


# ---- scenarios -------------------------------------------------------------------

def _row_cols(rows):
    rp, cols = [0], []
    for r in rows:
        cols += r
        rp.append(len(cols))
    return rp, cols


def test_insert_lookup_release_and_lru_order():
    B = 2
    bm = mf.BlockManager(B, 1, 5)
    t1 = [1, 2, 3, 4]            # two rows
    t2 = [9, 9]                  # one row
    rp, cols = _row_cols([[0], [0, 1]])
    assert list(bm.insert(0, t1, 0, rp, cols)) == [0, 1, 2]
    rp2, cols2 = _row_cols([[0]])
    assert list(bm.insert(0, t2, 0, rp2, cols2)) == [3]
    r, c, p = bm.lookup(0, t1 + [5, 6])          # the third chunk is not cached
    assert list(r) == [0, 1, 3] and list(c) == [0, 0, 1] and list(p) == [0, 1, 2]
    s = bm.stats()
    assert (s["hits"], s["misses"], s["held_rows"], s["free_pages"]) == (2, 1, 2, 1)
    # 3 pages needed, 1 free: only t2's row is evictable -> capacity error, nothing changes
    rp3, cols3 = _row_cols([[0, 1, 2]])
    with pytest.raises(mf.CapacityError):
        bm.insert(0, [5, 5, 6, 6, 7, 7], 2, rp3, cols3)
    assert bm.stats()["cached_rows"] == 3
    bm.release(0, t1, 2)
    # now t1's rows (used more recently than t2's) are evicted after t2's row
    pages = bm.insert(0, [5, 5, 6, 6, 7, 7], 2, rp3, cols3)
    assert bm.stats()["evictions"] == 2 and sorted(pages) == [0, 3, 4]
    assert len(bm.lookup(0, t2)[0]) == 1        # t2's row is gone
    bm.close()


def test_held_rows_are_never_evicted_and_release_checks_holds():
    bm = mf.BlockManager(1, 2, 2)
    rp, cols = _row_cols([[0]])
    bm.insert(1, [4], 0, rp, cols)
    bm.lookup(1, [4])
    with pytest.raises(mf.CapacityError):
        bm.insert(1, [5, 6], 0, *_row_cols([[0], [0, 1]]))
    bm.release(1, [4], 1)
    with pytest.raises(mf.MapflowError):
        bm.release(1, [4], 1)                   # not held any more
    bm.close()


def test_rows_already_cached_get_no_pages_and_partial_chunks_are_not_cached():
    bm = mf.BlockManager(4, 1, 10)
    rp, cols = _row_cols([[0], [1]])
    p1 = bm.insert(0, list(range(10)), 0, rp, cols)        # 10 tokens: rows 0, 1 (8 full)
    assert list(p1) == [0, 1]
    p2 = bm.insert(0, list(range(8)), 0, rp, cols)
    assert list(p2) == [-1, -1]
    assert len(bm.lookup(0, list(range(11)))[0]) == 3      # 2 full rows, the rest not cached
    with pytest.raises(mf.MapflowError):                   # a row needs its whole chunk
        bm.insert(0, list(range(10)), 2, *_row_cols([[0]]))
    bm.close()


def test_rejects_bad_arguments():
    with pytest.raises(mf.MapflowError):
        mf.BlockManager(0, 1, 4)
    bm = mf.BlockManager(2, 1, 4)
    with pytest.raises(mf.MapflowError):
        bm.lookup(1, [1, 2])                               # layer out of range
    with pytest.raises(mf.MapflowError):
        bm.insert(0, [1, 2, 3, 4], 0, [0, 1, 2], [0, 2])   # column past its row
    with pytest.raises(mf.MapflowError):
        bm.insert(0, [1, 2, 3, 4], 0, [0, 2, 2], [1, 0])   # not ascending
    bm.close()


# ---- random operation sequences: library against the model ------------------------

def _random_ops(seed, n_ops=400):
    rng = np.random.default_rng(seed)
    B, layers, pages = int(rng.integers(1, 4)), 2, int(rng.integers(4, 30))
    base = [rng.integers(0, 3, size=12).tolist() for _ in range(3)]   # shared prefixes
    lib, mod = mf.BlockManager(B, layers, pages, seed), ref.BlockManagerRef(B, layers, pages, seed)
    held = []                                 # (layer, tokens, n_rows) returned by lookups
    for _ in range(n_ops):
        layer = int(rng.integers(0, layers))
        toks = list(base[int(rng.integers(0, 3))][: int(rng.integers(0, 13))])
        if rng.random() < 0.3 and toks:
            toks[int(rng.integers(0, len(toks)))] = int(rng.integers(0, 3))
        op = rng.random()
        if op < 0.4:
            n_full = len(toks) // B
            row0 = int(rng.integers(0, n_full + 1))
            n_rows = int(rng.integers(0, n_full - row0 + 1))
            rows = []
            for i in range(n_rows):
                cand = np.arange(row0 + i + 1)
                k = int(rng.integers(1, len(cand) + 1))
                rows.append(sorted(int(x) for x in rng.choice(cand, size=k, replace=False)))
            rp, cols = _row_cols(rows)
            st, out = mod.insert(layer, toks, row0, rp, cols)
            try:
                got, gst = list(lib.insert(layer, toks, row0, rp, cols)), ref.OK
            except mf.CapacityError:
                got, gst = None, ref.CAPACITY
            assert gst == st, ("insert", st, gst)
            if st == ref.OK:
                assert got == out
        elif op < 0.75:
            max_rows = int(rng.integers(0, 6))
            cap = int(rng.integers(0, 12))
            st, n, rp, cols, pg = mod.lookup(layer, toks, max_rows, cap)
            try:
                r, c, p = lib.lookup(layer, toks, max_rows=max_rows, cap=cap)
                gst = ref.OK
            except mf.CapacityError:
                gst = ref.CAPACITY
            assert gst == st, ("lookup", st, gst)
            if st == ref.OK:
                assert list(r) == rp and list(c) == cols and list(p) == pg
                if n:
                    held.append((layer, toks, n))
        elif held:
            layer, toks, n = held.pop(int(rng.integers(0, len(held))))
            assert mod.release(layer, toks, n) == ref.OK
            lib.release(layer, toks, n)
        assert lib.stats() == mod.stats()
    lib.close()


@pytest.mark.parametrize("seed", range(12))
def test_random_operations_match_the_model(seed):
    _random_ops(seed)
