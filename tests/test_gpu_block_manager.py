"""GPU side of the Block Manager: tile copies into the pool, and a cached
prefix reused end to end, also against the oracle's retrieval through the
same pool pages.

A causal map's rows below position n depend on tokens 0..n-1 only, so the map
of a sequence's first n tokens is exactly the top-left n x n corner of the
longer sequence's map.  The test compresses the prefix alone and caches its
block rows, then serves the whole sequence with those rows taken from the
cache (through the block table of the packed-batch retrieval) and the rest
compressed fresh.  Bars: the cached rows' kept columns and pool tiles equal the
fresh compression's bit for bit, and so does the retrieval output.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import cross_model_sparse_amd as mf
import oracle
import synth
from tests._compare import check_output

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_pool_store_copies_only_pages_inside_the_pool():
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(5)
    vals = torch.randn(6, 3, 16, 16, generator=g).to(torch.bfloat16).to(dev)
    pool = torch.zeros(5, 3, 16, 16, dtype=torch.bfloat16, device=dev)
    pages = torch.tensor([4, -1, 0, 7, 2, -5], dtype=torch.int32, device=dev)
    mf.pool_store(vals, pages, pool)
    torch.cuda.synchronize()
    want = torch.zeros_like(pool)
    for k, p in enumerate(pages.tolist()):
        if 0 <= p < 5:
            want[p] = vals[k]
    assert torch.equal(pool, want)


@pytest.mark.parametrize("recipe,N,n_pre", [("pair14b8b-bf16", 1000, 512), ("pair8b3b-f16", 900, 320)])
def test_cached_prefix_serves_the_longer_sequence(recipe, N, n_pre):
    say(f"[bm] {recipe} N={N} prefix={n_pre}")
    dev = torch.device("cuda:0")
    w = synth.workload(recipe, N=N)
    B, p = w.B, w.p
    L = synth.gen_layer(w, device=dev, seed=6100)
    A, W, V = L["A"], L["W"].to(dev), L["V"].to(dev)
    tokens = np.random.default_rng(1).integers(0, 50000, size=N).astype(np.int32)
    n_pages = 2 * w.T * (w.T + 1) // 2
    pool = torch.empty(n_pages, w.H_s, B, B, dtype=A.dtype, device=dev)
    bm = mf.BlockManager(B, 1, n_pages, seed=12345)

    # request 1: the prefix alone
    A_pre = A[:, :n_pre, :n_pre].contiguous()
    _, rp1, ci1, vals1, nz1 = mf.compress(A_pre, B, p)
    k_rows = n_pre // B
    pages1 = bm.insert(0, tokens[:n_pre], 0, rp1.cpu().numpy(), ci1[:nz1].cpu().numpy())
    mf.pool_store(vals1[:nz1], torch.from_numpy(pages1).to(dev), pool)

    # request 2: the whole sequence
    rp_c, ci_c, pg_c = bm.lookup(0, tokens)
    assert len(rp_c) - 1 == k_rows
    _, rp, ci, vals, nz = mf.compress(A, B, p)
    rp_h, ci_h = rp.cpu().numpy(), ci[:nz].cpu().numpy()
    k0 = int(rp_h[k_rows])
    assert np.array_equal(rp_c, rp_h[: k_rows + 1]) and np.array_equal(ci_c, ci_h[:k0])
    torch.cuda.synchronize()
    assert torch.equal(pool[torch.from_numpy(pg_c).long().to(dev)], vals[:k0])
    # new full rows go into the cache as well; the partial last row is served fresh
    full = N // B
    pages_new = bm.insert(0, tokens, k_rows, rp_h[k_rows: full + 1] - k0, ci_h[k0: int(rp_h[full])])
    mf.pool_store(vals[k0: int(rp_h[full])], torch.from_numpy(pages_new).to(dev), pool)
    tail0 = int(rp_h[full])
    tail = torch.arange(n_pages - (nz - tail0), n_pages, dtype=torch.int32, device=dev)
    mf.pool_store(vals[tail0:nz], tail, pool)
    table = torch.cat([torch.from_numpy(pg_c).to(dev), torch.from_numpy(pages_new).to(dev), tail])
    cu = torch.tensor([0, N], dtype=torch.int32, device=dev)
    cr = torch.tensor([0, w.T], dtype=torch.int32, device=dev)
    O_cache = mf.retrieve_fused_varlen(cu, cr, rp, ci, pool, nz, W, V, B, block_table=table)
    O_fresh = mf.retrieve_fused(rp, ci, vals, nz, W, V, N, B)
    torch.cuda.synchronize()
    assert torch.equal(O_cache, O_fresh)
    # the cached path against the oracle: its own compression of the host copy
    # of the map, its tiles placed in a host pool at the manager's pages, and
    # its packed-batch retrieval through the same block table
    A_h = A.float().cpu().numpy()
    _, _, rp_o, ci_o, vals_o = oracle.compress(A_h, B, p)
    assert np.array_equal(rp_o, rp_h) and np.array_equal(ci_o, ci_h), "selection differs from the oracle"
    tab = table.cpu().numpy().astype(np.int64)
    pool_o = np.zeros((n_pages,) + vals_o.shape[1:], dtype=vals_o.dtype)
    pool_o[tab] = vals_o
    O_ref = oracle.retrieve_varlen([0, N], [0, w.T], rp_o, ci_o, pool_o, L["W"].numpy(),
                                   L["V"].float().numpy(), B, block_table=tab)
    rel = check_output(O_cache.float().cpu().numpy(), O_ref, w.dtype)
    say(f"[bm] cached path vs oracle: max err/max = {rel:.3e}")
    s = bm.stats()
    assert s["hits"] == k_rows and s["held_rows"] == k_rows
    bm.release(0, tokens, k_rows)
    assert bm.stats()["held_rows"] == 0
    bm.close()
