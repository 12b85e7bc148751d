"""GPU parity of the packed-batch retrieval (mf_retrieve_fused_varlen).

Each case packs several sequences of one workload recipe (ragged lengths, one
shorter than a block, an empty one) with their tiles placed in a pool in a
random page order.  Bars:
  * bit for bit against mf_retrieve_fused run on each sequence alone (the
    batch runs the same kernels on the same data, so nothing may differ);
  * against the oracle's retrieve_varlen on the oracle's own BSR states (built
    from host copies of the maps), at the output bars of tests/_compare.py, on
    the rows whose kept sets equal the oracle's;
  * a page outside the pool contributes nothing: equal, bit for bit, to the
    sequence's retrieval with that block's column marked invalid.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import cross_model_sparse_amd as mf
import oracle
import synth
from tests._compare import check_output, selection_ok

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


# name, workload recipe, sequence lengths, p
CASES = [
    ("bf16-mfma-B64", "varlen-bf16", [700, 64, 1, 0, 1100, 333], 0.9),
    ("f32-plain-B16", "tiny-f32", [200, 17, 256, 1], 0.9),
    ("f16-mfma-B128", "long32k-f16", [300, 520], 0.9),
]


def build_batch(recipe, lens, p, dev, seed0):
    """Per sequence: maps, GPU compression and single-sequence retrieval."""
    seqs = []
    W = None
    for s, n in enumerate(lens):
        if n == 0:
            seqs.append(None)
            continue
        w = synth.workload(recipe, N=n)
        L = synth.gen_layer(w, device=dev, seed=seed0 + s)
        if W is None:
            W = L["W"].to(dev)
        A, V = L["A"], L["V"].to(dev)
        _, rp, ci, vals, nnzb = mf.compress(A, w.B, p)
        O = mf.retrieve_fused(rp, ci, vals, nnzb, W, V, n, w.B)
        seqs.append(dict(N=n, A=A, V=V, rp=rp, ci=ci, vals=vals[:nnzb], nnzb=nnzb, O=O))
    return seqs, W


def pack(seqs, lens, B, dev, rng):
    cu = np.cumsum([0] + lens)
    cr = np.cumsum([0] + [-(-n // B) for n in lens])
    rps, cis, tiles = [torch.zeros(1, dtype=torch.int32, device=dev)], [], []
    base = 0
    for sq in seqs:
        if sq is None:
            continue
        rps.append(sq["rp"][1:] + base)
        cis.append(sq["ci"][: sq["nnzb"]])
        tiles.append(sq["vals"])
        base += sq["nnzb"]
    row_ptr = torch.cat(rps).to(torch.int32)
    col_idx = torch.cat(cis).to(torch.int32)
    allv = torch.cat(tiles)
    perm = torch.from_numpy(rng.permutation(base)).to(dev)
    pool = torch.empty_like(allv)
    pool[perm] = allv
    V = torch.cat([sq["V"] for sq in seqs if sq is not None])
    as_i32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(dev)
    return dict(cu=as_i32(cu), cr=as_i32(cr), row_ptr=row_ptr, col_idx=col_idx, pool=pool,
                table=perm.to(torch.int32), nnzb=base, V=V, cu_h=cu, cr_h=cr)


@pytest.mark.parametrize("name,recipe,lens,p", CASES, ids=[c[0] for c in CASES])
def test_varlen_batch(name, recipe, lens, p):
    say(f"[varlen] {name} lens={lens} p={p}")
    dev = torch.device("cuda:0")
    B = synth.workload(recipe).B
    rng = np.random.default_rng(len(name))
    seqs, W = build_batch(recipe, lens, p, dev, 9000)
    b = pack(seqs, lens, B, dev, rng)
    O = mf.retrieve_fused_varlen(b["cu"], b["cr"], b["row_ptr"], b["col_idx"], b["pool"], b["nnzb"],
                                 W, b["V"], B, block_table=b["table"])
    torch.cuda.synchronize()
    # 1. bit for bit against each sequence alone
    for s, sq in enumerate(seqs):
        if sq is None:
            continue
        t0, t1 = int(b["cu_h"][s]), int(b["cu_h"][s + 1])
        assert torch.equal(O[t0:t1], sq["O"]), f"sequence {s} differs from its single retrieval"
    # 2. against the oracle on its own BSR states
    dt = synth.workload(recipe).dtype
    o_seqs, o_V = [], []
    for sq in seqs:
        if sq is None:
            continue
        A_h = host(sq["A"]).astype(np.float64)
        _, kept, rp, ci, vals = oracle.compress(A_h, B, p)
        o_seqs.append((sq, kept, rp, ci, vals))
        o_V.append(host(sq["V"]).astype(np.float64))
    o_cr = np.cumsum([0] + [len(t[2]) - 1 for t in o_seqs])
    o_cu = np.cumsum([0] + [t[0]["N"] for t in o_seqs])
    o_rp = np.concatenate([[0]] + [t[2][1:] + sum(len(u[3]) for u in o_seqs[:i])
                                   for i, t in enumerate(o_seqs)])
    o_ci = np.concatenate([t[3] for t in o_seqs])
    o_pool = np.concatenate([t[4] for t in o_seqs])
    O_ref = oracle.retrieve_varlen(o_cu, o_cr, o_rp, o_ci, o_pool, host(W).astype(np.float64),
                                   np.concatenate(o_V), B)
    O_h = host(O).astype(np.float64)
    rows, ties = [], 0
    for i, (sq, kept, *_rest) in enumerate(o_seqs):
        rp_g, ci_g = host(sq["rp"]), host(sq["ci"])
        m_ref = oracle.block_mass(host(sq["A"]).astype(np.float64), B)
        for I in range(len(kept)):
            how = selection_ok(oracle.decision_masses(m_ref)[I, : I + 1], kept[I],
                               ci_g[rp_g[I]:rp_g[I + 1]], p)
            if how != "exact":
                ties += 1
                continue
            rows.extend(range(o_cu[i] + I * B, min(o_cu[i + 1], o_cu[i] + (I + 1) * B)))
    assert ties <= 2, f"{ties} tied rows"
    check_output(O_h[rows], O_ref[rows], dt, f"O ({name})")
    # 3. a page outside the pool contributes nothing
    s0 = next(s for s, sq in enumerate(seqs) if sq is not None and sq["nnzb"] > 1)
    sq = seqs[s0]
    k_local = sq["nnzb"] // 2
    k_global = sum(seqs[s]["nnzb"] for s in range(s0) if seqs[s] is not None) + k_local
    table = b["table"].clone()
    table[k_global] = b["pool"].shape[0]
    O2 = mf.retrieve_fused_varlen(b["cu"], b["cr"], b["row_ptr"], b["col_idx"], b["pool"],
                                  b["nnzb"], W, b["V"], B, block_table=table)
    ci_bad = sq["ci"].clone()
    ci_bad[k_local] = -1
    O_s = mf.retrieve_fused(sq["rp"], ci_bad, sq["vals"], sq["nnzb"], W, sq["V"], sq["N"], B)
    torch.cuda.synchronize()
    t0, t1 = int(b["cu_h"][s0]), int(b["cu_h"][s0 + 1])
    assert torch.equal(O2[t0:t1], O_s)


def test_varlen_without_table_equals_with_identity_table():
    dev = torch.device("cuda:0")
    lens = [130, 64, 257]
    seqs, W = build_batch("varlen-bf16", lens, 0.8, dev, 9100)
    b = pack(seqs, lens, 64, dev, np.random.default_rng(1))
    ident = torch.empty_like(b["pool"])
    ident[torch.arange(b["nnzb"], device=dev)] = b["pool"][b["table"].long()]
    O1 = mf.retrieve_fused_varlen(b["cu"], b["cr"], b["row_ptr"], b["col_idx"], ident, b["nnzb"],
                                  W, b["V"], 64)
    O2 = mf.retrieve_fused_varlen(b["cu"], b["cr"], b["row_ptr"], b["col_idx"], b["pool"],
                                  b["nnzb"], W, b["V"], 64, block_table=b["table"])
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)
