"""GPU parity of one sender state feeding several receivers
(mf_retrieve_fused_multi).

Each case compresses one sender layer of a workload recipe and feeds the BSR
state to 2-4 receivers with their own head maps W_i ~ N(0, 1/H_s) and values
V_i ~ N(0, 1) (seeded, H_r / H_kv per receiver).  Bars:
  * bit for bit against mf_retrieve_fused run for each receiver alone (the
    joint launch runs the same kernels on the same data);
  * against the oracle's retrieve on the oracle's own BSR state, for every
    receiver, at the output bars of tests/_compare.py, on the rows whose kept
    sets equal the oracle's.
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


# name, recipe, overrides, [(H_r, H_kv)], expected joint launch
CASES = [
    ("bf16-3recv", "pair14b8b-bf16", dict(N=1000), [(32, 8), (16, 8), (24, 8)], True),
    ("f16-B128-2recv", "long32k-f16", dict(N=700), [(32, 8), (8, 8)], True),
    ("bf16-4recv-B16", "pair14b8b-bf16", dict(N=300, B=16), [(8, 8), (16, 4), (32, 8), (24, 8)], True),
    ("f32-plain-2recv", "tiny-f32", dict(), [(4, 4), (8, 2)], False),
    ("bf16-mixed-fallback", "pair14b8b-bf16", dict(N=500), [(32, 8), (40, 8)], False),
]


@pytest.mark.parametrize("name,recipe,over,recv,joint", CASES, ids=[c[0] for c in CASES])
def test_multi_receiver(name, recipe, over, recv, joint):
    say(f"[multi] {name} receivers={recv}")
    dev = torch.device("cuda:0")
    w = synth.workload(recipe, **over)
    L = synth.gen_layer(w, device=dev, seed=7100)
    A = L["A"]
    _, rp, ci, vals, nnzb = mf.compress(A, w.B, w.p)
    rcv = []
    for i, (H_r, H_kv) in enumerate(recv):
        wi = w.with_(H_r=H_r, H_kv=H_kv)
        rcv.append((synth.gen_W(wi, 7200 + i).to(dev), synth.gen_V(wi, 7200 + i).to(dev)))
    outs = mf.retrieve_fused_multi(rp, ci, vals, nnzb, rcv, w.N, w.B)
    singles = [mf.retrieve_fused(rp, ci, vals, nnzb, W, V, w.N, w.B) for W, V in rcv]
    torch.cuda.synchronize()
    for i, (o, s1) in enumerate(zip(outs, singles)):
        assert torch.equal(o, s1), f"receiver {i} differs from its single retrieval"
    # oracle on its own BSR state
    A_h = host(A).astype(np.float64)
    m_ref, kept, o_rp, o_ci, o_vals = oracle.compress(A_h, w.B, w.p)
    rp_g, ci_g = host(rp), host(ci)
    rows, ties = [], 0
    for I in range(w.T):
        if selection_ok(oracle.decision_masses(m_ref)[I, : I + 1], kept[I],
                        ci_g[rp_g[I]:rp_g[I + 1]], w.p) != "exact":
            ties += 1
            continue
        rows.extend(range(I * w.B, min(w.N, (I + 1) * w.B)))
    assert ties <= 2, ties
    for i, (W, V) in enumerate(rcv):
        O_ref = oracle.retrieve(o_rp, o_ci, o_vals, host(W).astype(np.float64),
                                host(V).astype(np.float64), w.N, w.B)
        check_output(host(outs[i]).astype(np.float64)[rows], O_ref[rows], w.dtype,
                     f"O receiver {i} ({name})")


def test_multi_single_receiver_equals_single_call():
    dev = torch.device("cuda:0")
    w = synth.workload("pair14b8b-bf16", N=640)
    L = synth.gen_layer(w, device=dev, seed=7300)
    _, rp, ci, vals, nnzb = mf.compress(L["A"], w.B, w.p)
    W, V = L["W"].to(dev), L["V"].to(dev)
    (o,) = mf.retrieve_fused_multi(rp, ci, vals, nnzb, [(W, V)], w.N, w.B)
    s1 = mf.retrieve_fused(rp, ci, vals, nnzb, W, V, w.N, w.B)
    torch.cuda.synchronize()
    assert torch.equal(o, s1)
