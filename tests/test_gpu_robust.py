"""GPU: what the retrieval kernels must ignore.

A BSR state may carry tile positions that are not part of the map: the
padding of a partial last block (key columns and query rows at or beyond N)
and, in a hand-built state, blocks whose column lies outside [0, T).  The
boundary promises that these contribute nothing to O, whatever they hold.
Each case fills them with NaN and huge values and compares the output with
the oracle's on the clean state; both retrieval kernels are exercised.
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


def host(t):
    t = t.detach()
    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()


def poisoned(rp, ci, vals, N, B, T, rng):
    """The same state with NaN in every padding position and, in a third of
    the rows, two extra blocks (columns -1 and T + 3) full of huge values."""
    vals = vals.astype(np.float32).copy()
    rows_pad = N - (T - 1) * B                       # valid rows of the last block row
    for I in range(T):
        for k in range(rp[I], rp[I + 1]):
            if ci[k] == T - 1:
                vals[k][:, :, rows_pad:] = np.nan     # key columns >= N
            if I == T - 1:
                vals[k][:, rows_pad:, :] = np.nan     # query rows >= N
    new_rp, new_ci, new_vals = [0], [], []
    for I in range(T):
        blocks = [(int(ci[k]), vals[k]) for k in range(rp[I], rp[I + 1])]
        if I % 3 == 1:
            bad = np.full(vals.shape[1:], 3.0e38, dtype=np.float32)
            blocks = [(-1, bad)] + blocks + [(T + 3, np.full_like(bad, np.nan))]
        for J, t in blocks:
            new_ci.append(J)
            new_vals.append(t)
        new_rp.append(len(new_ci))
    return (np.array(new_rp, dtype=np.int32), np.array(new_ci, dtype=np.int32),
            np.stack(new_vals))


CASES = [
    ("pair14b8b-bf16", dict(N=1000), "mfma"),
    ("long32k-f16", dict(N=900), "mfma"),
    ("pair14b8b-bf16", dict(N=200, B=16, H_s=16, H_r=8, H_kv=2), "mfma"),
    ("pair14b8b-bf16", dict(N=300, H_s=64, H_r=16, H_kv=4), "plain"),
    ("tiny-f32", dict(N=250), "plain"),
]


@pytest.mark.parametrize("name,ov,kernel", CASES)
def test_padding_and_foreign_blocks_contribute_nothing(gpu, name, ov, kernel):
    w = synth.workload(name, **ov)
    say(f"[robust] {name} {ov}")
    assert w.N % w.B != 0
    L = synth.gen_layer(w)
    A_h, W_h, V_h = host(L["A"]), host(L["W"]), host(L["V"])
    _, _, rp, ci, vals = oracle.compress(A_h, w.B, w.p)
    O_ref = oracle.retrieve(rp, ci, vals, W_h, V_h, w.N, w.B)
    prp, pci, pvals = poisoned(rp, ci, vals, w.N, w.B, w.T, np.random.default_rng(0))
    tdt = synth.torch_dtype(w.dtype)
    d_vals = torch.from_numpy(pvals).to(gpu).to(tdt)
    assert torch.isnan(d_vals.float()).any()
    d_W, d_V = L["W"].to(gpu), L["V"].to(gpu)
    assert mf.retrieve_kernel(d_vals, d_V, d_W, w.N, w.B) == kernel
    O = mf.retrieve_fused(torch.from_numpy(prp).to(gpu), torch.from_numpy(pci).to(gpu), d_vals,
                          len(pci), d_W, d_V, w.N, w.B)
    torch.cuda.synchronize()
    rel = check_output(host(O), O_ref, w.dtype)
    say(f"[robust] nnzb={len(pci)} (with {len(pci) - len(ci)} foreign blocks) max err/max={rel:.3e}")
