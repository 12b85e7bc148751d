"""GPU: retrieval with long block rows split into parts (fp32 partials added
in part order by a second kernel), against the fp64 oracle.

Near-dense maps keep up to T blocks in a row, far more than one CU's share of
a launch, so the library splits such rows when it gets a workspace of
mf_retrieve_split_workspace_bytes.  Checked: every block row at full size
(8B->3B-like layer) end to end, ragged and bf16 and B = 128 cases on
oracle-built BSR states, a workspace full of NaN beforehand (its contents
need no initialisation), and repeat runs bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import cross_model_sparse_amd as mf
import oracle
import synth
from tests._compare import check_bsr_structure, check_output
from tests.test_gpu_parity import HostView, check_rows, host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def split_ws(w, nnzb, device):
    n = mf.retrieve_split_workspace_bytes(nnzb, synth.torch_dtype(w.dtype), w.H_s, w.N, w.B, w.H_r,
                                          w.H_kv, w.d)
    assert n > 0, "splitting should apply to this near-dense case"
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    ws.view(torch.float32)[:n // 4].fill_(float("nan"))
    return ws


CASES = [
    ("pair8b3b-f16", dict(N=1000)),                       # ragged, fp16, G = 3
    ("pair8b3b-f16", dict(N=2000, dtype="bf16")),         # bf16 hi/lo path
    ("pair8b3b-f16", dict(N=900, B=128, H_r=32, H_kv=8)),  # B = 128
    ("pair8b3b-f16", dict(N=777, B=32, H_r=16, H_kv=8)),   # B = 32, one receiver pair per wave
]


@pytest.mark.parametrize("name,ov", CASES)
def test_split_rows_on_oracle_bsr(gpu, name, ov):
    w = synth.workload(name, **ov)
    say(f"[split] {name} {ov}")
    L = synth.gen_layer(w)
    A_h, W_h, V_h = host(L["A"]), host(L["W"]), host(L["V"])
    _, kept, rp, ci, vals = oracle.compress(A_h, w.B, w.p)
    O_ref = oracle.retrieve(rp, ci, vals, W_h, V_h, w.N, w.B)
    tdt = synth.torch_dtype(w.dtype)
    d_vals = torch.from_numpy(vals).to(gpu).to(tdt)
    d_rp = torch.from_numpy(rp.astype(np.int32)).to(gpu)
    d_ci = torch.from_numpy(ci.astype(np.int32)).to(gpu)
    d_W, d_V = L["W"].to(gpu), L["V"].to(gpu)
    nnzb = len(ci)
    ws = split_ws(w, nnzb, gpu)
    O1 = mf.retrieve_fused(d_rp, d_ci, d_vals, nnzb, d_W, d_V, w.N, w.B, workspace=ws)
    O2 = mf.retrieve_fused(d_rp, d_ci, d_vals, nnzb, d_W, d_V, w.N, w.B, workspace=ws)
    O0 = mf.retrieve_fused(d_rp, d_ci, d_vals, nnzb, d_W, d_V, w.N, w.B)      # rows kept whole
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16)), "split runs differ"
    rel = check_output(host(O1), O_ref, w.dtype)
    rel0 = check_output(host(O0), O_ref, w.dtype)
    longest = int(np.diff(rp).max())
    say(f"[split] nnzb={nnzb} longest row {longest} blocks; max err/max split {rel:.3e} whole {rel0:.3e}")


def test_split_rows_full_size_every_row(gpu):
    """The 8B->3B-like layer at full size (N = 4096, near-dense, p = 0.95):
    compression on the GPU, retrieval with split rows, every block row
    checked against the oracle (masses, selection, tiles, outputs)."""
    w = synth.workload("pair8b3b-f16")
    say(f"[split] full {w.name} N={w.N}")
    L = synth.gen_layer(w, device=gpu)
    A, W, V = L["A"], L["W"].to(gpu), L["V"].to(gpu)
    mass = mf.block_mass(A, w.B)
    rp, ci, vals, nnzb = mf.topp_select_bsr(mass, A, w.B, w.p)
    ws = split_ws(w, nnzb, gpu)
    O = mf.retrieve_fused(rp, ci, vals, nnzb, W, V, w.N, w.B, workspace=ws)
    O_again = mf.retrieve_fused(rp, ci, vals, nnzb, W, V, w.N, w.B, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16), O_again.view(torch.int16))
    g_rp = host(rp).astype(np.int64)
    check_bsr_structure(g_rp, host(ci)[:nnzb], w.T)
    rows = list(range(w.T))
    g_vals = {k: host(vals[k]) for I in rows for k in range(g_rp[I], g_rp[I + 1])}
    ties, rel = check_rows(rows, HostView(A), host(L["W"]), host(L["V"]), w.B, w.p, w.dtype,
                           host(mass), g_rp, host(ci), g_vals, host(O))
    say(f"[split] nnzb={nnzb} rows={len(rows)} ties={ties} max err/max={rel:.3e}")
    assert ties <= 2
