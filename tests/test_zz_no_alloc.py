"""GPU: the allocation-free Top-p/BSR entry point against the one with a
workspace, through the C boundary.  Two calls in a row share the library's
fixed scratch; the second is smaller, so stale contents of the first must not
leak into it.  Bar: row_ptr, col_idx and vals bit for bit (integer and copy
work)."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import cross_model_sparse_amd as mf
import synth

pytestmark = pytest.mark.gpu


def _call_both(L, mass, A, B, p, cap):
    H_s, N = A.shape[0], A.shape[1]
    T = -(-N // B)
    dt = {torch.bfloat16: 2, torch.float16: 1, torch.float32: 0}[A.dtype]
    st = torch.cuda.current_stream().cuda_stream
    outs = []
    for noalloc in (False, True):
        rp = torch.full((T + 1,), -7, dtype=torch.int32, device=A.device)
        ci = torch.full((cap,), -7, dtype=torch.int32, device=A.device)
        vals = torch.full((cap, H_s, B, B), 3.0, dtype=A.dtype, device=A.device)
        if noalloc:
            r = L.mf_topp_select_bsr_noalloc(mass.data_ptr(), A.data_ptr(), dt, H_s, N, B,
                                             ctypes.c_float(p), rp.data_ptr(), ci.data_ptr(),
                                             vals.data_ptr(), cap, st)
        else:
            ws = torch.empty(L.mf_topp_workspace_bytes(N, B), dtype=torch.uint8, device=A.device)
            r = L.mf_topp_select_bsr(mass.data_ptr(), A.data_ptr(), dt, H_s, N, B, ctypes.c_float(p),
                                     rp.data_ptr(), ci.data_ptr(), vals.data_ptr(), cap, None,
                                     ws.data_ptr(), ws.numel(), st)
        assert r == 0, (noalloc, r, L.mf_last_error())
        torch.cuda.synchronize()
        outs.append((rp.cpu(), ci.cpu(), vals.cpu()))
    return outs


@pytest.mark.parametrize("name,ov", [("pair14b8b-bf16", dict(N=1000)), ("long32k-f16", dict(N=700))])
def test_noalloc_equals_workspace_call_twice(gpu, name, ov):
    L = mf.load()
    w = synth.workload(name, **ov)
    small = w.with_(N=w.N // 3 + 5)
    for ww in (w, small):                       # two calls in a row, the second smaller
        print(f"[noalloc] {ww.name} N={ww.N} B={ww.B}", flush=True)
        sys.stdout.flush()
        A = synth.gen_layer(ww, device=gpu)["A"]
        mass = mf.block_mass(A, ww.B)
        T = ww.T
        cap = T * (T + 1) // 2
        (rp0, ci0, v0), (rp1, ci1, v1) = _call_both(L, mass, A, ww.B, ww.p, cap)
        nnzb = int(rp0[T])
        assert 0 < nnzb <= cap
        assert torch.equal(rp0, rp1)
        assert torch.equal(ci0[:nnzb], ci1[:nnzb])
        assert torch.equal(v0[:nnzb].view(torch.int16), v1[:nnzb].view(torch.int16))
        # capacity overflow: the fixed-scratch call leaves col_idx/vals untouched as well
        (rp2, ci2, v2), (rp3, ci3, v3) = _call_both(L, mass, A, ww.B, ww.p, nnzb - 1)
        assert torch.equal(rp2, rp3) and int(rp3[T]) == nnzb
        assert (ci3 == -7).all() and (v3 == 3.0).all()
