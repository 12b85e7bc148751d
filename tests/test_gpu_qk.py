"""GPU parity of the compression from Q and K (no dense map) against the fp64 oracle.

Inputs: seeded Q, K in the storage dtype and a per-head score scale; the oracle
upcasts the same host values exactly.  Bars (derived from the arithmetic, see
the design notes):
  lse     |gpu - ref| <= N * 2^-24 + 1e-5        (fp32 online sum of <= N terms)
  mass    relative (16 B) * 2^-24 + 1e-5          (fp32 partial of <= 16 B positive terms)
  tiles   |gpu - ref| <= (half ulp of dtype + 1e-5) |ref| + 2^-25 (fp16 subnormals)
          or 2^-126 (values below it may be stored as 0)
  O       the retrieval bars of tests/_compare.py
The mass and tile checks feed the oracle's lse (rounded to fp32) to both sides,
so each step is checked on its own; the end-to-end check runs the product
path (lse from the library) against the oracle with its own fp64 lse.
"""
from __future__ import annotations

import math
import zlib
import sys

import numpy as np
import pytest
import torch

import cross_model_sparse_amd as mf
import oracle
from tests._compare import check_bsr_structure, check_output, selection_ok

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
HALF_ULP = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def make_inputs(seed, H_s, H_ks, N, d, dt, temp=True):
    g = torch.Generator().manual_seed(seed)
    Q = torch.randn(H_s, N, d, generator=g, dtype=torch.float64).to(TD[dt])
    K = torch.randn(H_ks, N, d, generator=g, dtype=torch.float64).to(TD[dt])
    tau = (torch.rand(H_s, generator=g, dtype=torch.float64) * 1.5 + 0.5) if temp else torch.ones(H_s, dtype=torch.float64)
    scale = (1.0 / (math.sqrt(d) * tau)).to(torch.float32)
    return Q, K, scale


# name, (H_s, H_ks, N, d, B, dtype, p[, scale multiplier])
CASES = [
    ("tiny-f32-plain", (4, 4, 200, 64, 16, "f32", 0.9)),
    ("f16-B64-gqa-ragged", (8, 2, 1000, 128, 64, "f16", 0.95)),
    ("bf16-B32-d64", (6, 3, 777, 64, 32, "bf16", 0.9)),
    ("bf16-B128-mqa", (4, 1, 600, 128, 128, "bf16", 0.8)),
    ("f16-B16-plain-mass", (4, 2, 300, 64, 16, "f16", 0.9)),
    ("bf16-short", (2, 1, 40, 128, 32, "bf16", 1.0)),
    # degenerate cases: one token, fewer tokens than a score tile, a negative
    # score scale (the log-sum-exp takes its maximum from the smallest
    # product), a zero scale (every row uniform over its causal keys)
    ("bf16-one-token", (2, 1, 1, 128, 32, "bf16", 0.9)),
    ("f16-under-a-tile", (3, 3, 29, 128, 64, "f16", 0.7)),
    ("f16-negative-scale", (4, 2, 500, 128, 64, "f16", 0.9, -1.0)),
    ("bf16-zero-scale", (4, 4, 300, 64, 32, "bf16", 0.5, 0.0)),
]


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_qk_compression_parity(name, cfg):
    H_s, H_ks, N, d, B, dt, p = cfg[:7]
    smul = cfg[7] if len(cfg) > 7 else 1.0
    say(f"[qk] {name} H_s={H_s} H_ks={H_ks} N={N} d={d} B={B} {dt} p={p} scale x {smul}")
    Q, K, scale = make_inputs(zlib.crc32(name.encode()) % 10000, H_s, H_ks, N, d, dt)
    scale = scale * smul
    Qh, Kh, sch = host(Q), host(K), scale.double().numpy()
    dev = torch.device("cuda:0")
    Qd, Kd, scd = Q.to(dev), K.to(dev), scale.to(dev)
    T = -(-N // B)

    # 1. row log-sum-exp
    lse_gpu = host(mf.row_lse(Qd, Kd, scd))
    lse_ref = oracle.row_lse(Qh, Kh, sch)
    err = np.abs(lse_gpu - lse_ref).max()
    assert err <= N * 2.0 ** -24 + 1e-5, f"lse err {err:.3e}"

    # 2. block mass from the oracle's lse (rounded to fp32 on both sides)
    lse32 = lse_ref.astype(np.float32)
    lse_in = torch.from_numpy(lse32).to(dev)
    A_ref = oracle.QKMap(Qh, Kh, sch, lse32.astype(np.float64))
    mass_ref = oracle.block_mass(A_ref, B)
    mass_gpu = host(mf.block_mass_qk(Qd, Kd, scd, lse_in, B))
    tol = 16 * B * 2.0 ** -24 + 1e-5
    rel = np.abs(mass_gpu - mass_ref) / np.maximum(np.abs(mass_ref), 1e-30)
    assert np.all(np.triu(mass_gpu, 1) == 0)
    assert rel[np.tril_indices(T)].max() <= tol, f"mass max rel err {rel[np.tril_indices(T)].max():.3e}"

    # 3. selection and recomputed tiles
    rp, ci, vals, nnzb = mf.topp_select_bsr_qk(torch.from_numpy(mass_ref.astype(np.float32)).to(dev),
                                               Qd, Kd, scd, lse_in, B, p)
    torch.cuda.synchronize()
    rp_h, ci_h = rp.cpu().numpy(), ci.cpu().numpy()
    check_bsr_structure(rp_h, ci_h[:nnzb], T)
    kept_ref = oracle.topp_select(mass_ref, p)
    vals_h = host(vals[:max(nnzb, 1)])
    ties = 0
    for I in range(T):
        kept_gpu = ci_h[rp_h[I]:rp_h[I + 1]]
        if selection_ok(oracle.decision_masses(mass_ref)[I, : I + 1], kept_ref[I], kept_gpu, p) != "exact":
            ties += 1
            continue
        for t, J in enumerate(kept_ref[I]):
            ref = oracle.bsr_tile(A_ref, B, I, int(J))
            got = vals_h[rp_h[I] + t]
            # + fp16 subnormal spacing; values below 2^-126 may be stored as 0
            bound = (HALF_ULP[dt] + 1e-5) * np.abs(ref) + (2.0 ** -25 if dt == "f16" else 2.0 ** -126)
            bad = np.abs(got - ref) > bound
            assert not bad.any(), f"row {I} block {J}: {int(bad.sum())} tile entries out of bound"
    assert ties <= max(1, T // 10), f"{ties} tied rows"

    # 4. end to end: product path (library lse) -> retrieval, against the oracle
    H_r, H_kv = 2 * H_s if H_s <= 16 else H_s, 2
    gW = torch.Generator().manual_seed(7)
    W = (torch.randn(H_r, H_s, generator=gW, dtype=torch.float64) / math.sqrt(H_s)).to(torch.float32)
    V = torch.randn(N, H_kv, d, generator=gW, dtype=torch.float64).to(TD[dt])
    lse_g, mass_g, rp_g, ci_g, vals_g, nnzb_g = mf.compress_qk(Qd, Kd, scd, B, p)
    O = mf.retrieve_fused(rp_g, ci_g, vals_g, nnzb_g, W.to(dev), V.to(dev), N, B)
    torch.cuda.synchronize()
    _, m_o, kept_o, rp_o, ci_o, vals_o = oracle.compress_qk(Qh, Kh, sch, B, p)
    O_ref = oracle.retrieve(rp_o, ci_o, vals_o, W.double().numpy(), host(V), N, B)
    rp_gh, ci_gh = rp_g.cpu().numpy(), ci_g.cpu().numpy()
    same = [I for I in range(T)
            if np.array_equal(np.sort(ci_gh[rp_gh[I]:rp_gh[I + 1]]), kept_o[I])]
    assert len(same) >= T - max(1, T // 10)
    rows = np.concatenate([np.arange(I * B, min(N, (I + 1) * B)) for I in same])
    check_output(host(O)[rows], O_ref[rows], dt, f"O ({name})")


def test_qk_full_size_sampled_rows():
    # the 8B->3B-like shape: N = 4096, B = 64, H_s = 32 (8 KV heads), d = 128, fp16
    H_s, H_ks, N, d, B, dt = 32, 8, 4096, 128, 64, "f16"
    say(f"[qk] full size H_s={H_s} N={N}")
    Q, K, scale = make_inputs(4242, H_s, H_ks, N, d, dt)
    Qh, Kh, sch = host(Q), host(K), scale.double().numpy()
    dev = torch.device("cuda:0")
    Qd, Kd, scd = Q.to(dev), K.to(dev), scale.to(dev)
    lse_gpu = mf.row_lse(Qd, Kd, scd)
    mass_gpu = host(mf.block_mass_qk(Qd, Kd, scd, lse_gpu, B))
    lse_gh = host(lse_gpu)
    T = N // B
    for I in (0, 1, T // 2, T - 1):
        rows = np.arange(I * B, (I + 1) * B)
        lse_ref = oracle.row_lse(Qh, Kh, sch, rows=rows)
        assert np.abs(lse_gh[:, rows] - lse_ref).max() <= N * 2.0 ** -24 + 1e-5
        # mass row I from the library's lse: the oracle view takes the same fp32 values
        lse_view = np.zeros((H_s, N))
        lse_view[:, rows] = lse_gh[:, rows]
        m_ref = oracle.block_mass_row(oracle.QKMap(Qh, Kh, sch, lse_view), B, I)
        rel = np.abs(mass_gpu[I, : I + 1] - m_ref) / np.maximum(m_ref, 1e-30)
        assert rel.max() <= 16 * B * 2.0 ** -24 + 1e-5, (I, rel.max())
        # each row of the map sums to one: the block row's masses sum to B
        assert abs(mass_gpu[I, : I + 1].sum() - B) <= 1e-3 * B


def test_qk_repeat_runs_are_bitwise_identical():
    Q, K, scale = make_inputs(99, 4, 2, 700, 128, "bf16")
    dev = torch.device("cuda:0")
    Qd, Kd, scd = Q.to(dev), K.to(dev), scale.to(dev)
    a = mf.compress_qk(Qd, Kd, scd, 64, 0.9)
    b = mf.compress_qk(Qd, Kd, scd, 64, 0.9)
    torch.cuda.synchronize()
    for x, y in zip(a[:5], b[:5]):
        assert torch.equal(x, y)
    assert a[5] == b[5]


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_lse_and_mass_in_one_pass(name, cfg):
    # mf_lse_block_mass_qk: lse against the oracle; masses against the oracle
    # on the map the library's lse defines (the oracle takes the same fp32
    # values) and against the two-pass mf_block_mass_qk; repeat runs identical
    H_s, H_ks, N, d, B, dt, p = cfg[:7]
    smul = cfg[7] if len(cfg) > 7 else 1.0
    say(f"[qk one pass] {name} H_s={H_s} H_ks={H_ks} N={N} d={d} B={B} {dt} scale x {smul}")
    Q, K, scale = make_inputs(zlib.crc32(name.encode()) % 10000, H_s, H_ks, N, d, dt)
    scale = scale * smul
    Qh, Kh, sch = host(Q), host(K), scale.double().numpy()
    dev = torch.device("cuda:0")
    Qd, Kd, scd = Q.to(dev), K.to(dev), scale.to(dev)
    T = -(-N // B)
    lse_g, mass_g = mf.lse_block_mass_qk(Qd, Kd, scd, B)
    lse_g2, mass_g2 = mf.lse_block_mass_qk(Qd, Kd, scd, B)
    mass_two = mf.block_mass_qk(Qd, Kd, scd, lse_g, B)
    torch.cuda.synchronize()
    assert torch.equal(lse_g, lse_g2) and torch.equal(mass_g, mass_g2)
    lse_h = host(lse_g)
    assert np.abs(lse_h - oracle.row_lse(Qh, Kh, sch)).max() <= N * 2.0 ** -24 + 1e-5
    m1, m2 = host(mass_g), host(mass_two)
    assert np.all(np.triu(m1, 1) == 0)
    mass_ref = oracle.block_mass(oracle.QKMap(Qh, Kh, sch, lse_h.astype(np.float64)), B)
    tri = np.tril_indices(T)
    tol = 16 * B * 2.0 ** -24 + 1e-5
    for m in (m1, m2):
        rel = np.abs(m[tri] - mass_ref[tri]) / np.maximum(np.abs(mass_ref[tri]), 1e-30)
        assert rel.max() <= tol, f"mass max rel err {rel.max():.3e}"


def test_lse_and_mass_in_one_pass_full_size():
    # the 8B->3B-like shape, sampled block rows against the oracle
    H_s, H_ks, N, d, B, dt = 32, 8, 4096, 128, 64, "f16"
    say(f"[qk one pass] full size H_s={H_s} N={N}")
    Q, K, scale = make_inputs(4242, H_s, H_ks, N, d, dt)
    Qh, Kh, sch = host(Q), host(K), scale.double().numpy()
    dev = torch.device("cuda:0")
    Qd, Kd, scd = Q.to(dev), K.to(dev), scale.to(dev)
    lse_g, mass_g = mf.lse_block_mass_qk(Qd, Kd, scd, B)
    mass_h, lse_h = host(mass_g), host(lse_g)
    T = N // B
    for I in (0, 1, T // 2, T - 1):
        rows = np.arange(I * B, (I + 1) * B)
        assert np.abs(lse_h[:, rows] - oracle.row_lse(Qh, Kh, sch, rows=rows)).max() <= N * 2.0 ** -24 + 1e-5
        lse_view = np.zeros((H_s, N))
        lse_view[:, rows] = lse_h[:, rows]
        m_ref = oracle.block_mass_row(oracle.QKMap(Qh, Kh, sch, lse_view), B, I)
        rel = np.abs(mass_h[I, : I + 1] - m_ref) / np.maximum(m_ref, 1e-30)
        assert rel.max() <= 16 * B * 2.0 ** -24 + 1e-5, (I, rel.max())
