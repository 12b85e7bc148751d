"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test ties an oracle step to an independent fact: a library routine
(torch SDPA, scipy.sparse BSR), brute force, a closed form, an invariant of
the Top-p rule, or a hand-worked example.  Together they catch a dropped term,
a wrong sign or index and a transposed operand anywhere in the oracle.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.sparse as sp
import torch

import oracle
import synth
from tests._compare import check_bsr_structure, selection_ok

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dense_from_bsr(row_ptr, col_idx, vals, N, B):
    """Scatter a BSR state to a dense [H_s][N][N] map (test-side brute force)."""
    H = vals.shape[1]
    T = len(row_ptr) - 1
    D = np.zeros((H, T * B, T * B))
    for I in range(T):
        for k in range(row_ptr[I], row_ptr[I + 1]):
            J = col_idx[k]
            D[:, I * B:(I + 1) * B, J * B:(J + 1) * B] = vals[k]
    return D[:, :N, :N]


def _dense_retrieval(A_dense, W, V):
    """O = (W (x) A) V over the full dense map, one receiver head at a time."""
    H_r = W.shape[0]
    H_kv = V.shape[1]
    G = H_r // H_kv
    N = A_dense.shape[1]
    O = np.zeros((N, H_r, V.shape[2]))
    for r in range(H_r):
        Ahat = np.tensordot(W[r], A_dense, axes=(0, 0))     # [N][N]
        O[:, r, :] = Ahat @ V[:, r // G, :]
    return O


def _random_causal_map(rng, H, N, dirichlet=False):
    A = rng.random((H, N, N)) ** 3
    A *= np.tril(np.ones((N, N)))[None]
    A /= A.sum(-1, keepdims=True)
    return A


# ---- P1: identity -> dense causal attention (torch SDPA) -------------------

@pytest.mark.parametrize("N,B", [(256, 16), (250, 16), (100, 32)])
def test_identity_reproduces_dense_attention_fp64(N, B):
    w = synth.workload("tiny-f32", N=N, B=B)
    L = synth.gen_layer(w, map_dtype="f64", return_qk=True)
    A = L["A"].numpy()
    V = L["V"].double().numpy()
    W = np.eye(w.H_s)
    _, kept, rp, ci, vals = oracle.compress(A, B, 1.0)
    assert rp[-1] == w.T * (w.T + 1) // 2
    O = oracle.retrieve(rp, ci, vals, W, V, N, B)
    q, k = L["Q"], L["K"]                                # [H][N][d] fp64
    v = torch.from_numpy(V).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    ref = ref.permute(1, 0, 2).numpy()
    err = np.abs(O - ref).max() / np.abs(ref).max()
    assert err < 1e-12, err


def test_identity_with_fp32_maps_within_fp32_bar():
    w = synth.workload("tiny-f32")
    L = synth.gen_layer(w, return_qk=True)               # maps stored fp32
    A = L["A"].numpy()
    V = L["V"].double().numpy()
    _, _, rp, ci, vals = oracle.compress(A, w.B, 1.0)
    O = oracle.retrieve(rp, ci, vals, np.eye(w.H_s), V, w.N, w.B)
    v = torch.from_numpy(V).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(L["Q"], L["K"], v, is_causal=True)
    ref = ref.permute(1, 0, 2).numpy()
    assert np.abs(O - ref).max() <= 1e-5 * np.abs(ref).max()


# ---- P2: brute-force decompress-then-matmul, scipy BSR ---------------------

@pytest.mark.parametrize("N,B,H_s,H_r,H_kv,d,p", [
    (100, 16, 3, 6, 2, 8, 0.7),
    (64, 16, 4, 4, 4, 5, 0.9),
    (37, 32, 2, 3, 1, 4, 0.5),
])
def test_retrieval_matches_dense_brute_force(N, B, H_s, H_r, H_kv, d, p):
    rng = np.random.default_rng(N * 7 + H_s)
    A = _random_causal_map(rng, H_s, N)
    W = rng.standard_normal((H_r, H_s))
    V = rng.standard_normal((N, H_kv, d))
    _, kept, rp, ci, vals = oracle.compress(A, B, p)
    O = oracle.retrieve(rp, ci, vals, W, V, N, B)
    ref = _dense_retrieval(_dense_from_bsr(rp, ci, vals, N, B), W, V)
    assert np.abs(O - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_retrieval_matches_scipy_bsr_for_one_hot_head_map():
    rng = np.random.default_rng(3)
    N, B, H_s = 96, 16, 3
    A = _random_causal_map(rng, H_s, N)
    V = rng.standard_normal((N, 1, 6))
    _, _, rp, ci, vals = oracle.compress(A, B, 0.8)
    for s0 in range(H_s):
        W = np.zeros((1, H_s))
        W[0, s0] = 1.0
        O = oracle.retrieve(rp, ci, vals, W, V, N, B)
        M = sp.bsr_matrix((vals[:, s0], ci, rp), shape=(N, N))
        ref = M @ V[:, 0, :]
        assert np.abs(O[:, 0, :] - ref).max() < 1e-12


def test_retrieval_of_arbitrary_pattern_matches_brute_force():
    """Retrieval must not rely on the pattern being a Top-p pattern."""
    rng = np.random.default_rng(11)
    N, B, H_s, H_r, H_kv, d = 70, 16, 3, 4, 2, 3
    T = oracle.n_blocks(N, B)
    A = rng.standard_normal((H_s, N, N))          # not even a probability map
    kept = [np.sort(rng.choice(I + 1, size=rng.integers(0, I + 2), replace=False))
            for I in range(T)]
    rp, ci, vals = oracle.build_bsr(A, B, kept)
    W = rng.standard_normal((H_r, H_s))
    V = rng.standard_normal((N, H_kv, d))
    O = oracle.retrieve(rp, ci, vals, W, V, N, B)
    ref = _dense_retrieval(_dense_from_bsr(rp, ci, vals, N, B), W, V)
    assert np.abs(O - ref).max() <= 1e-12 * np.abs(ref).max()


# ---- P3/P4/P5: Top-p invariants, brute force, monotonicity, extremes -------

def _brute_force_topp(m, p):
    """Smallest subset reaching p*total; among those, the heaviest (exhaustive)."""
    n = len(m)
    tot = float(np.sum(m))
    thr = float(np.float32(p)) * tot
    for size in range(1, n + 1):
        best = None
        for sub in itertools.combinations(range(n), size):
            s = sum(m[j] for j in sub)
            if s >= thr * (1 - 1e-12) and (best is None or s > best[0]):
                best = (s, sub)
        if best is not None:
            return size, best[0]
    return n, tot


@pytest.mark.parametrize("seed", range(6))
def test_topp_matches_exhaustive_search(seed):
    rng = np.random.default_rng(seed)
    for n in range(1, 11):
        m = rng.random(n) ** 4
        for p in (0.3, 0.6, 0.9, 0.99):
            kept = oracle.topp_row(m, p)
            size, best = _brute_force_topp(m, p)
            assert len(kept) == size, (m, p, kept)
            assert abs(sum(m[j] for j in kept) - best) <= 1e-12


@pytest.mark.parametrize("p", [0.5, 0.8, 0.9, 0.95, 0.999])
def test_topp_invariants_on_maps(p):
    w = synth.workload("pair14b8b-bf16", N=640, H_s=4)
    A = synth.gen_layer(w)["A"].float().numpy()
    mass = oracle.block_mass(A, w.B)
    kept = oracle.topp_select(mass, p)
    T = w.T
    rp, ci, vals = oracle.build_bsr(A, w.B, kept)
    check_bsr_structure(rp, ci, T)
    m32 = oracle.decision_masses(mass)
    for I in range(T):
        m = m32[I, : I + 1]
        S = set(kept[I].tolist())
        ks = np.array([m[j] for j in S])
        tot = m.sum()
        assert ks.sum() >= float(np.float32(p)) * tot * (1 - 1e-12)
        assert ks.sum() - ks.min() < float(np.float32(p)) * tot      # minimal
        dropped = [m[j] for j in range(I + 1) if j not in S]
        if dropped:
            assert ks.min() >= max(dropped)                          # heaviest kept
        assert selection_ok(mass[I, : I + 1], kept[I], kept[I], p) == "exact"


def test_topp_monotone_in_p():
    rng = np.random.default_rng(5)
    T = 24
    mass = np.tril(rng.random((T, T)) ** 3)
    prev = None
    nn_prev = 0
    for p in (0.1, 0.5, 0.8, 0.9, 0.95, 1.0):
        kept = oracle.topp_select(mass, p)
        nn = sum(len(k) for k in kept)
        assert nn >= nn_prev
        if prev is not None:
            for a, b in zip(prev, kept):
                assert set(a.tolist()) <= set(b.tolist())
        prev, nn_prev = kept, nn


def test_topp_extremes_and_ties():
    m = np.array([0.2, 0.5, 0.5, 0.1])
    assert oracle.topp_row(m, 1.0).tolist() == [0, 1, 2, 3]
    assert oracle.topp_row(m, 1e-9).tolist() == [1]        # arg-max, tie -> lower J
    assert oracle.topp_row(m, 0.38).tolist() == [1]        # 0.5 >= 0.38*1.3 = 0.494
    assert oracle.topp_row(m, 0.4).tolist() == [1, 2]      # 0.52 needs the tied block 2
    assert oracle.topp_row(np.zeros(5), 0.9).tolist() == [0]  # zero row: first block
    T = 9
    mass = np.tril(np.ones((T, T)))
    kept = oracle.topp_select(mass, 1.0)
    assert sum(len(k) for k in kept) == T * (T + 1) // 2
    kept = oracle.topp_select(mass, 1e-7)
    assert all(k.tolist() == [0] for k in kept)           # all tied -> column 0


# ---- P6: block-mass identities and a closed form ---------------------------

@pytest.mark.parametrize("N,B", [(256, 16), (250, 16), (97, 32)])
def test_block_mass_rows_sum_to_valid_row_count(N, B):
    w = synth.workload("tiny-f32", N=N, B=B)
    A = synth.gen_layer(w, map_dtype="f64")["A"].numpy()
    mass = oracle.block_mass(A, B)
    T = w.T
    for I in range(T):
        rows = min(N, (I + 1) * B) - I * B
        assert abs(mass[I].sum() - rows) < 1e-12
        assert (mass[I, I + 1:] == 0).all()


def test_block_mass_closed_form_uniform_attention():
    """A[h][i][j] = 1/(i+1) for j <= i: mass[I][J] = sum_i |J cap [0,i]| / (i+1)."""
    N, B, H = 23, 4, 3
    A = np.zeros((H, N, N))
    for i in range(N):
        A[:, i, : i + 1] = 1.0 / (i + 1)
    A[1] *= 2.0                                # heads weigh equally in the average
    A[2] *= 0.5
    mass = oracle.block_mass(A, B)
    T = oracle.n_blocks(N, B)
    scale = (1.0 + 2.0 + 0.5) / 3
    for I in range(T):
        for J in range(T):
            expect = 0.0
            if J <= I:
                for i in range(I * B, min(N, (I + 1) * B)):
                    lo, hi = J * B, min(N, (J + 1) * B, i + 1)
                    expect += max(0, hi - lo) / (i + 1)
            assert abs(mass[I, J] - scale * expect) < 1e-12, (I, J)


# ---- P7: algebra of the retrieval ------------------------------------------

def test_retrieval_algebra():
    rng = np.random.default_rng(9)
    N, B, H_s, H_r, H_kv, d = 80, 16, 3, 4, 2, 5
    A = _random_causal_map(rng, H_s, N)
    _, _, rp, ci, vals = oracle.compress(A, B, 0.85)
    W1, W2 = rng.standard_normal((2, H_r, H_s))
    V1, V2 = rng.standard_normal((2, N, H_kv, d))
    R = lambda W, V: oracle.retrieve(rp, ci, vals, W, V, N, B)
    assert np.abs(R(np.zeros((H_r, H_s)), V1)).max() == 0.0
    assert np.abs(R(W1 + W2, V1) - R(W1, V1) - R(W2, V1)).max() < 1e-12
    assert np.abs(R(W1, V1 + 2 * V2) - R(W1, V1) - 2 * R(W1, V2)).max() < 1e-12
    # swapping two receiver heads of one KV group swaps their outputs
    Wp = W1.copy()
    Wp[[0, 1]] = Wp[[1, 0]]
    assert np.abs(R(Wp, V1)[:, [1, 0]] - R(W1, V1)[:, [0, 1]]).max() < 1e-12


def test_single_block_is_a_dense_matmul():
    rng = np.random.default_rng(4)
    N, B, H_r, d = 13, 16, 3, 4
    A = _random_causal_map(rng, 1, N)
    W = rng.standard_normal((H_r, 1))
    V = rng.standard_normal((N, 1, d))
    _, _, rp, ci, vals = oracle.compress(A, B, 0.5)
    assert rp.tolist() == [0, 1]
    O = oracle.retrieve(rp, ci, vals, W, V, N, B)
    for r in range(H_r):
        assert np.abs(O[:, r, :] - W[r, 0] * (A[0] @ V[:, 0, :])).max() < 1e-12


def test_gqa_groups_are_consecutive_heads():
    rng = np.random.default_rng(2)
    N, B, H_s, H_r, H_kv, d = 32, 16, 2, 6, 3, 2
    A = _random_causal_map(rng, H_s, N)
    _, _, rp, ci, vals = oracle.compress(A, B, 1.0)
    W = np.ones((H_r, H_s))
    V = np.zeros((N, H_kv, d))
    V[:, 1, :] = 1.0                     # only KV head 1 is non-zero
    O = oracle.retrieve(rp, ci, vals, W, V, N, B)
    nz = [r for r in range(H_r) if np.abs(O[:, r, :]).max() > 0]
    assert nz == [2, 3]                  # G = 2: receiver heads 2, 3 read KV head 1


# ---- hand-worked example ----------------------------------------------------

def test_handworked_example():
    with open(os.path.join(GOLDEN, "handworked_n4_b2.json")) as f:
        g = json.load(f)
    A = np.array(g["A"])
    W = np.array(g["W"])
    V = np.array(g["V"])
    B = g["B"]
    assert np.abs(oracle.block_mass(A, B) - np.array(g["mass"])).max() < 1e-12
    for case in g["cases"]:
        mass, kept, rp, ci, vals = oracle.compress(A, B, case["p"])
        assert [k.tolist() for k in kept] == case["kept"]
        assert rp.tolist() == case["row_ptr"] and ci.tolist() == case["col_idx"]
        O = oracle.retrieve(rp, ci, vals, W, V, 4, B)
        assert np.abs(O[:, 0, 0] - np.array(case["O"])).max() < 1e-12


# ---- P8: the harness detects planted mistakes in the oracle's output -------

def test_planted_mistakes_are_detected():
    from tests._compare import check_output
    rng = np.random.default_rng(8)
    N, B, H_s, H_r, H_kv, d = 96, 16, 3, 4, 2, 8
    A = _random_causal_map(rng, H_s, N).astype(np.float32)
    W = rng.standard_normal((H_r, H_s))
    V = rng.standard_normal((N, H_kv, d))
    mass, kept, rp, ci, vals = oracle.compress(A, B, 0.9)
    O = oracle.retrieve(rp, ci, vals, W, V, N, B)
    check_output(O.astype(np.float32), O, "f32")
    # flip one kept value
    v2 = vals.copy()
    v2[len(v2) // 2, 1, 3, 5] += 0.25
    with pytest.raises(AssertionError):
        check_output(oracle.retrieve(rp, ci, v2, W, V, N, B), O, "f16")
    # drop one kept block
    I = oracle.n_blocks(N, B) - 1
    k2 = [k.copy() for k in kept]
    k2[I] = k2[I][1:]
    rp2, ci2, vals2 = oracle.build_bsr(A, B, k2)
    with pytest.raises(AssertionError):
        check_output(oracle.retrieve(rp2, ci2, vals2, W, V, N, B), O, "bf16")
    with pytest.raises(AssertionError):
        selection_ok(mass[I, : I + 1], kept[I], k2[I], 0.9)
    # permute col_idx within a row
    ci3 = ci.copy()
    a, b = rp[I], rp[I] + 1
    ci3[a], ci3[b] = ci3[b], ci3[a]
    with pytest.raises(AssertionError):
        check_output(oracle.retrieve(rp, ci3, vals, W, V, N, B), O, "f16")
    with pytest.raises(AssertionError):
        check_bsr_structure(rp, ci3, oracle.n_blocks(N, B))
    # a heavier block swapped for a lighter one is not a valid tie
    m = np.array([0.5, 0.3, 0.2])
    with pytest.raises(AssertionError):
        selection_ok(m, [0, 1], [0, 2], 0.75)


# ---------------------------------------------------------------------------
# compression from Q and K (no dense map)
# ---------------------------------------------------------------------------

def _qk_inputs(rng, H_s=4, H_ks=2, N=70, d=16):
    Q = rng.standard_normal((H_s, N, d))
    K = rng.standard_normal((H_ks, N, d))
    scale = rng.uniform(0.05, 0.6, H_s)
    return Q, K, scale


def _torch_causal(Q, K, scale):
    """Scores, causal softmax and logsumexp in float64 with torch (GQA by
    repeating each K head over consecutive sender heads)."""
    H_s, N, _ = Q.shape
    G = H_s // K.shape[0]
    q = torch.from_numpy(Q)
    k = torch.from_numpy(np.repeat(K, G, axis=0))
    s = torch.einsum("hid,hjd->hij", q, k) * torch.from_numpy(scale)[:, None, None]
    mask = torch.ones(N, N, dtype=torch.bool).triu_(1)
    s = s.masked_fill(mask, float("-inf"))
    return torch.softmax(s, dim=-1).numpy(), torch.logsumexp(s, dim=-1).numpy()


def test_qk_map_matches_torch_causal_softmax():
    rng = np.random.default_rng(11)
    Q, K, scale = _qk_inputs(rng)
    A_ref, lse_ref = _torch_causal(Q, K, scale)
    lse = oracle.row_lse(Q, K, scale)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)
    A = oracle.QKMap(Q, K, scale, lse)
    np.testing.assert_allclose(A[:, :, :], A_ref, rtol=0, atol=1e-14)
    # a sampled row range and column range of the lazy view
    np.testing.assert_allclose(A[1:3, 17:40, 5:33], A_ref[1:3, 17:40, 5:33], rtol=0, atol=1e-14)
    rows = np.array([0, 9, 69])
    np.testing.assert_allclose(oracle.row_lse(Q, K, scale, rows=rows), lse_ref[:, rows],
                               rtol=0, atol=1e-12)


def test_qk_zero_scores_closed_form():
    # all scores zero: every row i attends uniformly to keys 0..i
    N, B, H_s = 37, 8, 3
    Q = np.zeros((H_s, N, 4))
    K = np.ones((1, N, 4))
    scale = np.full(H_s, 0.5)
    lse = oracle.row_lse(Q, K, scale)
    np.testing.assert_allclose(lse, np.log(np.arange(1, N + 1))[None, :].repeat(H_s, 0),
                               rtol=0, atol=1e-14)
    mass = oracle.block_mass(oracle.QKMap(Q, K, scale, lse), B)
    T = oracle.n_blocks(N, B)
    for I in range(T):
        for J in range(I + 1):
            want = sum(len([j for j in range(J * B, min(N, (J + 1) * B)) if j <= i]) / (i + 1)
                       for i in range(I * B, min(N, (I + 1) * B)))
            assert abs(mass[I, J] - want) < 1e-13, (I, J)


def test_qk_brute_force_tiny():
    rng = np.random.default_rng(12)
    H_s, H_ks, N, d = 4, 2, 6, 3
    Q, K, scale = _qk_inputs(rng, H_s, H_ks, N, d)
    lse = oracle.row_lse(Q, K, scale)
    A = oracle.QKMap(Q, K, scale, lse)[:, :, :]
    for h in range(H_s):
        g = h // (H_s // H_ks)
        for i in range(N):
            s = [scale[h] * sum(Q[h, i, t] * K[g, j, t] for t in range(d)) for j in range(i + 1)]
            tot = sum(math.exp(x) for x in s)
            assert abs(lse[h, i] - math.log(tot)) < 1e-12
            for j in range(N):
                want = math.exp(s[j]) / tot if j <= i else 0.0
                assert abs(A[h, i, j] - want) < 1e-14


def test_compress_qk_equals_dense_compression():
    rng = np.random.default_rng(13)
    Q, K, scale = _qk_inputs(rng, H_s=3, H_ks=1, N=90, d=8)
    A_ref, _ = _torch_causal(Q, K, scale)
    for B, p in ((16, 0.9), (32, 0.5), (64, 1.0)):
        lse, mass, kept, rp, ci, vals = oracle.compress_qk(Q, K, scale, B, p)
        m2, k2, rp2, ci2, v2 = oracle.compress(A_ref, B, p)
        np.testing.assert_allclose(mass, m2, rtol=0, atol=1e-12)
        assert all(np.array_equal(a, b) for a, b in zip(kept, k2))
        assert np.array_equal(rp, rp2) and np.array_equal(ci, ci2)
        np.testing.assert_allclose(vals, v2, rtol=0, atol=1e-14)


def test_qk_planted_mistakes_are_detected():
    rng = np.random.default_rng(14)
    Q, K, scale = _qk_inputs(rng)
    A_ref, lse_ref = _torch_causal(Q, K, scale)
    H_s, N, _ = Q.shape

    def lse_with(kidx, causal=True, use_scale=True):
        out = np.empty((H_s, N))
        for h in range(H_s):
            s = (scale[h] if use_scale else 1.0) * (Q[h] @ K[kidx(h)].T)
            if causal:
                s = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], s, -np.inf)
            m = s.max(axis=1)
            out[h] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
        return out

    good = lse_with(lambda h: h // 2)
    np.testing.assert_allclose(good, lse_ref, rtol=0, atol=1e-12)
    for bad in (lse_with(lambda h: h % 2),            # interleaved instead of grouped KV heads
                lse_with(lambda h: h // 2, causal=False),
                lse_with(lambda h: h // 2, use_scale=False)):
        with pytest.raises(AssertionError):
            np.testing.assert_allclose(bad, lse_ref, rtol=0, atol=1e-6)


# ---- packed batches: retrieve_varlen -----------------------------------------

def _pack(seqs, B, rng, shuffle=True):
    """Pack per-sequence BSR states (row_ptr, col_idx, vals) into one batch with
    the pool pages in a random order; returns the batch arrays and the table."""
    cu, cr, rp, ci, tiles = [0], [0], [0], [], []
    for (N, row_ptr, col_idx, vals) in seqs:
        cu.append(cu[-1] + N)
        cr.append(cr[-1] + len(row_ptr) - 1)
        base = rp[-1]
        rp.extend(int(x) + base for x in row_ptr[1:])
        ci.extend(int(x) for x in col_idx)
        tiles.extend(vals)
    nnzb = len(ci)
    perm = rng.permutation(nnzb) if shuffle else np.arange(nnzb)
    pool = np.zeros((nnzb,) + np.asarray(tiles[0]).shape)
    for k in range(nnzb):
        pool[perm[k]] = tiles[k]
    return np.array(cu), np.array(cr), np.array(rp), np.array(ci), pool, perm


def test_varlen_identity_reproduces_each_sequence_attention():
    # p = 1, W = I: every sequence of the batch is its own dense causal attention
    rng = np.random.default_rng(31)
    B, H, d = 16, 3, 8
    lens = [1, 40, 16, 73]
    seqs, refs, Vs = [], [], []
    for n in lens:
        q = torch.from_numpy(rng.standard_normal((H, n, d)))
        k = torch.from_numpy(rng.standard_normal((H, n, d)))
        v = rng.standard_normal((n, H, d))
        A = torch.softmax((q @ k.transpose(1, 2)) / math.sqrt(d) +
                          torch.triu(torch.full((n, n), -math.inf, dtype=torch.float64), 1), -1).numpy()
        _, _, rp, ci, vals = oracle.compress(A, B, 1.0)
        seqs.append((n, rp, ci, vals))
        vt = torch.from_numpy(v).permute(1, 0, 2).contiguous()
        refs.append(torch.nn.functional.scaled_dot_product_attention(q, k, vt, is_causal=True)
                    .permute(1, 0, 2).numpy())
        Vs.append(v)
    cu, cr, rp, ci, pool, table = _pack(seqs, B, rng)
    O = oracle.retrieve_varlen(cu, cr, rp, ci, pool, np.eye(H), np.concatenate(Vs), B, table)
    ref = np.concatenate(refs)
    assert np.abs(O - ref).max() < 1e-12 * np.abs(ref).max()


def _varlen_brute(cu, cr, rp, ci, pool, W, V, B, table):
    """Token by token: O[t][r] = sum over the kept blocks of t's block row of
    sum_c (sum_s W[r][s] tile[s][i][c]) V[first token + J*B + c][r/G]."""
    H_r, d = W.shape[0], V.shape[2]
    G = H_r // V.shape[1]
    O = np.zeros((V.shape[0], H_r, d))
    for s in range(len(cu) - 1):
        for t in range(cu[s], cu[s + 1]):
            loc = t - cu[s]
            g = cr[s] + loc // B
            i = loc % B
            for k in range(rp[g], rp[g + 1]):
                J = ci[k]
                tile = pool[table[k]]
                for c in range(B):
                    key = J * B + c
                    if key >= cu[s + 1] - cu[s]:
                        continue
                    for r in range(H_r):
                        a = sum(W[r, h] * tile[h, i, c] for h in range(tile.shape[0]))
                        O[t, r] += a * V[cu[s] + key, r // G]
    return O


def test_varlen_matches_token_by_token_brute_force():
    rng = np.random.default_rng(32)
    B, H_s, H_r, H_kv, d = 8, 2, 4, 2, 3
    lens = [5, 17, 8, 0, 12]
    seqs = []
    for n in lens:
        if n == 0:
            seqs.append((0, np.array([0]), np.array([], dtype=np.int64), np.zeros((0, H_s, B, B))))
            continue
        A = _random_causal_map(rng, H_s, n)
        _, _, rp, ci, vals = oracle.compress(A, B, 0.7)
        seqs.append((n, rp, ci, vals))
    tiles = [v for s in seqs for v in s[3]]
    cu, cr, rp, ci, _, _ = _pack([s for s in seqs if s[0]], B, rng, shuffle=False)
    # rebuild with the empty sequence kept in place
    cu = np.cumsum([0] + lens)
    cr = np.cumsum([0] + [oracle.n_blocks(n, B) if n else 0 for n in lens])
    perm = rng.permutation(len(tiles))
    pool = np.zeros((len(tiles), H_s, B, B))
    for k, t in enumerate(tiles):
        pool[perm[k]] = t
    W = rng.standard_normal((H_r, H_s))
    V = rng.standard_normal((cu[-1], H_kv, d))
    O = oracle.retrieve_varlen(cu, cr, rp, ci, pool, W, V, B, perm)
    ref = _varlen_brute(cu, cr, rp, ci, pool, W, V, B, perm)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def test_varlen_planted_mistakes_are_detected():
    # the brute force above rejects: ignoring the block table, global instead of
    # local columns, and a sequence's V taken from the start of the batch
    rng = np.random.default_rng(33)
    B, H_s, H_r, H_kv, d = 8, 2, 2, 1, 4
    lens = [9, 20]
    seqs = []
    for n in lens:
        A = _random_causal_map(rng, H_s, n)
        _, _, rp, ci, vals = oracle.compress(A, B, 0.9)
        seqs.append((n, rp, ci, vals))
    cu, cr, rp, ci, pool, table = _pack(seqs, B, rng)
    W = rng.standard_normal((H_r, H_s))
    V = rng.standard_normal((cu[-1], H_kv, d))
    ref = _varlen_brute(cu, cr, rp, ci, pool, W, V, B, table)
    good = oracle.retrieve_varlen(cu, cr, rp, ci, pool, W, V, B, table)
    np.testing.assert_allclose(good, ref, atol=1e-12)
    bad_table = oracle.retrieve_varlen(cu, cr, rp, ci, pool, W, V, B, None)
    ci_global = ci.copy()
    for s in range(len(lens)):
        k0, k1 = rp[cr[s]], rp[cr[s + 1]]
        ci_global[k0:k1] += cr[s]
    # global columns point past the second sequence's own blocks: clamp so the
    # oracle still runs, which must change the result
    bad_cols = oracle.retrieve_varlen(cu, cr, rp, np.minimum(ci_global, 2), pool, W, V, B, table)
    V_shift = V.copy()
    V_shift[cu[1]:] = V[:cu[-1] - cu[1]]
    bad_v = oracle.retrieve_varlen(cu, cr, rp, ci, pool, W, V_shift, B, table)
    for bad in (bad_table, bad_cols, bad_v):
        assert np.abs(bad - ref).max() > 1e-6


# ---------------------------------------------------------------------------
# the per-row pipeline (row oracle of the end-to-end GPU cases)
# ---------------------------------------------------------------------------

def _pipeline_rows_match(fn, A, V, W, B, p):
    """True when fn(A, V, W, B, p, I) returns, for every block row I, exactly
    the row of the whole-map path: block_mass -> topp_select -> build_bsr ->
    retrieve (mass row, kept set, tiles, O rows)."""
    N = A.shape[1]
    mass, kept, rp, ci, vals = oracle.compress(A, B, p)
    O = oracle.retrieve(rp, ci, vals, W, V, N, B)
    for I in range(oracle.n_blocks(N, B)):
        m, k, tiles, O_r = fn(A, V, W, B, p, I)
        r0, r1 = I * B, min(N, (I + 1) * B)
        if not np.array_equal(m, mass[I, : I + 1]) or not np.array_equal(k, kept[I]):
            return False
        if len(tiles) != rp[I + 1] - rp[I]:
            return False
        for t, v in zip(tiles, vals[rp[I]:rp[I + 1]]):
            if t.dtype != v.dtype or not np.array_equal(t, v):
                return False
        if not np.array_equal(O_r, O[r0:r1]):
            return False
    return True


def _rounding_sensitive_map():
    """A 2-token, 1-token-block map whose second row's masses differ by 2^-30:
    as fp32 they tie (0.5, 0.5), so the decision on fp32 masses keeps the
    lower column; on the fp64 masses the heavier column 1 goes first."""
    u = 0.5 - 2.0 ** -30
    A = np.array([[[1.0, 0.0], [u, 1.0 - u]]])
    W = np.array([[1.5]])
    V = np.array([[[1.0]], [[-2.0]]])
    return A, V, W


@pytest.mark.parametrize("N,B,p,dtype", [(100, 16, 0.7, np.float64), (64, 16, 0.9, np.float32),
                                         (37, 32, 0.5, np.float64), (90, 16, 1.0, np.float32),
                                         (50, 16, 1e-7, np.float64)])
def test_pipeline_row_is_a_row_of_the_whole_map_path(N, B, p, dtype):
    rng = np.random.default_rng(N + int(p * 100))
    A = _random_causal_map(rng, 3, N).astype(dtype)
    W = rng.standard_normal((4, 3))
    V = rng.standard_normal((N, 2, 5))
    assert _pipeline_rows_match(oracle.pipeline_row, A, V, W, B, p)


def test_pipeline_row_decides_on_fp32_masses():
    A, V, W = _rounding_sensitive_map()
    m, kept, tiles, O = oracle.pipeline_row(A, V, W, 1, 0.5, 1)
    assert kept.tolist() == [0]                          # the fp32 tie goes to the lower column
    assert O[0, 0, 0] == pytest.approx(1.5 * (0.5 - 2.0 ** -30) * 1.0, abs=1e-15)
    assert _pipeline_rows_match(oracle.pipeline_row, A, V, W, 1, 0.5)


def test_pipeline_row_handworked_example():
    with open(os.path.join(GOLDEN, "handworked_n4_b2.json")) as f:
        g = json.load(f)
    A, W, V, B = np.array(g["A"]), np.array(g["W"]), np.array(g["V"]), g["B"]
    for case in g["cases"]:
        for I in range(2):
            m, kept, tiles, O = oracle.pipeline_row(A, V, W, B, case["p"], I)
            assert np.abs(m - np.array(g["mass"])[I, : I + 1]).max() < 1e-12
            assert kept.tolist() == case["kept"][I]
            assert np.abs(O[:, 0, 0] - np.array(case["O"])[I * B:(I + 1) * B]).max() < 1e-12


def test_pipeline_row_identity_reproduces_dense_attention():
    w = synth.workload("tiny-f32", N=100, B=16)
    L = synth.gen_layer(w, map_dtype="f64", return_qk=True)
    A, V = L["A"].numpy(), L["V"].double().numpy()
    v = torch.from_numpy(V).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(L["Q"], L["K"], v, is_causal=True)
    ref = ref.permute(1, 0, 2).numpy()
    for I in range(w.T):
        _, kept, _, O = oracle.pipeline_row(A, V, np.eye(w.H_s), w.B, 1.0, I)
        assert kept.tolist() == list(range(I + 1))
        r0, r1 = I * w.B, min(w.N, (I + 1) * w.B)
        assert np.abs(O - ref[r0:r1]).max() < 1e-12 * np.abs(ref).max()


def test_pipeline_row_matches_dense_brute_force():
    rng = np.random.default_rng(21)
    N, B = 70, 16
    A = _random_causal_map(rng, 3, N)
    W = rng.standard_normal((4, 3))
    V = rng.standard_normal((N, 2, 5))
    for I in range(oracle.n_blocks(N, B)):
        _, kept, tiles, O = oracle.pipeline_row(A, V, W, B, 0.8, I)
        D = np.zeros((3, N, N))                            # only this row's kept blocks
        for J, t in zip(kept, tiles):
            c1 = min(N, (J + 1) * B)
            D[:, I * B:min(N, (I + 1) * B), J * B:c1] = t[:, : min(N, (I + 1) * B) - I * B, : c1 - J * B]
        ref = _dense_retrieval(D, W, V)[I * B:min(N, (I + 1) * B)]
        assert np.abs(O - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_pipeline_row_planted_mistakes_are_detected():
    def unrounded(A, V, W, B, p, I):                     # decides on the fp64 masses
        m = oracle.block_mass_row(A, B, I)
        kept = oracle.topp_row(m, p)
        tiles = [oracle.bsr_tile(A, B, I, int(J)) for J in kept]
        return m, kept, tiles, oracle.retrieve_row(I, kept, tiles, W, V, A.shape[1], B)

    def swapped(A, V, W, B, p, I):                       # tile indices transposed
        m = oracle.block_mass_row(A, B, I)
        kept = oracle.topp_row(oracle.decision_masses(m), p)
        tiles = [oracle.bsr_tile(A, B, int(J), I) for J in kept]
        return m, kept, tiles, oracle.retrieve_row(I, kept, tiles, W, V, A.shape[1], B)

    A, V, W = _rounding_sensitive_map()
    assert not _pipeline_rows_match(unrounded, A, V, W, 1, 0.5)
    rng = np.random.default_rng(5)
    A2 = _random_causal_map(rng, 3, 64)
    W2, V2 = rng.standard_normal((4, 3)), rng.standard_normal((64, 2, 5))
    assert not _pipeline_rows_match(swapped, A2, V2, W2, 16, 0.9)
    assert _pipeline_rows_match(oracle.pipeline_row, A2, V2, W2, 16, 0.9)
