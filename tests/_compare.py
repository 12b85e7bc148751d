"""Comparators shared by the parity tests (test harness, not the product)."""
from __future__ import annotations

import numpy as np

EPS_TIE = 1e-6   # relative mass within which two blocks count as tied


def out_tolerance(dtype: str, O_ref: np.ndarray) -> np.ndarray:
    """Elementwise max-abs error allowed for an output of storage `dtype`.

    fp32: 1e-5 * max|O_ref|; fp16: 2e-3 * max|O_ref| (both as stated for the
    path).  bf16 has no stated bar; the path rounds its fp32 result to bf16
    once, which alone can cost half an ulp (2^-8 relative), so the bar is that
    half ulp plus the same 2e-3 * max|O_ref| compute allowance as fp16.
    """
    mx = float(np.abs(O_ref).max()) if O_ref.size else 0.0
    if dtype == "f32":
        return np.full(O_ref.shape, 1e-5 * mx)
    if dtype == "f16":
        return np.full(O_ref.shape, 2e-3 * mx)
    if dtype == "bf16":
        return 2.0 ** -8 * np.abs(O_ref) + 2e-3 * mx
    raise ValueError(dtype)


def check_output(O_gpu: np.ndarray, O_ref: np.ndarray, dtype: str, what: str = "O"):
    """Asserts |O_gpu - O_ref| <= tolerance elementwise; returns err/max."""
    O_gpu = np.asarray(O_gpu, dtype=np.float64)
    assert O_gpu.shape == O_ref.shape, (O_gpu.shape, O_ref.shape)
    assert np.isfinite(O_gpu).all(), f"{what}: non-finite outputs"
    err = np.abs(O_gpu - O_ref)
    tol = out_tolerance(dtype, O_ref)
    bad = err > tol
    mx = float(np.abs(O_ref).max()) if O_ref.size else 0.0
    rel = float(err.max() / mx) if mx > 0 else float(err.max(initial=0.0))
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} elements out of tolerance (dtype {dtype}); first at "
            f"{tuple(idx)}: gpu {O_gpu[tuple(idx)]!r} ref {O_ref[tuple(idx)]!r}; "
            f"max err/max|ref| = {rel:.3e}")
    return rel


def selection_ok(m_ref: np.ndarray, kept_ref, kept_gpu, p: float,
                 eps: float = EPS_TIE) -> str:
    """Compares one row's GPU kept set with the oracle's.

    Returns "exact" when the sets are equal, "tie" when they differ but the GPU
    set is still a valid Top-p set under masses perturbed within `eps`
    relative (contained in the causal range, reaches p, minimal, drops no
    heavier block), and raises otherwise.  m_ref are the oracle's masses of the
    row's candidates.
    """
    S = sorted(int(x) for x in kept_gpu)
    R = sorted(int(x) for x in kept_ref)
    if S == R:
        return "exact"
    n = len(m_ref)
    p = float(np.float32(p))
    if p >= 1.0:
        raise AssertionError(f"p=1 must keep all {n} blocks, got {S}")
    if not S or S[0] < 0 or S[-1] >= n or len(set(S)) != len(S):
        raise AssertionError(f"kept set {S} not inside 0..{n - 1}")
    tot = float(np.sum(m_ref))
    ms = np.asarray([m_ref[j] for j in S])
    if not ms.sum() >= (p - eps) * tot:
        raise AssertionError(f"kept mass {ms.sum()} < p*total {p * tot} (ref {R})")
    if not ms.sum() - ms.min() < (p + eps) * tot:
        raise AssertionError(f"kept set {S} not minimal (ref {R})")
    dropped = [m_ref[j] for j in range(n) if j not in set(S)]
    if dropped and not ms.min() >= (1 - eps) * max(dropped):
        raise AssertionError(f"kept set {S} drops a heavier block (ref {R})")
    return "tie"


def check_bsr_structure(row_ptr, col_idx, T: int):
    """Invariants every BSR state satisfies."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    assert row_ptr.shape == (T + 1,)
    assert row_ptr[0] == 0
    assert (np.diff(row_ptr) >= 0).all()
    nnzb = int(row_ptr[-1])
    assert nnzb <= T * (T + 1) // 2
    assert len(col_idx) >= nnzb
    for I in range(T):
        c = col_idx[row_ptr[I]:row_ptr[I + 1]]
        assert (c >= 0).all() and (c <= I).all(), f"row {I}: {c}"
        assert (np.diff(c) > 0).all(), f"row {I} not strictly ascending: {c}"
