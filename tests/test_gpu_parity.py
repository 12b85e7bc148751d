"""GPU parity: libmapflow (through its C boundary) against the fp64 oracle.

Inputs come from the seeded recipes in `synth`; the oracle always works on a
host copy of the same tensors and builds its own BSR, so nothing it consumes
comes from the HIP path.  Bars: block masses to 1e-6 relative; selection
equal to the oracle's apart from ties within 1e-6 relative mass; BSR values
bit for bit; outputs within the dtype bars of tests/_compare.py.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import cross_model_sparse_amd as mf
import oracle
import synth
from tests._compare import check_bsr_structure, check_output, selection_ok

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


class HostView:
    """Lazy host copy of a device map: slicing returns numpy (fp32 for bf16)."""

    def __init__(self, A: torch.Tensor):
        self.A = A
        self.shape = tuple(A.shape)

    def __getitem__(self, idx):
        return host(self.A[idx])


def gpu_pipeline(A, W, V, B, p, cap=None):
    mass = mf.block_mass(A, B)
    row_ptr, col_idx, vals, nnzb = mf.topp_select_bsr(mass, A, B, p, cap_nnzb=cap)
    O = mf.retrieve_fused(row_ptr, col_idx, vals, nnzb, W, V, A.shape[1], B)
    torch.cuda.synchronize()
    return mass, row_ptr, col_idx, vals, nnzb, O


def check_rows(rows, A_h, W_h, V_h, B, p, dtype, g_mass, g_rp, g_ci, g_vals, g_O,
               mass_tol=1e-6):
    """Per sampled block row: mass, selection, tiles bit for bit, outputs."""
    N = A_h.shape[1]
    ties = 0
    O_ref_rows, O_gpu_rows = [], []
    for I in rows:
        m_ref, kept_ref, tiles_ref, O_ref = oracle.pipeline_row(A_h, V_h, W_h, B, p, I)
        m_gpu = g_mass[I, : I + 1].astype(np.float64)
        assert np.all(np.abs(m_gpu - m_ref) <= mass_tol * np.abs(m_ref) + 1e-30), (
            f"row {I}: mass max rel err "
            f"{np.max(np.abs(m_gpu - m_ref) / np.maximum(np.abs(m_ref), 1e-30)):.3e}")
        assert np.all(g_mass[I, I + 1:] == 0)
        kept_gpu = g_ci[g_rp[I]:g_rp[I + 1]]
        how = selection_ok(m_ref, kept_ref, kept_gpu, p)
        if how == "tie":
            ties += 1
            continue
        for t, (J, tile_ref) in enumerate(zip(kept_ref, tiles_ref)):
            tile_gpu = g_vals[g_rp[I] + t]
            assert tile_gpu.dtype == tile_ref.dtype
            assert np.array_equal(tile_gpu, tile_ref), f"row {I} block {J}"
        r0, r1 = I * B, min(N, (I + 1) * B)
        O_ref_rows.append(O_ref)
        O_gpu_rows.append(g_O[r0:r1])
    if O_ref_rows:
        rel = check_output(np.concatenate(O_gpu_rows), np.concatenate(O_ref_rows), dtype)
    else:
        rel = 0.0
    return ties, rel


def run_end_to_end(w, device, rows=None, p=None, layer=0, seed=None):
    p = w.p if p is None else p
    say(f"[e2e] {w.name} N={w.N} B={w.B} H_s={w.H_s} H_r={w.H_r} H_kv={w.H_kv} "
        f"d={w.d} {w.dtype} p={p} seed={seed}")
    L = synth.gen_layer(w, layer=layer, device=device, seed=seed)
    A = L["A"]
    W = L["W"].to(device)
    V = L["V"].to(device)
    mass, rp, ci, vals, nnzb, O = gpu_pipeline(A, W, V, w.B, p)
    T = w.T
    g_rp = host(rp).astype(np.int64)
    check_bsr_structure(g_rp, host(ci)[:nnzb], T)
    assert g_rp[-1] == nnzb
    rows = list(range(T)) if rows is None else rows
    # copy only the kept tiles of the checked rows
    g_vals = {}
    for I in rows:
        for k in range(g_rp[I], g_rp[I + 1]):
            g_vals[k] = host(vals[k])
    ties, rel = check_rows(rows, HostView(A), host(L["W"]), host(L["V"]), w.B, p, w.dtype,
                           host(mass), g_rp, host(ci), g_vals, host(O))
    say(f"[e2e] nnzb={nnzb} density={nnzb / (T * (T + 1) / 2):.3f} "
        f"rows checked={len(rows)} ties={ties} max err/max={rel:.3e}")
    assert ties <= max(1, len(rows) // 50)
    return nnzb, mass, rp, O


# ---------------------------------------------------------------------------
# Retrieval alone on an oracle-built BSR
# ---------------------------------------------------------------------------

RETRIEVE_CASES = [
    # name, overrides, kernel that must run
    ("pair14b8b-bf16", dict(N=1000), "mfma"),                            # ragged, 5 sender chunks
    ("pair8b3b-f16", dict(N=1024), "mfma"),                              # fp16, G = 3, 3 receivers per wave
    ("long32k-f16", dict(N=900), "mfma"),                                # B = 128
    ("pair14b8b-bf16", dict(N=300, B=32, H_s=16, H_r=8, H_kv=2), "mfma"),  # B = 32, 1 receiver per wave
    ("pair14b8b-bf16", dict(N=520, H_s=48, H_r=32, H_kv=4), "mfma"),     # 6 chunks: two tile buffers
    ("pair8b3b-f16", dict(N=520, H_s=48, H_r=16, H_kv=8), "mfma"),       # fp16, 6 chunks, 2 per wave
    ("pair14b8b-bf16", dict(N=700, H_s=24, H_r=16, H_kv=4), "mfma"),     # 3 chunks (pair-style plan)
    ("pair14b8b-bf16", dict(N=333, H_s=8, H_r=24, H_kv=8), "mfma"),      # 1 chunk
    ("pair8b3b-f16", dict(N=200, B=16), "mfma"),                         # B = 16
    ("pair14b8b-bf16", dict(N=520, H_s=64, H_r=32, H_kv=4), "plain"),    # H_s > 48
    ("pair8b3b-f16", dict(N=400, d=64), "plain"),                        # d = 64
    ("pair14b8b-bf16", dict(N=260, H_r=48, H_kv=8), "plain"),            # H_r > 32
    ("pair14b8b-bf16", dict(N=130, H_r=64, H_kv=16, H_s=64, d=64), "plain"),  # max heads
    ("pair14b8b-bf16", dict(N=300, H_r=32, H_kv=32), "plain"),           # G = 1
    ("tiny-f32", dict(), "plain"),                                       # fp32
    ("tiny-f32", dict(N=333, B=64, d=128, H_r=8, H_kv=2), "plain"),      # fp32, B = 64
]


@pytest.mark.parametrize("name,ov,kernel", RETRIEVE_CASES)
def test_retrieve_on_oracle_bsr(gpu, name, ov, kernel):
    w = synth.workload(name, **ov)
    say(f"[retrieve] {name} {ov}")
    L = synth.gen_layer(w)                     # CPU generation: small sizes
    A_h, W_h, V_h = host(L["A"]), host(L["W"]), host(L["V"])
    _, kept, rp, ci, vals = oracle.compress(A_h, w.B, w.p)
    O_ref = oracle.retrieve(rp, ci, vals, W_h, V_h, w.N, w.B)
    tdt = synth.torch_dtype(w.dtype)
    d_vals = torch.from_numpy(vals).to(gpu).to(tdt)
    d_rp = torch.from_numpy(rp.astype(np.int32)).to(gpu)
    d_ci = torch.from_numpy(ci.astype(np.int32)).to(gpu)
    d_W, d_V = L["W"].to(gpu), L["V"].to(gpu)
    assert mf.retrieve_kernel(d_vals, d_V, d_W, w.N, w.B) == kernel
    O = mf.retrieve_fused(d_rp, d_ci, d_vals, len(ci), d_W, d_V, w.N, w.B)
    torch.cuda.synchronize()
    rel = check_output(host(O), O_ref, w.dtype)
    say(f"[retrieve] nnzb={len(ci)} max err/max={rel:.3e}")


# ---------------------------------------------------------------------------
# End to end (block mass -> Top-p/BSR -> retrieval), every row checked
# ---------------------------------------------------------------------------

E2E_CASES = [
    ("tiny-f32", dict()),
    ("tiny-f32", dict(N=250)),
    ("pair14b8b-bf16", dict(N=1000)),
    ("pair8b3b-f16", dict(N=1024)),
    ("long32k-f16", dict(N=1100)),
    ("varlen-bf16", dict(N=777)),
    ("pair14b8b-bf16", dict(N=300, B=32, H_s=16, H_r=8, H_kv=2)),
    ("pair8b3b-f16", dict(N=200, B=16, d=64)),
]


@pytest.mark.parametrize("name,ov", E2E_CASES)
def test_end_to_end_small(gpu, name, ov):
    run_end_to_end(synth.workload(name, **ov), gpu)


@pytest.mark.parametrize("p", [0.8, 0.95])
def test_end_to_end_varlen_p(gpu, p):
    run_end_to_end(synth.workload("varlen-bf16", N=1500), gpu, p=p)


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,B", [(1, 64), (7, 16), (50, 64), (64, 64), (65, 64)])
def test_tiny_and_partial_maps(gpu, N, B):
    for name in ("tiny-f32", "pair14b8b-bf16"):
        w = synth.workload(name, N=N, B=B, H_s=4 if name == "tiny-f32" else 40)
        run_end_to_end(w, gpu)


def test_p_one_keeps_every_causal_block(gpu):
    w = synth.workload("pair14b8b-bf16", N=640)
    nnzb, *_ = run_end_to_end(w, gpu, p=1.0)
    assert nnzb == w.T * (w.T + 1) // 2


def test_tiny_p_keeps_one_block_per_row(gpu):
    w = synth.workload("pair8b3b-f16", N=700)
    nnzb, *_ = run_end_to_end(w, gpu, p=1e-6)
    assert nnzb == w.T


def test_capacity_error_leaves_outputs_untouched(gpu):
    w = synth.workload("pair14b8b-bf16", N=640, H_s=8)
    A = synth.gen_layer(w, device=gpu)["A"]
    mass = mf.block_mass(A, w.B)
    _, _, _, nnzb = mf.topp_select_bsr(mass, A, w.B, w.p)
    cap = nnzb - 1
    ci = torch.full((cap,), -7, dtype=torch.int32, device=gpu)
    vals = torch.full((cap, w.H_s, w.B, w.B), 3.0, dtype=A.dtype, device=gpu)
    with pytest.raises(mf.CapacityError) as e:
        mf.topp_select_bsr(mass, A, w.B, w.p, cap_nnzb=cap, col_idx=ci, vals=vals)
    assert e.value.nnzb == nnzb
    torch.cuda.synchronize()
    assert (ci == -7).all().item() and (vals == 3.0).all().item()


def test_empty_rows_and_bad_columns(gpu):
    """Rows without kept blocks give O = 0; columns outside [0, T) and block
    indices beyond nnzb are skipped, not read."""
    w = synth.workload("pair14b8b-bf16", N=512)
    L = synth.gen_layer(w)
    A_h, W_h, V_h = host(L["A"]), host(L["W"]), host(L["V"])
    T = w.T
    kept = [np.array([0, I]) if I % 3 == 0 and I > 0 else np.zeros(0, np.int64)
            for I in range(T)]
    kept[0] = np.array([0])
    rp, ci, vals = oracle.build_bsr(A_h, w.B, kept)
    O_ref = oracle.retrieve(rp, ci, vals, W_h, V_h, w.N, w.B)
    bad_ci = ci.copy()
    # append a bogus block to the last row: column T (out of range)
    rp2 = rp.copy()
    rp2[-1] += 1
    bad_ci = np.concatenate([bad_ci, [T]])
    vals2 = np.concatenate([vals, vals[:1]])
    tdt = synth.torch_dtype(w.dtype)
    O = mf.retrieve_fused(torch.from_numpy(rp2.astype(np.int32)).to(gpu),
                          torch.from_numpy(bad_ci.astype(np.int32)).to(gpu),
                          torch.from_numpy(vals2).to(gpu).to(tdt), len(bad_ci),
                          L["W"].to(gpu), L["V"].to(gpu), w.N, w.B)
    torch.cuda.synchronize()
    check_output(host(O), O_ref, w.dtype)
    # nnzb smaller than row_ptr claims: blocks beyond it are skipped
    O2 = mf.retrieve_fused(torch.from_numpy(rp.astype(np.int32)).to(gpu),
                           torch.from_numpy(ci.astype(np.int32)).to(gpu),
                           torch.from_numpy(vals).to(gpu).to(tdt), 0,
                           L["W"].to(gpu), L["V"].to(gpu), w.N, w.B)
    torch.cuda.synchronize()
    assert (O2 == 0).all().item()


def test_strided_V_and_O(gpu):
    """V as a slice of a fused [N][3*H_kv*d] projection, O inside a wider buffer."""
    w = synth.workload("pair8b3b-f16", N=448)
    L = synth.gen_layer(w)
    A_h, W_h, V_h = host(L["A"]), host(L["W"]), host(L["V"])
    _, _, rp, ci, vals = oracle.compress(A_h, w.B, w.p)
    O_ref = oracle.retrieve(rp, ci, vals, W_h, V_h, w.N, w.B)
    tdt = synth.torch_dtype(w.dtype)
    qkv = torch.randn(w.N, 3, w.H_kv, w.d, dtype=tdt, device=gpu)
    qkv[:, 2] = L["V"].to(gpu)
    V = qkv[:, 2]
    assert V.stride(0) == 3 * w.H_kv * w.d
    Obuf = torch.full((w.N, w.H_r + 8, w.d), 9.0, dtype=tdt, device=gpu)
    O = Obuf[:, 4:4 + w.H_r]
    mf.retrieve_fused(torch.from_numpy(rp.astype(np.int32)).to(gpu),
                      torch.from_numpy(ci.astype(np.int32)).to(gpu),
                      torch.from_numpy(vals).to(gpu).to(tdt), len(ci),
                      L["W"].to(gpu), V, w.N, w.B, out=O)
    torch.cuda.synchronize()
    check_output(host(O), O_ref, w.dtype)
    assert (Obuf[:, :4] == 9.0).all().item() and (Obuf[:, 4 + w.H_r:] == 9.0).all().item()


def test_repeat_runs_are_bitwise_identical(gpu):
    w = synth.workload("pair14b8b-bf16", N=1024)
    L = synth.gen_layer(w, device=gpu)
    W, V = L["W"].to(gpu), L["V"].to(gpu)
    r1 = gpu_pipeline(L["A"], W, V, w.B, w.p)
    r2 = gpu_pipeline(L["A"], W, V, w.B, w.p)
    for a, b in zip(r1, r2):
        if isinstance(a, torch.Tensor):
            assert torch.equal(a, b)
        else:
            assert a == b


def test_selection_at_max_block_rows_kept_sets(gpu):
    """T = 4096 block rows (B = 16, one sender head): the kept columns of
    sampled rows equal the oracle's Top-p sets, ties aside.  The masses are
    random; the map only supplies tiles (never compared), so it is left
    uninitialised."""
    T, B = 4096, 16
    N = T * B
    g = torch.Generator().manual_seed(78)
    mass = torch.tril(torch.rand(T, T, generator=g) ** 6).contiguous()
    A = torch.empty(1, N, N, dtype=torch.float16, device=gpu)       # 8.6 GB, never read back
    rp, ci, vals, nnzb = mf.topp_select_bsr(mass.to(gpu), A, B, 0.9)
    g_rp = host(rp).astype(np.int64)
    g_ci = host(ci[:nnzb]).astype(np.int64)
    m32 = mass.numpy().astype(np.float64)
    ties = 0
    rows = [0, 1, 2, 100, 1023, 1024, 2047, 3000] + list(range(4088, 4096))
    for I in rows:
        kept_ref = oracle.topp_row(oracle.decision_masses(m32[I, : I + 1]), 0.9)
        kept_gpu = g_ci[g_rp[I]:g_rp[I + 1]]
        assert np.all(np.diff(kept_gpu) > 0) and kept_gpu[0] >= 0 and kept_gpu[-1] <= I
        ties += selection_ok(m32[I, : I + 1], kept_ref, kept_gpu, 0.9) == "tie"
    say(f"[T=4096] nnzb={nnzb} rows checked={len(rows)} ties={ties}")
    assert ties <= 1
    del A, vals


def test_selection_at_max_block_rows(gpu):
    """T = 4096 block rows: selection counts equal the oracle's on sampled rows.
    Capacity 0, so the map itself is never read."""
    T, B = 4096, 64
    N = T * B
    g = torch.Generator().manual_seed(77)
    mass = torch.rand(T, T, generator=g) ** 6
    mass = torch.tril(mass).contiguous()
    d_mass = mass.to(gpu)
    A_dummy = torch.zeros(1, 1, 1, dtype=torch.float16, device=gpu)
    L = mf.load()
    import ctypes
    ws = torch.empty(mf.topp_workspace_bytes(N, B), dtype=torch.uint8, device=gpu)
    rp = torch.empty(T + 1, dtype=torch.int32, device=gpu)
    n = ctypes.c_int64(0)
    st = L.mf_topp_select_bsr(d_mass.data_ptr(), A_dummy.data_ptr(), mf.MF_F16, 8, N, B,
                              0.9, rp.data_ptr(), None, None, 0, ctypes.byref(n),
                              ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == mf.MF_ERR_CAPACITY
    g_rp = host(rp).astype(np.int64)
    assert g_rp[-1] == n.value
    m32 = mass.numpy().astype(np.float64)
    for I in [0, 1, 100, 2047, 4094, 4095]:
        kept = oracle.topp_row(m32[I, : I + 1], 0.9)
        assert g_rp[I + 1] - g_rp[I] == len(kept), I


# ---------------------------------------------------------------------------
# Full sizes, sampled block rows (same launch configuration as the benchmark)
# ---------------------------------------------------------------------------

def _sample_rows(T, extra=6, seed=0):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, T // 2, T - 2, T - 1}
    return sorted(fixed | set(rng.choice(T, size=extra, replace=False).tolist()))


def test_full_pair14b8b_bf16_layer(gpu):
    """The headline layer at full size, every block row checked."""
    w = synth.workload("pair14b8b-bf16")
    nnzb, mass, rp, O = run_end_to_end(w, gpu, layer=3)
    dens = nnzb / (w.T * (w.T + 1) / 2)
    assert 0.05 <= dens <= 0.25, dens
    m = host(mass)
    rows = np.minimum(w.B, w.N - np.arange(w.T) * w.B)
    assert np.all(np.abs(m.sum(1) - rows) <= 1e-2 * rows)
    assert torch.isfinite(O.float()).all().item()


def test_full_pair8b3b_f16_every_row(gpu):
    w = synth.workload("pair8b3b-f16")
    nnzb, *_ = run_end_to_end(w, gpu)
    assert nnzb > 0.8 * w.T * (w.T + 1) / 2


def test_full_long32k_f16(gpu):
    w = synth.workload("long32k-f16")
    rows = _sample_rows(w.T, extra=30)
    assert len(rows) >= 32
    nnzb, *_ = run_end_to_end(w, gpu, rows=rows)
    dens = nnzb / (w.T * (w.T + 1) / 2)
    say(f"[long] density {dens:.3f}")
    assert 0.03 <= dens <= 0.2, dens


def test_full_varlen_sequences(gpu):
    w0 = synth.workload("varlen-bf16")
    lens = synth.varlen_lengths(w0)
    # shortest, longest and one ragged length of the packed batch, each p
    ragged = [l for l in lens if l % w0.B][:1]
    picks = sorted({min(lens), max(lens), *ragged})
    for i, n in enumerate(picks):
        for p in w0.extra["ps"]:
            w = w0.with_(N=n)
            run_end_to_end(w, gpu, rows=_sample_rows(w.T, extra=2, seed=i), p=p,
                           seed=5000 + lens.index(n))


def test_full_long32k_past_2_31_elements(gpu):
    """Long-context layer at p = 0.97: the compressed state passes 2^31
    elements of vals (4096 blocks of 32 x 128 x 128), so block offsets in the
    gather and the retrieval need 64 bits.  Sampled rows, the last ones
    (whose blocks sit beyond 2^31 elements) among them, against the oracle."""
    w = synth.workload("long32k-f16")
    rows = sorted({0, 1, 128, 200} | set(range(w.T - 6, w.T)))
    nnzb, mass, rp, O = run_end_to_end(w, gpu, rows=rows, p=0.97)
    elems = nnzb * w.H_s * w.B * w.B
    say(f"[long p=0.97] nnzb={nnzb}, vals elements {elems:.3e} (2^31 = {2**31:.3e})")
    assert elems > 2 ** 31
    assert int(host(rp)[w.T - 6]) * w.H_s * w.B * w.B > 2 ** 31   # the checked last rows lie past it


@pytest.mark.parametrize("name,ov", [("pair14b8b-bf16", dict(N=1111)), ("tiny-f32", dict(N=250)),
                                     ("pair8b3b-f16", dict(N=700, B=32))])
def test_block_mass_variants_agree(gpu, name, ov):
    # the row-streaming kernels (workspace) and the column-strip scan compute the
    # same statistic; both against the oracle, each bit-reproducible
    w = synth.workload(name, **ov)
    L = synth.gen_layer(w, device=gpu)
    A = L["A"]
    m_ws = mf.block_mass(A, w.B)
    m_ws2 = mf.block_mass(A, w.B)
    m_strip = mf.block_mass(A, w.B, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(m_ws, m_ws2)
    ref = oracle.block_mass(HostView(A), w.B)
    for m in (host(m_ws), host(m_strip)):
        tri = np.tril_indices(w.T)
        rel = np.abs(m[tri] - ref[tri]) / np.maximum(np.abs(ref[tri]), 1e-30)
        assert rel.max() <= 1e-6, rel.max()
        assert np.all(np.triu(m, 1) == 0)


@pytest.mark.parametrize("name,ov", [("pair14b8b-bf16", dict(N=640, H_s=8)),
                                     ("pair8b3b-f16", dict(N=333, H_s=8)),
                                     ("tiny-f32", dict(N=256))])
def test_map_off_a_16_byte_boundary(gpu, name, ov):
    # the same map stored one element into a larger buffer: every row starts off
    # a 16-byte boundary, so block mass and the tile gather take their
    # element-aligned 16-byte loads; results against the oracle as everywhere
    w = synth.workload(name, **ov)
    L = synth.gen_layer(w, device=gpu)
    A0 = L["A"]
    buf = torch.empty(A0.numel() + 1, dtype=A0.dtype, device=gpu)
    A = buf[1:].view(A0.shape)
    A.copy_(A0)
    assert A.data_ptr() % 16 != 0
    say(f"[offset map] {w.name} N={w.N} B={w.B} H_s={w.H_s} {w.dtype}")
    W, V = L["W"].to(gpu), L["V"].to(gpu)
    mass, rp, ci, vals, nnzb, O = gpu_pipeline(A, W, V, w.B, w.p)
    m_strip = mf.block_mass(A, w.B, workspace=False)
    torch.cuda.synchronize()
    g_rp = host(rp).astype(np.int64)
    check_bsr_structure(g_rp, host(ci)[:nnzb], w.T)
    g_vals = {k: host(vals[k]) for k in range(nnzb)}
    ties, _ = check_rows(list(range(w.T)), HostView(A0), host(L["W"]), host(L["V"]), w.B, w.p,
                         w.dtype, host(mass), g_rp, host(ci), g_vals, host(O))
    assert ties <= 1
    ref = oracle.block_mass(HostView(A0), w.B)
    tri = np.tril_indices(w.T)
    m = host(m_strip)
    assert (np.abs(m[tri] - ref[tri]) / np.maximum(np.abs(ref[tri]), 1e-30)).max() <= 1e-6
