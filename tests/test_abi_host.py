"""C boundary checks that need no GPU: the library loads, exports every symbol
declared in include/mapflow.h, and rejects bad arguments on the host before any
GPU work (every call below returns before its first HIP call)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import cross_model_sparse_amd as mf
from cross_model_sparse_amd import mapflow as mfb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mapflow.h")

FAKE = 0x10000   # never dereferenced: validation fails before any use


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mf_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return mf.load()


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(mf.EXPORTED)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", str(mf.lib_path())],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mf_[a-z_]+)\b", out))
    assert set(names) <= exported


def test_version_and_status_strings(L):
    assert mf.abi_version() == 7
    for st in range(5):
        assert L.mf_status_string(st)
    assert b"unknown" in L.mf_status_string(99)


def test_retrieve_workspace_size(L):
    # the retrieval kernels need no scratch: every configuration reports 0
    import torch
    for args in [(8192, 64, 8, 128, torch.bfloat16), (4096, 64, 8, 128, torch.float16),
                 (256, 16, 4, 64, torch.float32)]:
        assert mf.retrieve_workspace_bytes(*args) == 0
    assert L.mf_retrieve_workspace_bytes(0, 64, 8, 128, 2) == 0


def test_workspace_size(L):
    assert mf.topp_workspace_bytes(8192, 64) >= (128 * 128 + 128) * 4
    assert mf.topp_workspace_bytes(8192, 64) % 256 == 0
    assert mf.topp_workspace_bytes(0, 64) == 0


def _last(L):
    return L.mf_last_error().decode()


@pytest.mark.parametrize("args,frag", [
    ((None, 2, 40, 8192, 64), "null"),
    ((FAKE, 7, 40, 8192, 64), "dtype"),
    ((FAKE, 2, 0, 8192, 64), "H_s"),
    ((FAKE, 2, 65, 8192, 64), "H_s"),
    ((FAKE, 2, 40, 0, 64), "N must"),
    ((FAKE, 2, 40, 8192, 48), "B must"),
])
def test_block_mass_rejects(L, args, frag):
    A, dt, H_s, N, B = args
    st = L.mf_block_mass(A, dt, H_s, N, B, FAKE if A else FAKE, None)
    assert st == mf.MF_ERR_INVALID
    assert frag in _last(L)


def _topp(L, **kw):
    a = dict(mass=FAKE, A=FAKE, dt=2, H_s=40, N=8192, B=64, p=0.9, row_ptr=FAKE,
             col_idx=FAKE, vals=FAKE, cap=10, nnzb_out=None, ws=FAKE,
             ws_bytes=mf.topp_workspace_bytes(8192, 64))
    a.update(kw)
    return L.mf_topp_select_bsr(a["mass"], a["A"], a["dt"], a["H_s"], a["N"], a["B"],
                                a["p"], a["row_ptr"], a["col_idx"], a["vals"], a["cap"],
                                a["nnzb_out"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,st,frag", [
    (dict(p=0.0), mf.MF_ERR_INVALID, "p must"),
    (dict(p=1.5), mf.MF_ERR_INVALID, "p must"),
    (dict(p=float("nan")), mf.MF_ERR_INVALID, "p must"),
    (dict(p=-0.1), mf.MF_ERR_INVALID, "p must"),
    (dict(mass=None), mf.MF_ERR_INVALID, "null"),
    (dict(ws=None), mf.MF_ERR_INVALID, "null"),
    (dict(cap=-1), mf.MF_ERR_INVALID, "cap_nnzb"),
    (dict(vals=None), mf.MF_ERR_INVALID, "null col_idx/vals"),
    (dict(ws_bytes=100), mf.MF_ERR_INVALID, "workspace"),
    (dict(N=4096 * 128 + 1, B=128), mf.MF_ERR_UNSUPPORTED, "4096"),
    (dict(B=8), mf.MF_ERR_INVALID, "B must"),
])
def test_topp_rejects(L, kw, st, frag):
    assert _topp(L, **kw) == st
    assert frag in _last(L)


def _retr(L, **kw):
    a = dict(row_ptr=FAKE, col_idx=FAKE, vals=FAKE, nnzb=5, dt=2, H_s=40, N=8192,
             B=64, W=FAKE, H_r=32, V=FAKE, H_kv=8, d=128, ldV=8 * 128, O=FAKE,
             ldO=32 * 128, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return L.mf_retrieve_fused(a["row_ptr"], a["col_idx"], a["vals"], a["nnzb"], a["dt"],
                               a["H_s"], a["N"], a["B"], a["W"], a["H_r"], a["V"],
                               a["H_kv"], a["d"], a["ldV"], a["O"], a["ldO"], a["ws"],
                               a["ws_bytes"], None)


@pytest.mark.parametrize("kw,frag", [
    (dict(H_r=30), "multiple of H_kv"),
    (dict(H_kv=0), "multiple of H_kv"),
    (dict(H_r=65, H_kv=5), "H_r must"),
    (dict(d=96), "d must"),
    (dict(ldV=8 * 128 - 1), "ldV"),
    (dict(ldO=100), "ldO"),
    (dict(W=None), "null"),
    (dict(nnzb=-1), "nnzb"),
    (dict(vals=None), "null col_idx/vals"),
    (dict(dt=3), "dtype"),
])
def test_retrieve_rejects(L, kw, frag):
    assert _retr(L, **kw) == mf.MF_ERR_INVALID
    assert frag in _last(L)


A16 = 0x100000                           # 16-byte aligned fake address


@pytest.mark.parametrize("shape,expect", [
    # (dtype, H_s, N, B, H_r, H_kv, d), kernel
    ((2, 40, 8192, 64, 32, 8, 128), 1),      # 14B->8B-like pair, bf16
    ((1, 32, 4096, 64, 24, 8, 128), 1),      # 8B->3B-like pair, fp16, G = 3
    ((1, 32, 32768, 128, 32, 8, 128), 1),    # long context, B = 128
    ((2, 32, 4096, 64, 24, 8, 128), 1),      # varlen pair, bf16
    ((2, 16, 300, 32, 8, 2, 128), 1),        # one receiver per wavefront
    ((2, 48, 520, 64, 32, 4, 128), 1),       # 48 sender heads (two tile buffers)
    ((1, 8, 200, 16, 16, 8, 128), 1),        # B = 16
    ((0, 4, 256, 16, 4, 4, 64), 0),          # fp32
    ((1, 32, 400, 64, 24, 8, 64), 0),        # d = 64
    ((2, 64, 520, 64, 32, 4, 128), 0),       # H_s > 48
    ((2, 40, 260, 64, 48, 8, 128), 0),       # H_r > 32
    ((2, 40, 300, 64, 32, 32, 128), 0),      # 4 receivers per wavefront span 4 KV heads
    ((2, 40, 300, 64, 30, 10, 128), 0),      # H_r not a multiple of 8
])
def test_retrieve_kernel_choice(L, shape, expect):
    dt, H_s, N, B, H_r, H_kv, d = shape
    got = L.mf_retrieve_kernel(dt, H_s, N, B, H_r, H_kv, d, A16, A16, H_kv * d, A16, H_r * d)
    assert got == expect


def test_retrieve_kernel_alignment_and_errors(L):
    args = (2, 40, 8192, 64, 32, 8, 128)
    ok = L.mf_retrieve_kernel(*args, A16, A16, 8 * 128, A16, 32 * 128)
    assert ok == 1
    # V rows must be 16-byte aligned for the matrix-core kernel's direct-to-LDS copies
    assert L.mf_retrieve_kernel(*args, A16, A16 + 8, 8 * 128, A16, 32 * 128) == 0
    assert L.mf_retrieve_kernel(*args, A16, A16, 8 * 128 + 4, A16, 32 * 128) == 0
    assert L.mf_retrieve_kernel(*args, A16 + 8, A16, 8 * 128, A16, 32 * 128) == 0
    assert L.mf_retrieve_kernel(*args, A16, A16, 8 * 128, A16, 32 * 128 + 4) == 0
    # shapes mf_retrieve_fused rejects
    assert L.mf_retrieve_kernel(2, 40, 8192, 64, 30, 8, 128, A16, A16, 1024, A16, 4096) == -mf.MF_ERR_INVALID
    assert L.mf_retrieve_kernel(2, 40, 8192, 64, 32, 8, 96, A16, A16, 1024, A16, 4096) == -mf.MF_ERR_INVALID


def test_last_error_is_thread_local(L):
    import threading
    _retr(L, d=96)
    seen = {}

    def other():
        seen["msg"] = L.mf_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "d must" in _last(L)


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(mf.MapflowError):
        mf.block_mass(torch.zeros(2, 8, 8), 16)


def test_header_documents_every_entry_point():
    src = open(HEADER).read()
    for name in declared_functions():
        m = re.search(r"\n(?:int|size_t|void|const char\*|mf_block_manager\*)\s+" + name + r"\(", src)
        assert m, name
        before = src[max(0, m.start() - 1500):m.start()]
        assert before.rstrip().endswith("*/"), f"{name} has no comment block"


# ---- compression from Q and K ----------------------------------------------

def _qk_args(**kw):
    a = dict(Q=FAKE, K=FAKE, dt=2, H_s=32, H_ks=8, N=4096, d=128, B=64, scale=FAKE, lse=FAKE,
             mass=FAKE, ws=FAKE, ws_bytes=1 << 30, p=0.9, row_ptr=FAKE, col_idx=FAKE, vals=FAKE,
             cap=10)
    a.update(kw)
    return a


QK_BAD = [
    (dict(dt=7), "dtype"), (dict(H_s=0), "H_s"), (dict(H_s=65), "H_s"), (dict(N=0), "N must"),
    (dict(H_ks=0), "H_ks"), (dict(H_ks=3), "H_ks"), (dict(d=96), "d must"),
    (dict(Q=None), "null"), (dict(K=None), "null"), (dict(scale=None), "null"),
]


@pytest.mark.parametrize("kw,frag", QK_BAD)
def test_row_lse_rejects(L, kw, frag):
    a = _qk_args(**kw)
    st = L.mf_row_lse(a["Q"], a["K"], a["dt"], a["H_s"], a["H_ks"], a["N"], a["d"], a["scale"],
                      a["lse"], None)
    assert st == mf.MF_ERR_INVALID
    assert frag in L.mf_last_error().decode()


@pytest.mark.parametrize("kw,frag", QK_BAD + [(dict(B=48), "B must"), (dict(lse=None), "null"),
                                              (dict(ws=None), "null"), (dict(ws_bytes=16), "workspace")])
def test_block_mass_qk_rejects(L, kw, frag):
    a = _qk_args(**kw)
    st = L.mf_block_mass_qk(a["Q"], a["K"], a["scale"], a["lse"], a["dt"], a["H_s"], a["H_ks"],
                            a["N"], a["d"], a["B"], a["mass"], a["ws"], a["ws_bytes"], None)
    assert st == mf.MF_ERR_INVALID
    assert frag in L.mf_last_error().decode()


@pytest.mark.parametrize("kw,st,frag", [(k, mf.MF_ERR_INVALID, f) for k, f in QK_BAD] + [
    (dict(p=0.0), mf.MF_ERR_INVALID, "p must"), (dict(p=float("nan")), mf.MF_ERR_INVALID, "p must"),
    (dict(cap=-1), mf.MF_ERR_INVALID, "cap_nnzb"), (dict(vals=None), mf.MF_ERR_INVALID, "null"),
    (dict(ws_bytes=4), mf.MF_ERR_INVALID, "workspace"),
    (dict(N=16 * 4097, B=16), mf.MF_ERR_UNSUPPORTED, "4096")])
def test_topp_qk_rejects(L, kw, st, frag):
    a = _qk_args(**kw)
    r = L.mf_topp_select_bsr_qk(a["mass"], a["Q"], a["K"], a["scale"], a["lse"], a["dt"], a["H_s"],
                                a["H_ks"], a["N"], a["d"], a["B"], a["p"], a["row_ptr"], a["col_idx"],
                                a["vals"], a["cap"], None, a["ws"], a["ws_bytes"], None)
    assert r == st
    assert frag in L.mf_last_error().decode()


def test_block_mass_qk_workspace_size(L):
    # H_s * ceil(N/16) * T float32 partial sums
    assert L.mf_block_mass_qk_workspace_bytes(32, 4096, 64) == 32 * 256 * 64 * 4
    assert L.mf_block_mass_qk_workspace_bytes(3, 100, 32) == 3 * 7 * 4 * 4
    assert L.mf_block_mass_qk_workspace_bytes(0, 100, 32) == 0
    assert L.mf_block_mass_qk_workspace_bytes(3, 100, 48) == 0


# ---- packed batches -----------------------------------------------------------

def _varlen(L, **kw):
    a = dict(S=3, R=10, cu=FAKE, cr=FAKE, row_ptr=FAKE, col_idx=FAKE, table=None, vals=FAKE,
             n_pages=0, nnzb=5, dt=2, H_s=40, B=64, W=FAKE, H_r=32, V=FAKE, H_kv=8, d=128,
             ldV=8 * 128, O=FAKE, ldO=32 * 128)
    a.update(kw)
    return L.mf_retrieve_fused_varlen(a["S"], a["R"], a["cu"], a["cr"], a["row_ptr"], a["col_idx"],
                                      a["table"], a["vals"], a["n_pages"], a["nnzb"], a["dt"],
                                      a["H_s"], a["B"], a["W"], a["H_r"], a["V"], a["H_kv"], a["d"],
                                      a["ldV"], a["O"], a["ldO"], None)


@pytest.mark.parametrize("kw,frag", [
    (dict(S=0), "S must"), (dict(R=-1), "R < 0"), (dict(cu=None), "null"), (dict(cr=None), "null"),
    (dict(row_ptr=None), "null"), (dict(O=None), "null"), (dict(nnzb=-1), "nnzb"),
    (dict(col_idx=None), "null col_idx/vals"), (dict(table=FAKE, n_pages=-2), "n_pages"),
    (dict(B=48), "B must"), (dict(H_s=0), "H_s"), (dict(H_r=30), "multiple of H_kv"),
    (dict(d=96), "d must"), (dict(ldO=100), "ldO"), (dict(dt=5), "dtype"),
])
def test_retrieve_varlen_rejects(L, kw, frag):
    assert _varlen(L, **kw) == mf.MF_ERR_INVALID
    assert frag in _last(L)


def test_retrieve_varlen_empty_batch_launches_nothing(L):
    # R = 0 block rows: valid, nothing to do (no GPU work is queued)
    assert _varlen(L, R=0, nnzb=0, col_idx=None, vals=None) == mf.MF_OK


# ---- several receivers ----------------------------------------------------------

def _multi(L, n=2, **kw):
    import ctypes
    a = dict(row_ptr=FAKE, col_idx=FAKE, vals=FAKE, nnzb=5, dt=2, H_s=40, N=8192, B=64,
             W=[FAKE, FAKE + 4096], H_r=[32, 16], V=[FAKE, FAKE + 8192], H_kv=[8, 8], d=128,
             ldV=[1024, 1024], O=[FAKE, FAKE + 16384], ldO=[4096, 2048])
    a.update(kw)
    arr = lambda t, xs: None if xs is None else (t * len(xs))(*xs)
    return L.mf_retrieve_fused_multi(a["row_ptr"], a["col_idx"], a["vals"], a["nnzb"], a["dt"],
                                     a["H_s"], a["N"], a["B"], n,
                                     arr(ctypes.c_void_p, a["W"]), arr(ctypes.c_int, a["H_r"]),
                                     arr(ctypes.c_void_p, a["V"]), arr(ctypes.c_int, a["H_kv"]),
                                     a["d"], arr(ctypes.c_int64, a["ldV"]),
                                     arr(ctypes.c_void_p, a["O"]), arr(ctypes.c_int64, a["ldO"]),
                                     None)


@pytest.mark.parametrize("n,kw,frag", [
    (0, {}, "n_recv"), (5, {}, "n_recv"), (2, dict(W=None), "null receiver array"),
    (2, dict(ldO=None), "null receiver array"), (2, dict(row_ptr=None), "null pointer"),
    (2, dict(nnzb=-1), "nnzb"), (2, dict(vals=None), "null col_idx/vals"),
    (2, dict(H_r=[32, 30]), "receiver 1"), (2, dict(H_kv=[8, 0]), "multiple of H_kv"),
    (2, dict(ldV=[1024, 100]), "ldV"), (2, dict(O=[FAKE, FAKE]), "shared"),
    (2, dict(V=[FAKE, None]), "null pointer"), (2, dict(d=96), "d must"), (2, dict(B=24), "B must"),
])
def test_retrieve_multi_rejects(L, n, kw, frag):
    assert _multi(L, n, **kw) == mf.MF_ERR_INVALID
    assert frag in _last(L)


# ---- row-streaming block mass ----------------------------------------------------

def test_block_mass_ws_size_and_rejects(L):
    assert L.mf_block_mass_ws_bytes(40, 8192, 64) == 40 * 128 * 129 // 2 * 4
    assert L.mf_block_mass_ws_bytes(0, 8192, 64) == 0
    args = (FAKE, 2, 40, 8192, 64, FAKE)
    need = L.mf_block_mass_ws_bytes(40, 8192, 64)
    assert L.mf_block_mass_ws(*args, None, need, None) == mf.MF_ERR_INVALID
    assert "null" in _last(L)
    assert L.mf_block_mass_ws(*args, FAKE, need - 1, None) == mf.MF_ERR_INVALID
    assert "workspace" in _last(L)
    assert L.mf_block_mass_ws(FAKE, 2, 40, 8192, 48, FAKE, FAKE, need, None) == mf.MF_ERR_INVALID


# ---- the header as plain C ----------------------------------------------------

C_CALLER = r"""
#include <stdio.h>
#include <string.h>
#include "mapflow.h"
int main(void) {
  if (mf_abi_version() != MF_ABI_VERSION) return 1;
  if (strncmp(mf_status_string(MF_ERR_INVALID), "MF_ERR_INVALID", 14) != 0) return 2;
  /* an argument error is reported, not thrown: N = 0 */
  if (mf_block_mass((const void*)16, MF_BF16, 4, 0, 64, (float*)16, NULL) != MF_ERR_INVALID) return 3;
  if (strlen(mf_last_error()) == 0) return 4;
  printf("ok\n");
  return 0;
}
"""


def test_header_is_c_and_a_c_program_links_and_runs(tmp_path):
    # the boundary is a C ABI: the header compiles as pedantic C99, and a C
    # caller links against the library and gets statuses back (no GPU call)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    inc = os.path.join(root, "include")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                    "-x", "c", os.path.join(inc, "mapflow.h")], check=True)
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    libdir = os.path.dirname(mf.lib_path())
    exe = tmp_path / "caller"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", inc, str(src), "-L", libdir,
                    "-lmapflow", "-o", str(exe)], check=True)
    env = dict(os.environ, LD_LIBRARY_PATH=libdir + os.pathsep + os.environ.get("LD_LIBRARY_PATH", ""))
    out = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", (out.returncode, out.stdout, out.stderr)


def _bsr_args(torch, T=4, nnzb=6, H_s=3, B=16, cap=None):
    cap = nnzb if cap is None else cap
    rp = torch.zeros(T + 1, dtype=torch.int32)
    ci = torch.zeros(cap, dtype=torch.int32)
    vals = torch.zeros(cap, H_s, B, B, dtype=torch.float16)
    W = torch.zeros(2, H_s)
    V = torch.zeros(T * B, 1, 64, dtype=torch.float16)
    return rp, ci, vals, W, V


@pytest.mark.parametrize("case,frag", [
    ("stale_nnzb", "exceeds the"), ("short_col_idx", "col_idx has"), ("int64_row_ptr", "row_ptr must be"),
    ("short_row_ptr", "row_ptr"), ("strided_vals", "vals must be"), ("negative_nnzb", "nnzb < 0"),
    ("tile_size", "vals tiles"),
])
def test_binding_checks_bsr_before_launch(case, frag):
    """The binding refuses a BSR state whose nnzb, index arrays or tiles do not
    match, before anything reaches the device (host tensors: a check that
    passed would then fail on 'tensors must be on the GPU')."""
    import torch
    rp, ci, vals, W, V = _bsr_args(torch)
    nnzb, N, B = 6, 64, 16
    if case == "stale_nnzb":
        nnzb = 7
        ci = torch.zeros(7, dtype=torch.int32)
    elif case == "short_col_idx":
        ci = ci[:5]
    elif case == "int64_row_ptr":
        rp = rp.long()
    elif case == "short_row_ptr":
        rp = rp[:4]
    elif case == "strided_vals":
        vals = torch.zeros(6, 3, 16, 32, dtype=torch.float16)[..., ::2]
    elif case == "negative_nnzb":
        nnzb = -1
    elif case == "tile_size":
        B = 32
        N = 128
    with pytest.raises(mf.MapflowError, match=frag):
        mf.retrieve_fused(rp, ci, vals, nnzb, W, V, N, B)


def test_binding_checks_varlen_tables():
    import torch
    rp, ci, vals, W, V = _bsr_args(torch)
    cu = torch.tensor([0, 64], dtype=torch.int32)
    cr = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(mf.MapflowError, match="block_table has"):
        mf.retrieve_fused_varlen(cu, cr, rp, ci, vals, 6, W, V, 16,
                                 block_table=torch.zeros(5, dtype=torch.int32))
    with pytest.raises(mf.MapflowError, match="exceeds the"):
        mf.retrieve_fused_varlen(cu, cr, rp, ci, vals[:5], 6, W, V, 16)
    with pytest.raises(mf.MapflowError, match="R = 9"):
        mf.retrieve_fused_varlen(cu, cr, rp, ci, vals, 6, W, V, 16, R=9)
    # a pool smaller than nnzb is fine with a table (pages index the pool)
    with pytest.raises(mf.MapflowError, match="on the GPU"):
        mf.retrieve_fused_varlen(cu, cr, rp, ci, vals[:2], 6, W, V, 16,
                                 block_table=torch.zeros(6, dtype=torch.int32))
    with pytest.raises(mf.MapflowError, match="on the GPU"):
        mf.retrieve_fused(rp, ci, vals, 6, W, V, 64, 16)


def test_noalloc_rejects_before_any_launch(L):
    """Argument checks of mf_topp_select_bsr_noalloc run on the host: more block
    rows than its fixed scratch holds is MF_ERR_UNSUPPORTED, bad arguments are
    MF_ERR_INVALID, and none of them touches the GPU."""
    fake = 1 << 40
    f = L.mf_topp_select_bsr_noalloc
    assert f(fake, fake, 2, 40, 1025 * 64, 64, ctypes.c_float(0.9), fake, fake, fake, 10, None) == 2
    assert "1024" in _last(L)
    assert f(fake, fake, 2, 40, 1024 * 64, 64, ctypes.c_float(1.5), fake, fake, fake, 10, None) == 1
    assert f(None, fake, 2, 40, 4096, 64, ctypes.c_float(0.9), fake, fake, fake, 10, None) == 1
    assert f(fake, fake, 2, 40, 4096, 64, ctypes.c_float(0.9), fake, None, None, 10, None) == 1
    assert f(fake, fake, 2, 40, 4096, 64, ctypes.c_float(0.9), fake, fake, fake, -1, None) == 1
    assert f(fake, fake, 9, 40, 4096, 64, ctypes.c_float(0.9), fake, fake, fake, 10, None) == 1
