"""Python binding of libmapflow (argument marshalling only).

Every function takes torch tensors that already live on the GPU, passes their
device pointers, sizes and the current HIP stream to the C boundary declared in
include/mapflow.h, and turns a non-OK status into an exception.  No arithmetic
of the method runs here: block mass, Top-p selection, BSR build and the fused
retrieval all run in the library's HIP kernels.  If the library cannot be
loaded the functions raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import torch

_LIB_PATH = Path(__file__).resolve().parent / "libmapflow.so"

MF_OK, MF_ERR_INVALID, MF_ERR_UNSUPPORTED, MF_ERR_CAPACITY, MF_ERR_HIP = range(5)
MF_F32, MF_F16, MF_BF16 = 0, 1, 2

_DTYPE_CODE = {torch.float32: MF_F32, torch.float16: MF_F16, torch.bfloat16: MF_BF16}

EXPORTED = ("mf_abi_version", "mf_status_string", "mf_last_error", "mf_block_mass",
            "mf_block_mass_ws_bytes", "mf_block_mass_ws",
            "mf_topp_workspace_bytes", "mf_topp_select_bsr", "mf_topp_select_bsr_noalloc", "mf_row_lse",
            "mf_block_mass_qk_workspace_bytes", "mf_block_mass_qk",
            "mf_lse_block_mass_qk_workspace_bytes", "mf_lse_block_mass_qk", "mf_topp_select_bsr_qk",
            "mf_retrieve_workspace_bytes", "mf_retrieve_split_workspace_bytes", "mf_retrieve_kernel",
            "mf_retrieve_fused",
            "mf_retrieve_fused_multi", "mf_retrieve_fused_varlen", "mf_prefix_hashes",
            "mf_bm_create", "mf_bm_destroy", "mf_bm_lookup", "mf_bm_release", "mf_bm_insert",
            "mf_bm_stats", "mf_pool_store")


class MapflowError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class CapacityError(MapflowError):
    def __init__(self, status: int, msg: str, nnzb: int):
        super().__init__(status, msg)
        self.nnzb = nnzb


_lib = None


def lib_path() -> Path:
    return Path(os.environ.get("MAPFLOW_LIB", _LIB_PATH))


def load() -> ctypes.CDLL:
    """Loads libmapflow.so (built by cross_model_sparse_amd.build) once."""
    global _lib
    if _lib is not None:
        return _lib
    p = lib_path()
    if not p.exists():
        raise RuntimeError(f"libmapflow not built: {p} is missing "
                           "(run python -m cross_model_sparse_amd.build)")
    L = ctypes.CDLL(str(p))
    c_int, c_i64, c_sz, c_vp, c_f = (ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                                     ctypes.c_void_p, ctypes.c_float)
    L.mf_abi_version.restype = c_int
    L.mf_abi_version.argtypes = []
    L.mf_status_string.restype = ctypes.c_char_p
    L.mf_status_string.argtypes = [c_int]
    L.mf_last_error.restype = ctypes.c_char_p
    L.mf_last_error.argtypes = []
    L.mf_block_mass.restype = c_int
    L.mf_block_mass.argtypes = [c_vp, c_int, c_int, c_int, c_int, c_vp, c_vp]
    L.mf_topp_workspace_bytes.restype = c_sz
    L.mf_topp_workspace_bytes.argtypes = [c_int, c_int]
    L.mf_topp_select_bsr.restype = c_int
    L.mf_topp_select_bsr.argtypes = [c_vp, c_vp, c_int, c_int, c_int, c_int, c_f, c_vp,
                                     c_vp, c_vp, c_i64, ctypes.POINTER(c_i64), c_vp,
                                     c_sz, c_vp]
    L.mf_topp_select_bsr_noalloc.restype = c_int
    L.mf_topp_select_bsr_noalloc.argtypes = [c_vp, c_vp, c_int, c_int, c_int, c_int, c_f, c_vp,
                                             c_vp, c_vp, c_i64, c_vp]
    L.mf_row_lse.restype = c_int
    L.mf_row_lse.argtypes = [c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_vp, c_vp, c_vp]
    L.mf_block_mass_qk_workspace_bytes.restype = c_sz
    L.mf_block_mass_qk_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.mf_block_mass_qk.restype = c_int
    L.mf_block_mass_qk.argtypes = [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int,
                                   c_int, c_vp, c_vp, c_sz, c_vp]
    L.mf_lse_block_mass_qk_workspace_bytes.restype = c_sz
    L.mf_lse_block_mass_qk_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.mf_lse_block_mass_qk.restype = c_int
    L.mf_lse_block_mass_qk.argtypes = [c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                       c_vp, c_vp, c_vp, c_sz, c_vp]
    L.mf_topp_select_bsr_qk.restype = c_int
    L.mf_topp_select_bsr_qk.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                        c_int, c_int, c_f, c_vp, c_vp, c_vp, c_i64,
                                        ctypes.POINTER(c_i64), c_vp, c_sz, c_vp]
    L.mf_retrieve_workspace_bytes.restype = c_sz
    L.mf_retrieve_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
    L.mf_retrieve_split_workspace_bytes.restype = c_sz
    L.mf_retrieve_split_workspace_bytes.argtypes = [c_i64, c_int, c_int, c_int, c_int, c_int, c_int, c_int]
    L.mf_retrieve_kernel.restype = c_int
    L.mf_retrieve_kernel.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_vp,
                                     c_vp, c_i64, c_vp, c_i64]
    L.mf_retrieve_fused.restype = c_int
    L.mf_retrieve_fused.argtypes = [c_vp, c_vp, c_vp, c_i64, c_int, c_int, c_int, c_int,
                                    c_vp, c_int, c_vp, c_int, c_int, c_i64, c_vp, c_i64,
                                    c_vp, c_sz, c_vp]
    L.mf_retrieve_fused_multi.restype = c_int
    L.mf_retrieve_fused_multi.argtypes = [c_vp, c_vp, c_vp, c_i64, c_int, c_int, c_int, c_int,
                                          c_int, c_vp, c_vp, c_vp, c_vp, c_int, c_vp, c_vp, c_vp,
                                          c_vp]
    c_u64 = ctypes.c_uint64
    L.mf_prefix_hashes.restype = c_int
    L.mf_prefix_hashes.argtypes = [c_vp, c_i64, c_int, c_u64, c_vp]
    L.mf_bm_create.restype = c_vp
    L.mf_bm_create.argtypes = [c_int, c_int, c_i64, c_u64]
    L.mf_bm_destroy.restype = None
    L.mf_bm_destroy.argtypes = [c_vp]
    L.mf_bm_lookup.restype = c_int
    L.mf_bm_lookup.argtypes = [c_vp, c_int, c_vp, c_i64, c_int, c_vp, c_vp, c_vp, c_vp, c_i64]
    L.mf_bm_release.restype = c_int
    L.mf_bm_release.argtypes = [c_vp, c_int, c_vp, c_i64, c_int]
    L.mf_bm_insert.restype = c_int
    L.mf_bm_insert.argtypes = [c_vp, c_int, c_vp, c_i64, c_int, c_int, c_vp, c_vp, c_vp]
    L.mf_bm_stats.restype = c_int
    L.mf_bm_stats.argtypes = [c_vp, c_vp]
    L.mf_pool_store.restype = c_int
    L.mf_pool_store.argtypes = [c_vp, c_i64, c_vp, c_vp, c_i64, c_int, c_int, c_int, c_vp]
    L.mf_block_mass_ws_bytes.restype = c_sz
    L.mf_block_mass_ws_bytes.argtypes = [c_int, c_int, c_int]
    L.mf_block_mass_ws.restype = c_int
    L.mf_block_mass_ws.argtypes = [c_vp, c_int, c_int, c_int, c_int, c_vp, c_vp, c_sz, c_vp]
    L.mf_retrieve_fused_varlen.restype = c_int
    L.mf_retrieve_fused_varlen.argtypes = [c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                           c_i64, c_i64, c_int, c_int, c_int, c_vp, c_int,
                                           c_vp, c_int, c_int, c_i64, c_vp, c_i64, c_vp]
    _lib = L
    return L


def _check(st: int, nnzb: int | None = None) -> None:
    if st == MF_OK:
        return
    L = load()
    msg = L.mf_last_error().decode() or L.mf_status_string(st).decode()
    if st == MF_ERR_CAPACITY:
        raise CapacityError(st, msg, nnzb if nnzb is not None else -1)
    raise MapflowError(st, msg)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dcode(t: torch.Tensor) -> int:
    try:
        return _DTYPE_CODE[t.dtype]
    except KeyError:
        raise MapflowError(MF_ERR_INVALID, f"unsupported dtype {t.dtype}") from None


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise MapflowError(MF_ERR_INVALID, "tensors must be on the GPU")


def _check_index(t: torch.Tensor, name: str, min_len: int) -> None:
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise MapflowError(MF_ERR_INVALID, f"{name} must be a contiguous int32 tensor")
    if t.numel() < min_len:
        raise MapflowError(MF_ERR_INVALID, f"{name} has {t.numel()} entries, needs >= {min_len}")


def _check_bsr(row_ptr: torch.Tensor, col_idx: torch.Tensor, vals: torch.Tensor, nnzb: int,
               rows: int | None, pool: bool = False) -> None:
    """Host-side checks of a BSR state before the kernels see it: nnzb bounds
    every index the kernels read, so it must fit col_idx and (without a block
    table) vals; row_ptr has rows + 1 entries (rows None: any length)."""
    nnzb = int(nnzb)
    if nnzb < 0:
        raise MapflowError(MF_ERR_INVALID, "nnzb < 0")
    _check_index(row_ptr, "row_ptr", 1 if rows is None else rows + 1)
    if rows is not None and row_ptr.numel() != rows + 1:
        raise MapflowError(MF_ERR_INVALID, f"row_ptr must have {rows + 1} entries (got {row_ptr.numel()})")
    _check_index(col_idx, "col_idx", nnzb)
    if vals.dim() != 4 or vals.shape[2] != vals.shape[3] or not vals.is_contiguous():
        raise MapflowError(MF_ERR_INVALID, "vals must be a contiguous [nnzb][H_s][B][B] tensor")
    if not pool and vals.shape[0] < nnzb:
        raise MapflowError(MF_ERR_INVALID, f"nnzb = {nnzb} exceeds the {vals.shape[0]} tiles of vals")


def abi_version() -> int:
    return load().mf_abi_version()


def topp_workspace_bytes(N: int, B: int) -> int:
    return int(load().mf_topp_workspace_bytes(N, B))


def retrieve_workspace_bytes(N: int, B: int, H_kv: int, d: int, dtype: torch.dtype) -> int:
    return int(load().mf_retrieve_workspace_bytes(N, B, H_kv, d, _DTYPE_CODE[dtype]))


def retrieve_split_workspace_bytes(nnzb: int, dtype: torch.dtype, H_s: int, N: int, B: int,
                                   H_r: int, H_kv: int, d: int) -> int:
    """Workspace bytes that let retrieve_fused split long block rows (0: no split)."""
    return int(load().mf_retrieve_split_workspace_bytes(int(nnzb), _DTYPE_CODE[dtype], H_s, N, B,
                                                        H_r, H_kv, d))


def block_mass_ws_bytes(H_s: int, N: int, B: int) -> int:
    return int(load().mf_block_mass_ws_bytes(H_s, N, B))


def block_mass(A: torch.Tensor, B: int, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mass[T][T] fp32 of a contiguous [H_s][N][N] sender map.

    With a workspace (a uint8 device tensor of at least block_mass_ws_bytes)
    the row-streaming kernels run (mf_block_mass_ws); with workspace=False the
    allocation-free column-strip scan (mf_block_mass); by default a workspace
    is allocated."""
    _need_cuda(A)
    H_s, N, N2 = A.shape
    if N2 != N or not A.is_contiguous():
        raise MapflowError(MF_ERR_INVALID, "A must be a contiguous [H_s][N][N] tensor")
    T = -(-N // B)
    if out is None:
        out = torch.empty(T, T, dtype=torch.float32, device=A.device)
    if workspace is False:
        _check(load().mf_block_mass(_ptr(A), _dcode(A), H_s, N, B, _ptr(out), _stream(stream)))
        return out
    if workspace is None:
        workspace = torch.empty(max(1, block_mass_ws_bytes(H_s, N, B)), dtype=torch.uint8,
                                device=A.device)
    _check(load().mf_block_mass_ws(_ptr(A), _dcode(A), H_s, N, B, _ptr(out), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def topp_select_bsr(mass: torch.Tensor, A: torch.Tensor, B: int, p: float,
                    cap_nnzb: int | None = None, row_ptr=None, col_idx=None, vals=None,
                    workspace=None, sync: bool = True, stream=None):
    """Top-p selection + BSR build (mf_topp_select_bsr).

    Returns (row_ptr, col_idx, vals, nnzb).  With ``cap_nnzb`` None the call
    first learns nnzb with capacity 0, then allocates exactly and runs again.
    With ``sync=False`` nothing is read back and nnzb is returned as None."""
    _need_cuda(mass, A)
    H_s, N, _ = A.shape
    T = -(-N // B)
    L = load()
    dev = A.device
    if workspace is None:
        workspace = torch.empty(topp_workspace_bytes(N, B), dtype=torch.uint8, device=dev)
    if row_ptr is None:
        row_ptr = torch.empty(T + 1, dtype=torch.int32, device=dev)
    if cap_nnzb is None:
        n = ctypes.c_int64(0)
        st = L.mf_topp_select_bsr(_ptr(mass), _ptr(A), _dcode(A), H_s, N, B, float(p),
                                  _ptr(row_ptr), None, None, 0, ctypes.byref(n),
                                  _ptr(workspace), workspace.numel(), _stream(stream))
        if st not in (MF_OK, MF_ERR_CAPACITY):
            _check(st)
        cap_nnzb = int(n.value)
    if col_idx is None:
        col_idx = torch.empty(max(cap_nnzb, 1), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((max(cap_nnzb, 1), H_s, B, B), dtype=A.dtype, device=dev)
    n = ctypes.c_int64(-1)
    st = L.mf_topp_select_bsr(_ptr(mass), _ptr(A), _dcode(A), H_s, N, B, float(p),
                              _ptr(row_ptr), _ptr(col_idx), _ptr(vals), int(cap_nnzb),
                              ctypes.byref(n) if sync else None, _ptr(workspace),
                              workspace.numel(), _stream(stream))
    _check(st, int(n.value))
    nnzb = int(n.value) if sync else None
    return row_ptr, col_idx, vals, nnzb


def topp_select_bsr_noalloc(mass: torch.Tensor, A: torch.Tensor, B: int, p: float,
                            row_ptr: torch.Tensor, col_idx: torch.Tensor, vals: torch.Tensor,
                            cap_nnzb: int, stream=None) -> None:
    """Top-p selection and BSR build into the caller's buffers without any
    allocation (mf_topp_select_bsr_noalloc: fixed library scratch, T <= 1024,
    no synchronisation; nnzb is row_ptr[T]).  Calls that overlap on one GPU
    share the scratch and must not be issued."""
    H_s, N, N2 = A.shape
    if N2 != N or not A.is_contiguous():
        raise MapflowError(MF_ERR_INVALID, "A must be a contiguous [H_s][N][N] tensor")
    T = -(-N // B)
    _check_index(row_ptr, "row_ptr", T + 1)
    _check_index(col_idx, "col_idx", int(cap_nnzb))
    if vals.dtype != A.dtype or not vals.is_contiguous() or vals.shape[0] < cap_nnzb:
        raise MapflowError(MF_ERR_INVALID, "vals must be a contiguous [cap][H_s][B][B] tensor of A's dtype")
    _need_cuda(mass, A, row_ptr, col_idx, vals)
    _check(load().mf_topp_select_bsr_noalloc(_ptr(mass), _ptr(A), _dcode(A), H_s, N, B, float(p),
                                             _ptr(row_ptr), _ptr(col_idx), _ptr(vals), int(cap_nnzb),
                                             _stream(stream)))


def retrieve_kernel(vals: torch.Tensor, V: torch.Tensor, W: torch.Tensor, N: int, B: int,
                    out: torch.Tensor | None = None) -> str:
    """'mfma' or 'plain': the kernel retrieve_fused runs for these tensors
    (mf_retrieve_kernel; host-side decision, no GPU work)."""
    H_s, H_r, H_kv, d = vals.shape[1], W.shape[0], V.shape[1], V.shape[2]
    if out is None:
        o_ptr, ldO = 256, H_r * d           # a fresh allocation is 256-byte aligned
    else:
        o_ptr, ldO = out.data_ptr(), out.stride(0)
    r = load().mf_retrieve_kernel(_DTYPE_CODE[V.dtype], H_s, N, B, H_r, H_kv, d,
                                  vals.data_ptr(), V.data_ptr(), V.stride(0), o_ptr, ldO)
    if r < 0:
        _check(-r)
    return "mfma" if r == 1 else "plain"


def retrieve_fused(row_ptr: torch.Tensor, col_idx: torch.Tensor, vals: torch.Tensor,
                   nnzb: int, W: torch.Tensor, V: torch.Tensor, N: int, B: int,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """O[N][H_r][d] = fused head-mapped BSR retrieval (mf_retrieve_fused).

    V may be a [N][H_kv][d] tensor or a row-strided view whose last two dims
    are contiguous (e.g. a slice of a fused QKV projection)."""
    _check_bsr(row_ptr, col_idx, vals, nnzb, -(-N // B))
    if vals.shape[2] != B:
        raise MapflowError(MF_ERR_INVALID, f"vals tiles are {vals.shape[2]}x{vals.shape[3]}, B = {B}")
    _need_cuda(row_ptr, col_idx, vals, W, V)
    H_s = vals.shape[1]
    H_r = W.shape[0]
    if W.dtype != torch.float32 or not W.is_contiguous() or W.shape[1] != H_s:
        raise MapflowError(MF_ERR_INVALID, "W must be a contiguous fp32 [H_r][H_s] tensor")
    if V.dim() != 3 or V.stride(2) != 1 or V.stride(1) != V.shape[2]:
        raise MapflowError(MF_ERR_INVALID, "V must be [N][H_kv][d] with contiguous rows")
    if V.dtype != vals.dtype:
        raise MapflowError(MF_ERR_INVALID, "V and vals must share a dtype")
    H_kv, d = V.shape[1], V.shape[2]
    if out is None:
        out = torch.empty(N, H_r, d, dtype=V.dtype, device=V.device)
    if out.dim() != 3 or out.stride(2) != 1 or out.stride(1) != d:
        raise MapflowError(MF_ERR_INVALID, "out must be [N][H_r][d] with contiguous rows")
    need = retrieve_workspace_bytes(N, B, H_kv, d, V.dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=V.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().mf_retrieve_fused(_ptr(row_ptr), _ptr(col_idx), _ptr(vals), int(nnzb),
                                    _dcode(V), H_s, N, B, _ptr(W), H_r, _ptr(V), H_kv, d,
                                    V.stride(0), _ptr(out), out.stride(0), _ptr(workspace),
                                    ws_bytes, _stream(stream)))
    return out


def retrieve_fused_multi(row_ptr: torch.Tensor, col_idx: torch.Tensor, vals: torch.Tensor,
                         nnzb: int, receivers, N: int, B: int, outs=None, stream=None) -> list:
    """One sender BSR state feeding several receivers (mf_retrieve_fused_multi).
    receivers: a sequence of (W [H_r][H_s] fp32, V [N][H_kv][d]) pairs; returns
    the list of outputs O_i [N][H_r_i][d] (or fills `outs`)."""
    n = len(receivers)
    _check_bsr(row_ptr, col_idx, vals, nnzb, -(-N // B))
    _need_cuda(row_ptr, col_idx, vals, *[t for rv in receivers for t in rv])
    H_s = vals.shape[1]
    if outs is None:
        outs = [torch.empty(N, W.shape[0], V.shape[2], dtype=V.dtype, device=V.device)
                for W, V in receivers]
    for (W, V), O in zip(receivers, outs):
        if W.dtype != torch.float32 or not W.is_contiguous() or W.shape[1] != H_s:
            raise MapflowError(MF_ERR_INVALID, "W must be a contiguous fp32 [H_r][H_s] tensor")
        if V.dim() != 3 or V.stride(2) != 1 or V.stride(1) != V.shape[2] or V.dtype != vals.dtype:
            raise MapflowError(MF_ERR_INVALID, "V must be [N][H_kv][d] with contiguous rows, dtype of vals")
        if O.dim() != 3 or O.stride(2) != 1 or O.stride(1) != O.shape[2]:
            raise MapflowError(MF_ERR_INVALID, "out must be [N][H_r][d] with contiguous rows")
    d = receivers[0][1].shape[2]
    arr = lambda ctype, xs: (ctype * n)(*xs)
    _check(load().mf_retrieve_fused_multi(
        _ptr(row_ptr), _ptr(col_idx), _ptr(vals), int(nnzb), _dcode(vals), H_s, N, B, n,
        arr(ctypes.c_void_p, [W.data_ptr() for W, _ in receivers]),
        arr(ctypes.c_int, [W.shape[0] for W, _ in receivers]),
        arr(ctypes.c_void_p, [V.data_ptr() for _, V in receivers]),
        arr(ctypes.c_int, [V.shape[1] for _, V in receivers]), d,
        arr(ctypes.c_int64, [V.stride(0) for _, V in receivers]),
        arr(ctypes.c_void_p, [O.data_ptr() for O in outs]),
        arr(ctypes.c_int64, [O.stride(0) for O in outs]), _stream(stream)))
    return outs


def retrieve_fused_varlen(cu_seqlens: torch.Tensor, cu_rows: torch.Tensor,
                          row_ptr: torch.Tensor, col_idx: torch.Tensor, vals: torch.Tensor,
                          nnzb: int, W: torch.Tensor, V: torch.Tensor, B: int,
                          block_table: torch.Tensor | None = None, R: int | None = None,
                          out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """O[total][H_r][d] for a packed batch of sequences in one launch
    (mf_retrieve_fused_varlen).  cu_seqlens / cu_rows are device int32 [S+1];
    row_ptr covers the R = cu_rows[S] block rows of all sequences; col_idx is
    local to each sequence; vals is the tile pool [n_pages][H_s][B][B], indexed
    through block_table when given.  R, when not given, is len(row_ptr) - 1."""
    for t, name in ((cu_seqlens, "cu_seqlens"), (cu_rows, "cu_rows")):
        _check_index(t, name, 1)
    _check_bsr(row_ptr, col_idx, vals, nnzb, None, pool=block_table is not None)
    if block_table is not None:
        _check_index(block_table, "block_table", int(nnzb))
    if cu_rows.numel() != cu_seqlens.numel():
        raise MapflowError(MF_ERR_INVALID, "cu_rows and cu_seqlens must both have S+1 entries")
    S = cu_seqlens.numel() - 1
    R = row_ptr.numel() - 1 if R is None else int(R)
    if R < 0 or row_ptr.numel() < R + 1:
        raise MapflowError(MF_ERR_INVALID, f"row_ptr has {row_ptr.numel()} entries, R = {R} needs R + 1")
    _need_cuda(cu_seqlens, cu_rows, row_ptr, col_idx, vals, W, V)
    H_s = vals.shape[1]
    H_r = W.shape[0]
    if W.dtype != torch.float32 or not W.is_contiguous() or W.shape[1] != H_s:
        raise MapflowError(MF_ERR_INVALID, "W must be a contiguous fp32 [H_r][H_s] tensor")
    if V.dim() != 3 or V.stride(2) != 1 or V.stride(1) != V.shape[2]:
        raise MapflowError(MF_ERR_INVALID, "V must be [total][H_kv][d] with contiguous rows")
    if V.dtype != vals.dtype:
        raise MapflowError(MF_ERR_INVALID, "V and vals must share a dtype")
    H_kv, d = V.shape[1], V.shape[2]
    if out is None:
        out = torch.empty(V.shape[0], H_r, d, dtype=V.dtype, device=V.device)
    if out.dim() != 3 or out.stride(2) != 1 or out.stride(1) != d:
        raise MapflowError(MF_ERR_INVALID, "out must be [total][H_r][d] with contiguous rows")
    _check(load().mf_retrieve_fused_varlen(
        S, R, _ptr(cu_seqlens), _ptr(cu_rows), _ptr(row_ptr), _ptr(col_idx), _ptr(block_table),
        _ptr(vals), vals.shape[0], int(nnzb), _dcode(V), H_s, B, _ptr(W), H_r, _ptr(V), H_kv, d,
        V.stride(0), _ptr(out), out.stride(0), _stream(stream)))
    return out


def _qk_shapes(Q: torch.Tensor, K: torch.Tensor, scale: torch.Tensor):
    _need_cuda(Q, K, scale)
    if Q.dim() != 3 or K.dim() != 3 or not Q.is_contiguous() or not K.is_contiguous():
        raise MapflowError(MF_ERR_INVALID, "Q and K must be contiguous [H][N][d] tensors")
    if K.dtype != Q.dtype or K.shape[1:] != Q.shape[1:]:
        raise MapflowError(MF_ERR_INVALID, "K must match Q in dtype, N and d")
    if scale.dtype != torch.float32 or scale.numel() != Q.shape[0] or not scale.is_contiguous():
        raise MapflowError(MF_ERR_INVALID, "scale must be a contiguous float32 [H_s] tensor")
    return Q.shape[0], K.shape[0], Q.shape[1], Q.shape[2]


def row_lse(Q: torch.Tensor, K: torch.Tensor, scale: torch.Tensor,
            out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """lse[H_s][N] fp32: per-row log-sum-exp of the causal scores (mf_row_lse)."""
    H_s, H_ks, N, d = _qk_shapes(Q, K, scale)
    if out is None:
        out = torch.empty(H_s, N, dtype=torch.float32, device=Q.device)
    _check(load().mf_row_lse(_ptr(Q), _ptr(K), _dcode(Q), H_s, H_ks, N, d, _ptr(scale),
                             _ptr(out), _stream(stream)))
    return out


def block_mass_qk_workspace_bytes(H_s: int, N: int, B: int) -> int:
    return int(load().mf_block_mass_qk_workspace_bytes(H_s, N, B))


def block_mass_qk(Q: torch.Tensor, K: torch.Tensor, scale: torch.Tensor, lse: torch.Tensor,
                  B: int, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """mass[T][T] fp32 from Q, K, scale and lse, without a dense map (mf_block_mass_qk)."""
    H_s, H_ks, N, d = _qk_shapes(Q, K, scale)
    _need_cuda(lse)
    T = -(-N // B)
    if out is None:
        out = torch.empty(T, T, dtype=torch.float32, device=Q.device)
    if workspace is None:
        workspace = torch.empty(max(1, block_mass_qk_workspace_bytes(H_s, N, B)),
                                dtype=torch.uint8, device=Q.device)
    _check(load().mf_block_mass_qk(_ptr(Q), _ptr(K), _ptr(scale), _ptr(lse), _dcode(Q), H_s,
                                   H_ks, N, d, B, _ptr(out), _ptr(workspace), workspace.numel(),
                                   _stream(stream)))
    return out


def lse_block_mass_qk_workspace_bytes(H_s: int, N: int, B: int) -> int:
    return int(load().mf_lse_block_mass_qk_workspace_bytes(H_s, N, B))


def lse_block_mass_qk(Q: torch.Tensor, K: torch.Tensor, scale: torch.Tensor, B: int,
                      lse: torch.Tensor | None = None, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None):
    """(lse[H_s][N], mass[T][T]) fp32 in one pass over the scores
    (mf_lse_block_mass_qk)."""
    H_s, H_ks, N, d = _qk_shapes(Q, K, scale)
    T = -(-N // B)
    if lse is None:
        lse = torch.empty(H_s, N, dtype=torch.float32, device=Q.device)
    if out is None:
        out = torch.empty(T, T, dtype=torch.float32, device=Q.device)
    if workspace is None:
        workspace = torch.empty(max(1, lse_block_mass_qk_workspace_bytes(H_s, N, B)),
                                dtype=torch.uint8, device=Q.device)
    _check(load().mf_lse_block_mass_qk(_ptr(Q), _ptr(K), _ptr(scale), _dcode(Q), H_s, H_ks, N, d,
                                       B, _ptr(lse), _ptr(out), _ptr(workspace),
                                       workspace.numel(), _stream(stream)))
    return lse, out


def topp_select_bsr_qk(mass: torch.Tensor, Q: torch.Tensor, K: torch.Tensor,
                       scale: torch.Tensor, lse: torch.Tensor, B: int, p: float,
                       cap_nnzb: int | None = None, row_ptr=None, col_idx=None, vals=None,
                       workspace=None, sync: bool = True, stream=None):
    """Top-p selection + BSR build with the kept tiles recomputed from Q, K and
    lse (mf_topp_select_bsr_qk).  Same returns and capacity handling as
    topp_select_bsr."""
    H_s, H_ks, N, d = _qk_shapes(Q, K, scale)
    _need_cuda(mass, lse)
    T = -(-N // B)
    L = load()
    dev = Q.device
    if workspace is None:
        workspace = torch.empty(topp_workspace_bytes(N, B), dtype=torch.uint8, device=dev)
    if row_ptr is None:
        row_ptr = torch.empty(T + 1, dtype=torch.int32, device=dev)
    args = (_ptr(mass), _ptr(Q), _ptr(K), _ptr(scale), _ptr(lse), _dcode(Q), H_s, H_ks, N, d,
            B, float(p))
    if cap_nnzb is None:
        n = ctypes.c_int64(0)
        st = L.mf_topp_select_bsr_qk(*args, _ptr(row_ptr), None, None, 0, ctypes.byref(n),
                                     _ptr(workspace), workspace.numel(), _stream(stream))
        if st not in (MF_OK, MF_ERR_CAPACITY):
            _check(st)
        cap_nnzb = int(n.value)
    if col_idx is None:
        col_idx = torch.empty(max(cap_nnzb, 1), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((max(cap_nnzb, 1), H_s, B, B), dtype=Q.dtype, device=dev)
    n = ctypes.c_int64(-1)
    st = L.mf_topp_select_bsr_qk(*args, _ptr(row_ptr), _ptr(col_idx), _ptr(vals), int(cap_nnzb),
                                 ctypes.byref(n) if sync else None, _ptr(workspace),
                                 workspace.numel(), _stream(stream))
    _check(st, int(n.value))
    nnzb = int(n.value) if sync else None
    return row_ptr, col_idx, vals, nnzb


def compress_qk(Q: torch.Tensor, K: torch.Tensor, scale: torch.Tensor, B: int, p: float,
                lse: torch.Tensor | None = None, cap_nnzb: int | None = None, stream=None):
    """Compression without a dense map: (lse, mass, row_ptr, col_idx, vals, nnzb).
    Without a given lse, lse and the masses come from one pass over the scores
    (lse_block_mass_qk); with one, the masses from block_mass_qk."""
    if lse is None:
        lse, mass = lse_block_mass_qk(Q, K, scale, B, stream=stream)
    else:
        mass = block_mass_qk(Q, K, scale, lse, B, stream=stream)
    row_ptr, col_idx, vals, nnzb = topp_select_bsr_qk(mass, Q, K, scale, lse, B, p,
                                                      cap_nnzb=cap_nnzb, stream=stream)
    return lse, mass, row_ptr, col_idx, vals, nnzb


def compress(A: torch.Tensor, B: int, p: float, cap_nnzb: int | None = None, stream=None):
    """Block mass -> Top-p -> BSR on the GPU.  Returns (mass, row_ptr, col_idx, vals, nnzb)."""
    mass = block_mass(A, B, stream=stream)
    row_ptr, col_idx, vals, nnzb = topp_select_bsr(mass, A, B, p, cap_nnzb=cap_nnzb,
                                                   stream=stream)
    return mass, row_ptr, col_idx, vals, nnzb


# ---- Block Manager -----------------------------------------------------------

def _i32_host(a) -> "np.ndarray":
    import numpy as np
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def prefix_hashes(tokens, B: int, seed: int = 0):
    """uint64 prefix hashes h_1..h_n of the full B-token chunks (mf_prefix_hashes)."""
    import numpy as np
    tok = _i32_host(tokens)
    out = np.zeros(len(tok) // B, dtype=np.uint64)
    _check(load().mf_prefix_hashes(tok.ctypes.data, len(tok), B, seed, out.ctypes.data))
    return out


class BlockManager:
    """Prefix-hash index of cached BSR block rows (mf_bm_*); host bookkeeping
    for a caller-owned device tile pool of n_pages pages."""

    STATS = ("free_pages", "cached_rows", "held_rows", "hits", "misses", "evictions", "inserted")

    def __init__(self, B: int, n_layers: int, n_pages: int, seed: int = 0):
        self._L = load()
        self._m = self._L.mf_bm_create(B, n_layers, n_pages, seed)
        if not self._m:
            raise MapflowError(MF_ERR_INVALID, self._L.mf_last_error().decode())
        self.B, self.n_layers, self.n_pages = B, n_layers, n_pages

    def close(self):
        if getattr(self, "_m", None):
            self._L.mf_bm_destroy(self._m)
            self._m = None

    def __del__(self):
        self.close()

    def lookup(self, layer: int, tokens, max_rows: int | None = None, cap: int | None = None):
        """(row_ptr, col_idx, pages) numpy int32 of the longest cached prefix; the
        returned rows stay held until release()."""
        import numpy as np
        tok = _i32_host(tokens)
        n = len(tok) // self.B if max_rows is None else int(max_rows)
        if cap is None:
            cap = self.n_pages
        row_ptr = np.zeros(n + 1, dtype=np.int32)
        col = np.zeros(max(cap, 1), dtype=np.int32)
        pages = np.zeros(max(cap, 1), dtype=np.int32)
        nr = ctypes.c_int(0)
        _check(self._L.mf_bm_lookup(self._m, layer, tok.ctypes.data, len(tok), n, ctypes.byref(nr),
                                    row_ptr.ctypes.data, col.ctypes.data, pages.ctypes.data, cap))
        k = int(row_ptr[nr.value])
        return row_ptr[: nr.value + 1].copy(), col[:k].copy(), pages[:k].copy()

    def release(self, layer: int, tokens, n_rows: int):
        tok = _i32_host(tokens)
        _check(self._L.mf_bm_release(self._m, layer, tok.ctypes.data, len(tok), int(n_rows)))

    def insert(self, layer: int, tokens, row0: int, row_ptr, col_idx):
        """Caches rows row0.. (row_ptr from 0); returns the pages (numpy int32,
        -1 for rows already cached) to copy the tiles into."""
        import numpy as np
        tok, rp, ci = _i32_host(tokens), _i32_host(row_ptr), _i32_host(col_idx)
        pages = np.full(max(int(rp[-1]), 1), -1, dtype=np.int32)
        _check(self._L.mf_bm_insert(self._m, layer, tok.ctypes.data, len(tok), int(row0),
                                    len(rp) - 1, rp.ctypes.data, ci.ctypes.data if len(ci) else None,
                                    pages.ctypes.data))
        return pages[: int(rp[-1])]

    def stats(self) -> dict:
        import numpy as np
        out = np.zeros(7, dtype=np.int64)
        _check(self._L.mf_bm_stats(self._m, out.ctypes.data))
        return dict(zip(self.STATS, (int(x) for x in out)))


def pool_store(vals: torch.Tensor, pages: torch.Tensor, pool: torch.Tensor, stream=None):
    """pool[pages[k]] = vals[k] on the device (mf_pool_store); pages outside
    the pool (e.g. -1) are skipped."""
    _need_cuda(vals, pages, pool)
    if pages.dtype != torch.int32 or not pages.is_contiguous():
        raise MapflowError(MF_ERR_INVALID, "pages must be a contiguous int32 tensor")
    if vals.dtype != pool.dtype or vals.shape[1:] != pool.shape[1:]:
        raise MapflowError(MF_ERR_INVALID, "vals and pool must share dtype and tile shape")
    n = min(vals.shape[0], pages.numel())
    _check(load().mf_pool_store(_ptr(vals), n, _ptr(pages), _ptr(pool), pool.shape[0],
                                _dcode(vals), vals.shape[1], vals.shape[2], _stream(stream)))
