"""Sparse + low-rank (HSS) linear layer on AMD MI355X.

Thin Python binding of libhss.so (C ABI in include/hss.h).  The functions keep
the C names; they only marshal torch tensors (device memory) and the current
HIP stream into the C calls -- every step runs in the library's HIP kernels.

    W ~= S + U V^T,   Y = X (S + U V^T)^T

    sp = hss_split(W, "csr", frac=(5, 100), residual=True)   # stage 1 on the GPU
    A  = HSSMatrix.from_split(sp, U, V=V)                     # U: m x r, V: n x r
    Y  = hss_apply(A, X)                                      # X: b x n -> Y: b x m
"""
from __future__ import annotations

import contextlib
import ctypes
from dataclasses import dataclass, field
from typing import Optional

import torch

from ._lib import (HSS_BF16, HSS_COL16, HSS_DQ4, HSS_ERR_NONFINITE, HSS_HIER2, HSS_F32, HSS_FMT_2OF4, HSS_FMT_CSR,
                   HSS_MAX_BATCH, HSS_OK, HSS_OPT_BATCH_ROUTE, HSS_OPT_DECODE_FORCE_LOCAL, HSS_OPT_DECODE_MERGED,
                   HSS_OPT_DECODE_RPW, HSS_OPT_DECODE_WAVE_PRODUCERS,
                   HSS_OPT_DECODE_SPIN, HSS_OPT_GRAD_DS_ROUTE, HSSError, HssMatrixStruct, LIB_PATH, check, lib,
                   status_string)

__all__ = [
    "hss_version", "hss_topk_count", "hss_split_workspace_size", "hss_split", "hss_get_error",
    "hss_set_option", "hss_get_option", "option", "HSS_MAX_BATCH",
    "hss_apply_workspace_size", "hss_apply_workspace_init", "apply_workspace", "hss_apply", "hss_apply_noalloc",
    "hss_apply_group_workspace_size", "hss_apply_group",
    "hss_csr_cols_to_u16", "HSS_COL16", "HSS_DQ4", "HSS_HIER2",
    "hss_rcm_order", "hss_concentration", "hss_hier_pack", "hss_hier_pack_compact", "hss_csr_permute",
    "hss_grad", "hss_csr_transpose", "hss_gather_values", "hss_transpose", "hss_transposed_layer", "hss_backward",
    "hss_nm24_to_csr",
    "HSSMatrix", "SplitResult", "HSSError",
    "LIB_PATH", "status_string",
]

_DT = {torch.float32: HSS_F32, torch.bfloat16: HSS_BF16}
_FMT = {"csr": HSS_FMT_CSR, "2:4": HSS_FMT_2OF4, HSS_FMT_CSR: HSS_FMT_CSR, HSS_FMT_2OF4: HSS_FMT_2OF4}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("tensor must be on a GPU device")
    return t.device


def hss_version() -> int:
    return lib.hss_version()


# Diagnostic switches (hss_set_option); route names as the environment
# variables spell them.
_OPTS = {"batch_route": HSS_OPT_BATCH_ROUTE, "grad_ds_route": HSS_OPT_GRAD_DS_ROUTE,
         "decode_spin": HSS_OPT_DECODE_SPIN, "decode_merged": HSS_OPT_DECODE_MERGED,
         "decode_force_local": HSS_OPT_DECODE_FORCE_LOCAL, "decode_wave_producers": HSS_OPT_DECODE_WAVE_PRODUCERS,
         "decode_rpw": HSS_OPT_DECODE_RPW}
_OPT_WORDS = {"batch_route": {"auto": 0, "decode": 1, "spmm": 2, "densify": 3, "smfmac": 4},
              "grad_ds_route": {"auto": 0, "sparse": 1, "dense": 2}}


def hss_set_option(name: str, value) -> None:
    """Set a process-wide diagnostic switch: batch_route (auto | decode | spmm |
    densify | smfmac), grad_ds_route (auto | sparse | dense), decode_spin
    (int), decode_merged (0 | 1), decode_force_local (0 | 1)."""
    v = _OPT_WORDS.get(name, {}).get(value, value)
    check(lib.hss_set_option(_OPTS[name], int(v)), f"hss_set_option({name})")


def hss_get_option(name: str) -> int:
    return int(lib.hss_get_option(_OPTS[name]))


@contextlib.contextmanager
def option(name: str, value):
    """Scope a diagnostic switch: set on entry, the previous value restored on exit."""
    old = hss_get_option(name)
    hss_set_option(name, value)
    try:
        yield
    finally:
        check(lib.hss_set_option(_OPTS[name], old), f"hss_set_option({name})")


def hss_topk_count(m: int, n: int, num: int, den: int) -> int:
    """floor(m*n*num/den) computed exactly by the library."""
    k = lib.hss_topk_count(m, n, num, den)
    if k < 0:
        raise ValueError("invalid count arguments")
    return int(k)


def hss_split_workspace_size(fmt, dtype: int, m: int, n: int) -> int:
    out = ctypes.c_size_t(0)
    check(lib.hss_split_workspace_size(_FMT[fmt], dtype, m, n, ctypes.byref(out)), "hss_split_workspace_size")
    return int(out.value)


@dataclass
class SplitResult:
    fmt: int
    m: int
    n: int
    k: int
    row_ptr: Optional[torch.Tensor] = None    # int32 [m+1]
    col_idx: Optional[torch.Tensor] = None    # int32 [k]
    values: Optional[torch.Tensor] = None     # W dtype [k]
    nm_values: Optional[torch.Tensor] = None  # W dtype [m, n/2]
    nm_meta: Optional[torch.Tensor] = None    # int32 storage of uint32 [m, ceil(n/32)]
    residual: Optional[torch.Tensor] = None   # W dtype [m, n]
    ws: Optional[torch.Tensor] = field(default=None, repr=False)


def hss_split(W: torch.Tensor, fmt="csr", k: Optional[int] = None, frac=(5, 100),
              residual: bool = False, check_finite: bool = True) -> SplitResult:
    """Stage 1 on the GPU: magnitude top-k of W (m x n) into CSR or 2:4.

    fmt "csr": k defaults to floor(m*n*frac[0]/frac[1]).  fmt "2:4": k is m*n/2.
    check_finite synchronises and raises HSSError(HSS_ERR_NONFINITE) on NaN/Inf."""
    dev = _dev(W)
    if W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous 2-D tensor")
    dt = _dt(W)
    m, n = W.shape
    f = _FMT[fmt]
    ws_bytes = hss_split_workspace_size(f, dt, m, n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    res = torch.empty_like(W) if residual else None
    out = SplitResult(fmt=f, m=m, n=n, k=0, residual=res, ws=ws)
    if f == HSS_FMT_CSR:
        if k is None:
            k = hss_topk_count(m, n, *frac)
        out.k = int(k)
        out.row_ptr = torch.empty(m + 1, dtype=torch.int32, device=dev)
        out.col_idx = torch.empty(max(out.k, 0), dtype=torch.int32, device=dev)
        out.values = torch.empty(max(out.k, 0), dtype=W.dtype, device=dev)
        code = lib.hss_split(f, dt, m, n, _ptr(W), out.k, _ptr(out.row_ptr),
                             _ptr(out.col_idx) if out.k > 0 else None,
                             _ptr(out.values) if out.k > 0 else None, None, None, _ptr(res),
                             _ptr(ws), ws_bytes, _stream(dev))
    else:
        out.k = (m * n) // 2 if k is None else int(k)
        out.nm_values = torch.empty((m, n // 2), dtype=W.dtype, device=dev)
        out.nm_meta = torch.empty((m, (n + 31) // 32), dtype=torch.int32, device=dev)
        code = lib.hss_split(f, dt, m, n, _ptr(W), out.k, None, None, None, _ptr(out.nm_values),
                             _ptr(out.nm_meta), _ptr(res), _ptr(ws), ws_bytes, _stream(dev))
    check(code, "hss_split")
    if check_finite:
        check(hss_get_error(ws), "hss_split")
    return out


def hss_get_error(ws: torch.Tensor) -> int:
    """Synchronises the current stream and returns the split's device status code."""
    return int(lib.hss_get_error(_ptr(ws), _stream(ws.device)))


class HSSMatrix:
    """Compressed matrix S + U V^T (or S + D) in device memory; keeps its tensors alive.

    U: m x r row-major.  The factor V (n x r) is held as Vt (r x n row-major,
    i.e. V column-major), the layout the library reads.  CSR col_idx is
    int32, or 16-bit (a torch.int16 tensor holding the uint16 columns, n <=
    65536, see hss_csr_cols_to_u16) -- the matrix then carries HSS_COL16.
    dq_codes (uint8, m x n/2: the 4-bit codes of columns 2j and 2j+1 in the
    low and high nibble of byte j) with dq_levels (m x 16, the matrix dtype)
    add the quantised dense part D of the dense-and-sparse form (HSS_DQ4).
    hier_r (ranks of the 2 x 2 blocks 00, 01, 10, 11) makes the low-rank term
    the compact block form (HSS_HIER2): U m x (hier_r[0] + hier_r[1]) and
    Vt sum(hier_r) x (n - n // 2) as hss_hier_pack_compact writes them, the
    matrix in the blocks' (permuted) order."""

    def __init__(self, fmt, m, n, dtype, U=None, Vt=None, row_ptr=None, col_idx=None, values=None,
                 nnz=None, nm_values=None, nm_meta=None, dq_codes=None, dq_levels=None, hier_r=None):
        self.fmt = _FMT[fmt]
        self.flags = HSS_COL16 if (col_idx is not None and col_idx.dtype == torch.int16) else 0
        self.hier_r = None if hier_r is None else [int(v) for v in hier_r]
        if dq_codes is not None:
            assert dq_codes.dtype == torch.uint8 and dq_codes.is_contiguous() and dq_codes.numel() == m * n // 2
            assert dq_levels is not None and dq_levels.dtype == dtype and dq_levels.is_contiguous()
            assert dq_levels.numel() == m * 16
            self.flags |= HSS_DQ4
        self.dq_codes, self.dq_levels = dq_codes, dq_levels
        self.m, self.n = int(m), int(n)
        self.dtype = dtype
        self.U, self.Vt = U, Vt
        if self.hier_r is not None:
            self.flags |= HSS_HIER2
            self.r = sum(self.hier_r)
            ru = self.hier_r[0] + self.hier_r[1]
            if self.r > 0:
                assert U.shape == (self.m, ru) and Vt.shape == (self.r, self.n - self.n // 2)
        else:
            self.r = 0 if U is None else int(U.shape[1])
            if self.r > 0:
                assert U.shape == (self.m, self.r) and Vt.shape == (self.r, self.n)
        if self.r > 0:
            assert U.dtype == dtype and Vt.dtype == dtype and U.is_contiguous() and Vt.is_contiguous()
        self.row_ptr, self.col_idx, self.values = row_ptr, col_idx, values
        self.nm_values, self.nm_meta = nm_values, nm_meta
        self.nnz = int(nnz if nnz is not None else (values.numel() if values is not None else 0))
        self._ws = {}
        s = HssMatrixStruct()
        s.fmt, s.dtype = self.fmt, _DT[dtype]
        s.m, s.n, s.r, s.flags = self.m, self.n, self.r, self.flags
        s.nnz = self.nnz
        s.row_ptr, s.col_idx, s.values = _ptr(row_ptr), _ptr(col_idx), _ptr(values)
        s.nm_values, s.nm_meta = _ptr(nm_values), _ptr(nm_meta)
        s.U, s.Vt = (_ptr(U), _ptr(Vt)) if self.r > 0 else (None, None)
        s.dq_codes, s.dq_levels = _ptr(dq_codes), _ptr(dq_levels)
        if self.hier_r is not None:
            s.hier_r = (ctypes.c_int32 * 4)(*self.hier_r)
        self.struct = s

    @classmethod
    def from_split(cls, sp: SplitResult, U=None, V=None, Vt=None, dtype=None):
        if V is not None:
            Vt = V.t().contiguous()
        if dtype is None:
            dtype = (sp.values if sp.values is not None else sp.nm_values).dtype
        if sp.fmt == HSS_FMT_CSR:
            return cls("csr", sp.m, sp.n, dtype, U=U, Vt=Vt, row_ptr=sp.row_ptr,
                       col_idx=sp.col_idx, values=sp.values, nnz=sp.k)
        return cls("2:4", sp.m, sp.n, dtype, U=U, Vt=Vt, nm_values=sp.nm_values, nm_meta=sp.nm_meta)

    def with_col16(self) -> "HSSMatrix":
        """The same CSR matrix with 16-bit columns (converted on the device)."""
        if self.fmt != HSS_FMT_CSR:
            raise ValueError("16-bit columns are a CSR option")
        c16 = hss_csr_cols_to_u16(self.col_idx, self.n) if self.nnz > 0 else None
        return HSSMatrix("csr", self.m, self.n, self.dtype, U=self.U, Vt=self.Vt, row_ptr=self.row_ptr,
                         col_idx=c16 if c16 is not None else torch.zeros(0, dtype=torch.int16,
                                                                           device=self.row_ptr.device),
                         values=self.values, nnz=self.nnz, dq_codes=self.dq_codes, dq_levels=self.dq_levels,
                         hier_r=self.hier_r)

    def workspace(self, b: int, device=None) -> torch.Tensor:
        """Initialised apply workspace for batch b on the current stream.

        Cached per (device, stream, size): the decode kernel keeps state in
        its workspace from call to call, so calls that may overlap in time --
        those on different streams -- must not share one.  Calls on one
        stream are ordered and share it safely."""
        size = hss_apply_workspace_size(self, b)
        if device is None:
            held = [t for t in (self.U, self.row_ptr, self.values, self.nm_values, self.dq_codes) if t is not None]
            device = held[0].device
        dev = torch.device(device)
        key = (str(dev), _stream(dev), size)
        if key not in self._ws:
            if torch.cuda.is_current_stream_capturing():
                # its init kernel would be captured too and reset the state on
                # every replay, so that replays could take each other's T words
                raise RuntimeError("create the workspace before graph capture and pass it as ws=")
            self._ws[key] = apply_workspace(size, dev)
        return self._ws[key]


def hss_apply_workspace_init(ws: torch.Tensor) -> torch.Tensor:
    """Put an apply workspace in its initial state (a kernel on the current
    stream); call once before its first apply."""
    check(lib.hss_apply_workspace_init(_ptr(ws), ws.numel(), _stream(ws.device)), "hss_apply_workspace_init")
    return ws


def apply_workspace(size: int, device) -> torch.Tensor:
    """A new apply workspace of `size` bytes on `device`, initialised on the
    current stream.  Calls that share it must be ordered (one stream, or
    events between streams)."""
    ws = torch.empty(max(int(size), 1), dtype=torch.uint8, device=device)
    return hss_apply_workspace_init(ws)


def hss_apply_workspace_size(A: HSSMatrix, b: int) -> int:
    out = ctypes.c_size_t(0)
    check(lib.hss_apply_workspace_size(ctypes.byref(A.struct), int(b), ctypes.byref(out)),
          "hss_apply_workspace_size")
    return int(out.value)


def hss_apply(A: HSSMatrix, X: torch.Tensor, Y: Optional[torch.Tensor] = None,
              ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y (b x m) = X (b x n) (S + U V^T)^T on the current stream."""
    dev = _dev(X)
    if X.dim() != 2 or X.shape[1] != A.n or not X.is_contiguous() or X.dtype != A.dtype:
        raise ValueError("X must be a contiguous b x n tensor of the matrix dtype")
    b = X.shape[0]
    if Y is None:
        Y = torch.empty((b, A.m), dtype=A.dtype, device=dev)
    if ws is None:
        ws = A.workspace(b, dev)
    check(lib.hss_apply(ctypes.byref(A.struct), b, _ptr(X), _ptr(Y), _ptr(ws), ws.numel(),
                        _stream(dev)), "hss_apply")
    return Y


def hss_apply_noalloc(A: HSSMatrix, X: torch.Tensor, Y: torch.Tensor) -> torch.Tensor:
    """Y (b x m, preallocated) = X (b x n) (S + U V^T)^T on the current stream,
    with the library's own per-GPU scratch instead of a workspace: the call
    allocates nothing.  Calls that overlap in time on one GPU race."""
    dev = _dev(X)
    if X.dim() != 2 or X.shape[1] != A.n or not X.is_contiguous() or X.dtype != A.dtype:
        raise ValueError("X must be a contiguous b x n tensor of the matrix dtype")
    if Y.shape != (X.shape[0], A.m) or not Y.is_contiguous() or Y.dtype != A.dtype:
        raise ValueError("Y must be a contiguous b x m tensor of the matrix dtype")
    check(lib.hss_apply_noalloc(ctypes.byref(A.struct), X.shape[0], _ptr(X), _ptr(Y), _stream(dev)),
          "hss_apply_noalloc")
    return Y


def _group_structs(As):
    arr = (ctypes.POINTER(HssMatrixStruct) * len(As))(*[ctypes.pointer(A.struct) for A in As])
    return arr


def hss_apply_group_workspace_size(As, b: int) -> int:
    out = ctypes.c_size_t(0)
    check(lib.hss_apply_group_workspace_size(_group_structs(As), len(As), int(b), ctypes.byref(out)),
          "hss_apply_group_workspace_size")
    return int(out.value)


def hss_apply_group(As, X: torch.Tensor, Ys=None, ws: Optional[torch.Tensor] = None):
    """Y_g = X (S_g + U_g V_g^T)^T for every matrix of As (same n, dtype and
    format), in one launch per decode pass; returns the list of Y_g."""
    dev = _dev(X)
    As = list(As)
    for A in As:
        if X.dim() != 2 or X.shape[1] != A.n or not X.is_contiguous() or X.dtype != A.dtype:
            raise ValueError("X must be a contiguous b x n tensor of every matrix's dtype")
    b = X.shape[0]
    if Ys is None:
        Ys = [torch.empty((b, A.m), dtype=A.dtype, device=dev) for A in As]
    if ws is None:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("create the workspace before graph capture and pass it as ws=")
        ws = apply_workspace(hss_apply_group_workspace_size(As, b), dev)
    yp = (ctypes.c_void_p * len(As))(*[_ptr(Y) for Y in Ys])
    check(lib.hss_apply_group(_group_structs(As), len(As), b, _ptr(X), yp, _ptr(ws), ws.numel(),
                              _stream(dev)), "hss_apply_group")
    return Ys


def hss_csr_cols_to_u16(col_idx: torch.Tensor, n: int) -> torch.Tensor:
    """16-bit copy of int32 CSR columns (n <= 65536), as a torch.int16 tensor
    holding the uint16 bit patterns."""
    dev = _dev(col_idx)
    if col_idx.dtype != torch.int32 or not col_idx.is_contiguous():
        raise ValueError("col_idx must be a contiguous int32 tensor")
    out = torch.empty(col_idx.numel(), dtype=torch.int16, device=dev)
    check(lib.hss_csr_cols_to_u16(_ptr(col_idx), col_idx.numel(), int(n), _ptr(out), _stream(dev)),
          "hss_csr_cols_to_u16")
    return out


# ---------------------------------------------------------------------------
# Hierarchical variant
# ---------------------------------------------------------------------------

def hss_rcm_order(row_ptr, col_idx, n: int):
    """Reverse Cuthill-McKee order of a square CSR pattern (host arrays, or
    tensors copied to the host): numpy int32 perm, perm[i] = original index
    at position i."""
    import numpy as np
    rp = np.ascontiguousarray(row_ptr.cpu().numpy() if isinstance(row_ptr, torch.Tensor) else row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx.cpu().numpy() if isinstance(col_idx, torch.Tensor) else col_idx, dtype=np.int32)
    perm = np.zeros(int(n), dtype=np.int32)
    check(lib.hss_rcm_order(int(n), rp.ctypes.data, ci.ctypes.data if ci.size else None, perm.ctypes.data),
          "hss_rcm_order")
    return perm


def hss_concentration(W: torch.Tensor, perm: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device float64 tensor [rho, diagonal-block |W| sum, total |W| sum] of W
    (rows and columns in the order perm, a device int32 permutation)."""
    dev = _dev(W)
    if W.dim() != 2 or not W.is_contiguous() or W.dtype not in _DT:
        raise ValueError("W must be a contiguous 2-D fp32 or bf16 tensor")
    m, n = W.shape
    size = ctypes.c_size_t(0)
    check(lib.hss_concentration_workspace_size(m, n, ctypes.byref(size)), "hss_concentration_workspace_size")
    ws = torch.empty(size.value, dtype=torch.uint8, device=dev)
    out = torch.empty(3, dtype=torch.float64, device=dev)
    if perm is not None and (perm.dtype != torch.int32 or perm.numel() != n or not perm.is_contiguous()):
        raise ValueError("perm must be a contiguous int32 tensor of n entries")
    check(lib.hss_concentration(_DT[W.dtype], m, n, _ptr(W), _ptr(perm), _ptr(out), _ptr(ws), ws.numel(),
                                _stream(dev)), "hss_concentration")
    return out


def hss_hier_pack(U, Vt, m: int, n: int, perm: Optional[torch.Tensor] = None):
    """Flat factors (U_cat m x R, Vt_cat R x n) of the 2 x 2 block low-rank
    term with blocks U[b] Vt[b], b in the order 00, 01, 10, 11, on the matrix
    permuted by perm (device int32 or None)."""
    dtype = next(u.dtype for u in U if u is not None)
    dev = next(u.device for u in U if u is not None)
    r = [0 if u is None else int(u.shape[1]) for u in U]
    R = sum(r)
    Ucat = torch.empty((m, R), dtype=dtype, device=dev)
    Vtcat = torch.empty((R, n), dtype=dtype, device=dev)
    rows, cols = (m // 2, m - m // 2), (n // 2, n - n // 2)
    for b, (u, v) in enumerate(zip(U, Vt)):
        if u is None:
            continue
        if not u.is_contiguous() or not v.is_contiguous() or u.dtype != dtype or v.dtype != dtype:
            raise ValueError("blocks must be contiguous tensors of one dtype")
        if tuple(u.shape) != (rows[b >> 1], r[b]) or tuple(v.shape) != (r[b], cols[b & 1]):
            raise ValueError(f"block {b}: U {tuple(u.shape)} / Vt {tuple(v.shape)} do not fit a {m} x {n} matrix")
    r_arr = (ctypes.c_int32 * 4)(*r)
    u_arr = (ctypes.c_void_p * 4)(*[_ptr(u) for u in U])
    v_arr = (ctypes.c_void_p * 4)(*[_ptr(v) for v in Vt])
    check(lib.hss_hier_pack(_DT[dtype], int(m), int(n), r_arr, u_arr, v_arr, _ptr(perm), _ptr(Ucat), _ptr(Vtcat),
                            _stream(dev)), "hss_hier_pack")
    return Ucat, Vtcat


def hss_hier_pack_compact(U, Vt, m: int, n: int):
    """Compact factors (U_c m x ru, Vt_c R x (n - n // 2)) of an HSS_HIER2
    matrix from its blocks U[b] Vt[b], b in the order 00, 01, 10, 11 (None
    for a rank-0 block), in the blocks' own order; with hier_r = the block
    ranks they make HSSMatrix(..., hier_r=...)."""
    dtype = next(u.dtype for u in U if u is not None)
    dev = next(u.device for u in U if u is not None)
    r = [0 if u is None else int(u.shape[1]) for u in U]
    R, ru = sum(r), r[0] + r[1]
    rows, cols = (m // 2, m - m // 2), (n // 2, n - n // 2)
    for b, (u, v) in enumerate(zip(U, Vt)):
        if u is None:
            continue
        if not u.is_contiguous() or not v.is_contiguous() or u.dtype != dtype or v.dtype != dtype:
            raise ValueError("blocks must be contiguous tensors of one dtype")
        if tuple(u.shape) != (rows[b >> 1], r[b]) or tuple(v.shape) != (r[b], cols[b & 1]):
            raise ValueError(f"block {b}: U {tuple(u.shape)} / Vt {tuple(v.shape)} do not fit a {m} x {n} matrix")
    Uc = torch.empty((m, ru), dtype=dtype, device=dev)
    Vtc = torch.empty((R, n - n // 2), dtype=dtype, device=dev)
    r_arr = (ctypes.c_int32 * 4)(*r)
    u_arr = (ctypes.c_void_p * 4)(*[_ptr(u) for u in U])
    v_arr = (ctypes.c_void_p * 4)(*[_ptr(v) for v in Vt])
    check(lib.hss_hier_pack_compact(_DT[dtype], int(m), int(n), r_arr, u_arr, v_arr, _ptr(Uc), _ptr(Vtc),
                                    _stream(dev)), "hss_hier_pack_compact")
    return Uc, Vtc


def hss_csr_permute(row_ptr, col_idx, perm, n: int):
    """S' = P S P^T (S'[i][j] = S[perm[i]][perm[j]]) of a square CSR pattern,
    on the host: (row_ptr_p, col_idx_p, from), entry q of S' being entry
    from[q] of S (hss_gather_values moves the values)."""
    import numpy as np
    rp = np.ascontiguousarray(row_ptr.cpu().numpy() if isinstance(row_ptr, torch.Tensor) else row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx.cpu().numpy() if isinstance(col_idx, torch.Tensor) else col_idx, dtype=np.int32)
    pm = np.ascontiguousarray(perm.cpu().numpy() if isinstance(perm, torch.Tensor) else perm, dtype=np.int32)
    nnz = int(rp[n])
    rpp = np.zeros(int(n) + 1, dtype=np.int32)
    cip = np.zeros(max(nnz, 1), dtype=np.int32)
    frm = np.zeros(max(nnz, 1), dtype=np.int32)
    check(lib.hss_csr_permute(int(n), rp.ctypes.data, ci.ctypes.data if nnz else None, pm.ctypes.data,
                              rpp.ctypes.data, cip.ctypes.data, frm.ctypes.data), "hss_csr_permute")
    return rpp, cip[:nnz], frm[:nnz]



# ---------------------------------------------------------------------------
# Backward pass
# ---------------------------------------------------------------------------

def hss_grad(A: HSSMatrix, X: torch.Tensor, G: torch.Tensor, dS=True, dU=True, dVt=True,
             ws: Optional[torch.Tensor] = None) -> dict:
    """Parameter gradients of a bf16 layer (CSR or 2:4) for the upstream
    gradient G (b x m): fp32 dS (S's stored values, storage order: nnz for
    CSR, m x n/2 laid out as nm_values for 2:4), dU (m x r) and dVt (r x n,
    the gradient of the stored V^T).  Pass False to skip one."""
    dev = _dev(X)
    if X.dim() != 2 or X.shape[1] != A.n or not X.is_contiguous() or X.dtype != A.dtype:
        raise ValueError("X must be a contiguous b x n tensor of the matrix dtype")
    b = X.shape[0]
    if G.shape != (b, A.m) or not G.is_contiguous() or G.dtype != A.dtype:
        raise ValueError("G must be a contiguous b x m tensor of the matrix dtype")
    out = {}
    if dS:
        stored = A.m * (A.n // 2) if A.fmt == HSS_FMT_2OF4 else A.nnz
        out["dS"] = torch.empty(stored, dtype=torch.float32, device=dev)
    if dU:
        out["dU"] = torch.empty((A.m, A.r), dtype=torch.float32, device=dev)
    if dVt:
        out["dVt"] = torch.empty((A.r, A.n), dtype=torch.float32, device=dev)
    if ws is None:
        size = ctypes.c_size_t(0)
        check(lib.hss_grad_workspace_size(ctypes.byref(A.struct), b, ctypes.byref(size)), "hss_grad_workspace_size")
        ws = torch.empty(size.value, dtype=torch.uint8, device=dev)
    check(lib.hss_grad(ctypes.byref(A.struct), b, _ptr(X), _ptr(G), _ptr(out.get("dS")), _ptr(out.get("dU")),
                       _ptr(out.get("dVt")), _ptr(ws), ws.numel(), _stream(dev)), "hss_grad")
    return out


def hss_csr_transpose(row_ptr, col_idx, m: int, n: int):
    """S^T's CSR pattern (host int32 row_ptr_t, col_idx_t) and perm (entry q of
    S^T is entry perm[q] of S), computed on the host."""
    import numpy as np
    rp = np.ascontiguousarray(row_ptr.cpu().numpy() if isinstance(row_ptr, torch.Tensor) else row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx.cpu().numpy() if isinstance(col_idx, torch.Tensor) else col_idx, dtype=np.int32)
    nnz = int(rp[m])
    rpt = np.zeros(int(n) + 1, dtype=np.int32)
    cit = np.zeros(max(nnz, 1), dtype=np.int32)
    perm = np.zeros(max(nnz, 1), dtype=np.int32)
    check(lib.hss_csr_transpose(int(m), int(n), rp.ctypes.data, ci.ctypes.data if nnz else None, rpt.ctypes.data,
                                cit.ctypes.data, perm.ctypes.data), "hss_csr_transpose")
    return rpt, cit[:nnz], perm[:nnz]


def hss_gather_values(values: torch.Tensor, perm: torch.Tensor) -> torch.Tensor:
    """values[perm] on the device (bits copied)."""
    out = torch.empty(perm.numel(), dtype=values.dtype, device=values.device)
    check(lib.hss_gather_values(_DT[values.dtype], perm.numel(), _ptr(values), _ptr(perm), _ptr(out),
                                _stream(values.device)), "hss_gather_values")
    return out


def hss_transpose(t: torch.Tensor) -> torch.Tensor:
    """A contiguous 2-D fp32 / bf16 device tensor transposed by the library."""
    rows, cols = t.shape
    out = torch.empty((cols, rows), dtype=t.dtype, device=t.device)
    check(lib.hss_transpose(_DT[t.dtype], rows, cols, _ptr(t), _ptr(out), _stream(t.device)), "hss_transpose")
    return out


def hss_nm24_to_csr(A: HSSMatrix):
    """The stored positions of a 2:4 matrix as a device CSR pattern (row_ptr,
    col_idx) in storage order: its values array is nm_values flattened."""
    dev = A.nm_meta.device
    rp = torch.empty(A.m + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(A.m * (A.n // 2), dtype=torch.int32, device=dev)
    check(lib.hss_nm24_to_csr(A.m, A.n, _ptr(A.nm_meta), _ptr(rp), _ptr(ci), _stream(dev)), "hss_nm24_to_csr")
    return rp, ci


def hss_transposed_layer(A: HSSMatrix) -> HSSMatrix:
    """A^T = S^T + V U^T as an HSSMatrix (n x m, CSR): S^T's pattern from the
    host transpose (of the 2:4 positions for a 2:4 layer), its values
    gathered on the device, U' = V and V'^T = U^T from the stored factors.
    hss_apply(A^T, G) is the input gradient G A."""
    if A.flags & (HSS_DQ4 | HSS_HIER2):
        raise ValueError("the transposed layer is built for CSR and 2:4 layers with flat factors")
    if A.fmt == HSS_FMT_2OF4:
        dev = A.nm_meta.device
        row_ptr, cols = hss_nm24_to_csr(A)
        values, nnz = A.nm_values.reshape(-1), A.m * (A.n // 2)
    else:
        dev = A.row_ptr.device
        row_ptr, values, nnz = A.row_ptr, A.values, A.nnz
        cols = A.col_idx.to(torch.int32) if A.flags & HSS_COL16 else A.col_idx
        if A.flags & HSS_COL16:
            cols = cols & 0xFFFF
    rpt, cit, perm = hss_csr_transpose(row_ptr, cols if nnz else torch.zeros(0, dtype=torch.int32), A.m, A.n)
    perm_d = torch.from_numpy(perm).to(dev)
    vals = hss_gather_values(values, perm_d) if nnz else None
    U2 = hss_transpose(A.Vt) if A.r > 0 else None
    Vt2 = hss_transpose(A.U) if A.r > 0 else None
    At = HSSMatrix("csr", A.n, A.m, A.dtype, U=U2, Vt=Vt2, row_ptr=torch.from_numpy(rpt).to(dev),
                   col_idx=torch.from_numpy(cit).to(dev) if nnz else None, values=vals, nnz=nnz)
    At.perm_from_s = perm_d
    return At


def hss_backward(A: HSSMatrix, X: torch.Tensor, G: torch.Tensor, At: Optional[HSSMatrix] = None) -> dict:
    """dX (b x n, the layer dtype) = G A through the transposed layer, and
    the fp32 parameter gradients dS, dU, dVt of hss_grad."""
    if At is None:
        At = hss_transposed_layer(A)
    out = hss_grad(A, X, G)
    out["dX"] = hss_apply(At, G)
    return out
