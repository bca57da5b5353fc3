"""Thin Python binding of libsvq (ctypes).

Argument marshalling only: every step of the decode-and-multiply runs in the
HIP library.  PyTorch supplies device memory and streams.  The C functions
keep their names (``svq_pack``, ``svq_linear``, ``svq_moe_linear``); the
``pack``/``linear``/``moe_linear`` helpers below only allocate the
caller-owned buffers with torch and pass pointers.

If ``libsvq.so`` is missing the import of this module raises: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

# torch is imported before libsvq.so is loaded so that both bind to one HIP
# runtime: torch ships its own libamdhip64 with the same SONAME, and a
# second copy loaded later would not share device allocations or streams.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsvq.so")

SVQ_OK = 0
SVQ_ERR_INVALID_ARG = -1
SVQ_ERR_UNSUPPORTED = -2
SVQ_ERR_BUFFER_TOO_SMALL = -3
SVQ_ERR_HIP = -4
SVQ_BF16 = 0
SVQ_F32 = 1

EXPORTED = ("svq_pack", "svq_linear", "svq_linear_batched", "svq_linear_noalloc",
            "svq_moe_linear", "svq_moe_linear_batched", "svq_encode", "svq_encode_weighted", "svq_esg_perm", "svq_abs_select",
            "svq_status_string")
SVQ_SCRATCH_BYTES = 64 << 20
SVQ_NO_EXACT_SPLIT = -(1 << 31)


class SvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


class MatrixDesc(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int32), ("k", ctypes.c_int32),
        ("bd", ctypes.c_int32), ("br", ctypes.c_int32),
        ("codes", ctypes.c_void_p), ("dir_codebook", ctypes.c_void_p),
        ("radius_table", ctypes.c_void_p), ("perm", ctypes.c_void_p),
    ]


class Handle(ctypes.Structure):
    _fields_ = [
        ("dev", ctypes.c_void_p),
        ("n", ctypes.c_int32), ("k", ctypes.c_int32),
        ("bd", ctypes.c_int32), ("br", ctypes.c_int32),
        ("n_tiles", ctypes.c_int32), ("units", ctypes.c_int32),
        ("off_dtab", ctypes.c_uint64), ("off_rtab", ctypes.c_uint64),
        ("off_btab", ctypes.c_uint64), ("off_xtab", ctypes.c_uint64),
        ("off_perm", ctypes.c_uint64),
        ("off_codes", ctypes.c_uint64), ("code_bytes", ctypes.c_uint64),
        ("padded_code_bytes", ctypes.c_uint64), ("bytes", ctypes.c_uint64),
        ("xscale_log2", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "or python -m bit_spherical_vector_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    lib.svq_status_string.restype = ctypes.c_char_p
    lib.svq_status_string.argtypes = [ctypes.c_int]
    lib.svq_pack.restype = ctypes.c_int
    lib.svq_pack.argtypes = [ctypes.POINTER(MatrixDesc), ctypes.c_void_p,
                             ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(Handle),
                             ctypes.c_void_p]
    lib.svq_linear.restype = ctypes.c_int
    lib.svq_linear.argtypes = [ctypes.POINTER(Handle), ctypes.c_void_p, ctypes.c_int64,
                               ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                               ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    lib.svq_linear_batched.restype = ctypes.c_int
    lib.svq_linear_batched.argtypes = [ctypes.POINTER(Handle), ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_void_p),
                                       ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
                                       ctypes.POINTER(ctypes.c_void_p),
                                       ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                                       ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                                       ctypes.c_void_p]
    lib.svq_linear_noalloc.restype = ctypes.c_int
    lib.svq_linear_noalloc.argtypes = [ctypes.POINTER(Handle), ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_void_p]
    lib.svq_moe_linear.restype = ctypes.c_int
    lib.svq_moe_linear.argtypes = [ctypes.POINTER(Handle), ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    lib.svq_moe_linear_batched.restype = ctypes.c_int
    lib.svq_moe_linear_batched.argtypes = [ctypes.POINTER(ctypes.POINTER(Handle)), ctypes.c_int32,
                                           ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                                           ctypes.POINTER(ctypes.c_int64), ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_void_p),
                                           ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                                           ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.c_void_p]
    lib.svq_encode.restype = ctypes.c_int
    lib.svq_encode.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                               ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                               ctypes.c_void_p]
    lib.svq_encode_weighted.restype = ctypes.c_int
    lib.svq_encode_weighted.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    lib.svq_esg_perm.restype = ctypes.c_int
    lib.svq_esg_perm.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    lib.svq_abs_select.restype = ctypes.c_int
    lib.svq_abs_select.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.svq_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != SVQ_OK:
        raise SvqError(status, what)


# ---------------------------------------------------------------------------
# C calls with their own names (pointers and sizes in, status out)
# ---------------------------------------------------------------------------

def svq_pack(desc: MatrixDesc, dst_dev: Optional[int], dst_bytes: int,
             handle: Optional[Handle], stream: int) -> tuple:
    nbytes = ctypes.c_size_t(dst_bytes)
    st = LIB.svq_pack(ctypes.byref(desc), dst_dev, ctypes.byref(nbytes),
                      ctypes.byref(handle) if handle is not None else None, stream)
    return st, nbytes.value


def svq_linear(handle: Handle, x_ptr: int, m: int, ldx: int, y_ptr: int, ldy: int, ydt: int,
               ws_ptr: Optional[int], ws_bytes: int, stream: int) -> tuple:
    nbytes = ctypes.c_size_t(ws_bytes)
    st = LIB.svq_linear(ctypes.byref(handle), x_ptr, m, ldx, y_ptr, ldy, ydt, ws_ptr,
                        ctypes.byref(nbytes), stream)
    return st, nbytes.value


def svq_linear_noalloc(handle: Handle, x_ptr: int, m: int, ldx: int, y_ptr: int, ldy: int,
                       ydt: int, stream: int) -> int:
    return LIB.svq_linear_noalloc(ctypes.byref(handle), x_ptr, m, ldx, y_ptr, ldy, ydt, stream)


def svq_linear_batched(handles, count: int, x_ptrs, ldx, m: int, y_ptrs, ldy, ydt: int,
                       ws_ptr: Optional[int], ws_bytes: int, stream: int) -> tuple:
    """handles: ctypes array of Handle; x_ptrs/y_ptrs: ctypes c_void_p arrays;
    ldx/ldy: ctypes c_int64 arrays (or None for a workspace query)."""
    nbytes = ctypes.c_size_t(ws_bytes)
    st = LIB.svq_linear_batched(handles, count, x_ptrs, ldx, m, y_ptrs, ldy, ydt, ws_ptr,
                                ctypes.byref(nbytes), stream)
    return st, nbytes.value


def svq_moe_linear(handles, num_experts: int, x_ptr: int, ldx: int, x_per_slot: int,
                   ids_ptr: int, m: int, topk: int, y_ptr: int, ldy: int, ydt: int,
                   ws_ptr: Optional[int], ws_bytes: int, stream: int) -> tuple:
    nbytes = ctypes.c_size_t(ws_bytes)
    st = LIB.svq_moe_linear(handles, num_experts, x_ptr, ldx, x_per_slot, ids_ptr, m, topk,
                            y_ptr, ldy, ydt, ws_ptr, ctypes.byref(nbytes), stream)
    return st, nbytes.value


def svq_moe_linear_batched(handle_sets, count: int, num_experts: int, x_ptrs, ldx, x_per_slot: int,
                           ids_ptr: int, m: int, topk: int, y_ptrs, ldy, ydt: int,
                           ws_ptr: Optional[int], ws_bytes: int, stream: int) -> tuple:
    """handle_sets: sequence of `count` Handle arrays (one per projection);
    x_ptrs / ldx / y_ptrs / ldy: sequences of length count, or None (the
    workspace query)."""
    # arrays are sized by what is given (count itself is passed as is, so
    # that the library's own checks of it can be exercised)
    sets = (ctypes.POINTER(Handle) * len(handle_sets))(
        *[ctypes.cast(h, ctypes.POINTER(Handle)) for h in handle_sets])
    xp = (ctypes.c_void_p * len(x_ptrs))(*x_ptrs) if x_ptrs is not None else None
    lx = (ctypes.c_int64 * len(ldx))(*ldx) if ldx is not None else None
    yp = (ctypes.c_void_p * len(y_ptrs))(*y_ptrs) if y_ptrs is not None else None
    ly = (ctypes.c_int64 * len(ldy))(*ldy) if ldy is not None else None
    nbytes = ctypes.c_size_t(ws_bytes)
    st = LIB.svq_moe_linear_batched(sets, count, num_experts, xp, lx, x_per_slot, ids_ptr, m, topk, yp,
                                    ly, ydt, ws_ptr, ctypes.byref(nbytes), stream)
    return st, nbytes.value


def svq_encode(w_ptr: Optional[int], ldw: int, n: int, k: int, bd: int, codebook: np.ndarray,
               radius: np.ndarray, perm: np.ndarray, codes_ptr: Optional[int],
               ws_ptr: Optional[int], ws_bytes: int, stream: int) -> tuple:
    """codebook / radius: host uint16 arrays (fp16 bit patterns); perm: host
    int32 array."""
    cb = np.ascontiguousarray(codebook, dtype=np.uint16)
    rad = np.ascontiguousarray(radius, dtype=np.uint16)
    pm = np.ascontiguousarray(perm, dtype=np.int32)
    nbytes = ctypes.c_size_t(ws_bytes)
    st = LIB.svq_encode(w_ptr, ldw, n, k, bd, cb.ctypes.data, rad.ctypes.data, pm.ctypes.data,
                        codes_ptr, ws_ptr, ctypes.byref(nbytes), stream)
    return st, nbytes.value


def svq_encode_weighted(w_ptr: Optional[int], ldw: int, n: int, k: int, bd: int, codebook: np.ndarray,
                        radius: np.ndarray, perm: np.ndarray, h_ptr: Optional[int],
                        codes_ptr: Optional[int], ws_ptr: Optional[int], ws_bytes: int,
                        stream: int) -> tuple:
    """As :func:`svq_encode`, the code chosen by activation-weighted fitting
    with the device float64 channel weights at ``h_ptr``."""
    cb = np.ascontiguousarray(codebook, dtype=np.uint16)
    rad = np.ascontiguousarray(radius, dtype=np.uint16)
    pm = np.ascontiguousarray(perm, dtype=np.int32)
    nbytes = ctypes.c_size_t(ws_bytes)
    st = LIB.svq_encode_weighted(w_ptr, ldw, n, k, bd, cb.ctypes.data, rad.ctypes.data, pm.ctypes.data,
                                 h_ptr, codes_ptr, ws_ptr, ctypes.byref(nbytes), stream)
    return st, nbytes.value


def svq_esg_perm(x_ptr: Optional[int], t: int, ldx: int, k: int, energy_ptr: Optional[int],
                 perm_ptr: Optional[int], ws_ptr: Optional[int], ws_bytes: int,
                 stream: int) -> tuple:
    nbytes = ctypes.c_size_t(ws_bytes)
    st = LIB.svq_esg_perm(x_ptr, t, ldx, k, energy_ptr, perm_ptr, ws_ptr, ctypes.byref(nbytes), stream)
    return st, nbytes.value


def svq_abs_select(w_ptr: Optional[int], ldw: int, n: int, k: int, h_ptr: Optional[int],
                   perm: np.ndarray, candidates, codes_ptr: Optional[int], ws_ptr: Optional[int],
                   ws_bytes: int, stream: int, weighted_fit: int = 0) -> tuple:
    """candidates: sequence of (bd, codebook bits, radius bits) host arrays.
    Returns (status, workspace bytes, chosen index, errors)."""
    nc = len(candidates)
    pm = np.ascontiguousarray(perm, dtype=np.int32)
    bds = np.array([int(c[0]) for c in candidates] or [0], dtype=np.int32)
    cbs = [np.ascontiguousarray(c[1], dtype=np.uint16) for c in candidates]
    rads = [np.ascontiguousarray(c[2], dtype=np.uint16) for c in candidates]
    cb_ptrs = (ctypes.c_void_p * max(nc, 1))(*[a.ctypes.data for a in cbs])
    rad_ptrs = (ctypes.c_void_p * max(nc, 1))(*[a.ctypes.data for a in rads])
    errs = np.zeros(max(nc, 1), dtype=np.float64)
    chosen = ctypes.c_int32(-1)
    nbytes = ctypes.c_size_t(ws_bytes)
    st = LIB.svq_abs_select(w_ptr, ldw, n, k, h_ptr, pm.ctypes.data, nc, bds.ctypes.data, cb_ptrs,
                            rad_ptrs, weighted_fit, codes_ptr, ctypes.byref(chosen), errs.ctypes.data,
                            ws_ptr, ctypes.byref(nbytes), stream)
    return st, nbytes.value, chosen.value, errs[:nc]


# ---------------------------------------------------------------------------
# torch-side helpers (allocation of caller-owned buffers only)
# ---------------------------------------------------------------------------

def _stream_handle(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def make_desc(n: int, k: int, bd: int, br: int, codes: np.ndarray, codebook: np.ndarray,
              radius: np.ndarray, perm: np.ndarray) -> tuple:
    """Build a MatrixDesc over host numpy arrays (kept alive in the result)."""
    keep = (np.ascontiguousarray(codes, dtype=np.uint8),
            np.ascontiguousarray(codebook, dtype=np.uint16),
            np.ascontiguousarray(radius, dtype=np.uint16),
            np.ascontiguousarray(perm, dtype=np.int32))
    desc = MatrixDesc(n, k, bd, br, keep[0].ctypes.data, keep[1].ctypes.data,
                      keep[2].ctypes.data, keep[3].ctypes.data)
    return desc, keep


class PackedMatrix:
    """A packed SVQ matrix: torch device buffer + svq_handle."""

    def __init__(self, buf, handle: Handle):
        self.buf = buf
        self.handle = handle

    @property
    def n(self) -> int:
        return self.handle.n

    @property
    def k(self) -> int:
        return self.handle.k

    @property
    def code_bytes(self) -> int:
        return int(self.handle.code_bytes)

    @property
    def padded_code_bytes(self) -> int:
        return int(self.handle.padded_code_bytes)


def pack(mat, device="cuda", stream=None) -> PackedMatrix:
    """Pack a canonical matrix (any object with n, k, bd, br, codes, codebook,
    radius, perm attributes, e.g. ``synth.MatrixInputs``)."""
    import torch
    desc, keep = make_desc(mat.n, mat.k, mat.bd, mat.br, mat.codes, mat.codebook, mat.radius,
                           mat.perm)
    st, nbytes = svq_pack(desc, None, 0, None, 0)
    _check(st, "svq_pack (size query)")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    h = Handle()
    st, _ = svq_pack(desc, buf.data_ptr(), nbytes, h, _stream_handle(stream))
    _check(st, "svq_pack")
    del keep
    return PackedMatrix(buf, h)


def linear_workspace_bytes(pm: PackedMatrix, m: int) -> int:
    st, nbytes = svq_linear(pm.handle, None, m, pm.k, None, pm.n, SVQ_BF16, None, 0, 0)
    _check(st, "svq_linear (workspace query)")
    return nbytes


def linear(pm: PackedMatrix, x, out=None, out_dtype=None, workspace=None, stream=None):
    """y = x @ What^T.  x: bf16 [m, >=k] CUDA tensor (row stride = x.stride(0))."""
    import torch
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    m = x.shape[0]
    if out is None:
        dt = out_dtype or torch.bfloat16
        out = torch.empty((m, pm.n), dtype=dt, device=x.device)
    ydt = SVQ_F32 if out.dtype == torch.float32 else SVQ_BF16
    if out.dtype not in (torch.float32, torch.bfloat16) or out.stride(1) != 1:
        raise ValueError("out must be bf16 or fp32 with unit column stride")
    need = linear_workspace_bytes(pm, m)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st, _ = svq_linear(pm.handle, x.data_ptr(), m, x.stride(0), out.data_ptr(), out.stride(0),
                       ydt, workspace.data_ptr(), workspace.numel(), _stream_handle(stream))
    _check(st, "svq_linear")
    return out


def linear_noalloc(pm: PackedMatrix, x, out, stream=None):
    """y = x @ What^T into a caller-given ``out`` through svq_linear_noalloc
    (no workspace: the library's own scratch is used)."""
    import torch
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    if out.dtype not in (torch.float32, torch.bfloat16) or out.stride(1) != 1:
        raise ValueError("out must be bf16 or fp32 with unit column stride")
    ydt = SVQ_F32 if out.dtype == torch.float32 else SVQ_BF16
    st = svq_linear_noalloc(pm.handle, x.data_ptr(), x.shape[0], x.stride(0), out.data_ptr(),
                            out.stride(0), ydt, _stream_handle(stream))
    _check(st, "svq_linear_noalloc")
    return out


class BatchedCall:
    """Pre-marshalled arguments of one svq_linear_batched call (device
    tensors are owned by the caller and must outlive the object)."""

    def __init__(self, pms: Sequence[PackedMatrix], xs, ys, workspace=None, stream=None):
        import torch
        n = len(pms)
        self.keep = (list(pms), list(xs), list(ys))
        self.handles = handle_array(pms)
        self.count = n
        self.m = xs[0].shape[0]
        self.x_ptrs = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
        self.y_ptrs = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
        self.ldx = (ctypes.c_int64 * n)(*[x.stride(0) for x in xs])
        self.ldy = (ctypes.c_int64 * n)(*[y.stride(0) for y in ys])
        self.ydt = SVQ_F32 if ys[0].dtype == torch.float32 else SVQ_BF16
        st, need = svq_linear_batched(self.handles, n, None, None, self.m, None, None, self.ydt,
                                      None, 0, 0)
        _check(st, "svq_linear_batched (workspace query)")
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xs[0].device)
        self.workspace = workspace
        self.stream = _stream_handle(stream)

    def __call__(self) -> None:
        st, _ = svq_linear_batched(self.handles, self.count, self.x_ptrs, self.ldx, self.m,
                                   self.y_ptrs, self.ldy, self.ydt, self.workspace.data_ptr(),
                                   self.workspace.numel(), self.stream)
        _check(st, "svq_linear_batched")


class MoeCall:
    """Pre-marshalled arguments of one svq_moe_linear call (device tensors and
    the packed experts are owned by the caller and must outlive the object)."""

    def __init__(self, pms: Sequence[PackedMatrix], x, expert_ids, topk: int, x_per_slot: bool,
                 y, workspace=None, stream=None):
        import torch
        self.keep = (list(pms), x, expert_ids, y)
        self.handles = handle_array(pms)
        self.n_exp = len(pms)
        self.topk = topk
        self.m = expert_ids.numel() // topk
        self.x_per_slot = int(x_per_slot)
        self.args_x = (x.data_ptr(), x.stride(0))
        self.ids = expert_ids.data_ptr()
        self.args_y = (y.data_ptr(), y.stride(0))
        self.ydt = SVQ_F32 if y.dtype == torch.float32 else SVQ_BF16
        need = moe_workspace_bytes(self.handles, self.n_exp, self.m, topk, self.x_per_slot)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
        self.workspace = workspace
        self.stream = _stream_handle(stream)

    def __call__(self) -> None:
        st, _ = svq_moe_linear(self.handles, self.n_exp, self.args_x[0], self.args_x[1],
                               self.x_per_slot, self.ids, self.m, self.topk, self.args_y[0],
                               self.args_y[1], self.ydt, self.workspace.data_ptr(),
                               self.workspace.numel(), self.stream)
        _check(st, "svq_moe_linear")


class MoeBatchedCall:
    """Pre-marshalled arguments of one svq_moe_linear_batched call: several
    projections (e.g. an FFN's gate and up) that share expert_ids, topk and
    x_per_slot.  pm_sets[c] are projection c's packed experts, xs[c] / ys[c]
    its device input and output (owned by the caller; they must outlive the
    object)."""

    def __init__(self, pm_sets, xs, expert_ids, topk: int, x_per_slot: bool, ys, workspace=None,
                 stream=None):
        import torch
        self.keep = ([list(p) for p in pm_sets], list(xs), expert_ids, list(ys))
        self.sets = [handle_array(p) for p in pm_sets]
        self.count = len(self.sets)
        self.n_exp = len(pm_sets[0])
        self.topk = topk
        self.m = expert_ids.numel() // topk
        self.x_per_slot = int(x_per_slot)
        self.x_ptrs = [x.data_ptr() for x in xs]
        self.ldx = [x.stride(0) for x in xs]
        self.ids = expert_ids.data_ptr()
        self.y_ptrs = [y.data_ptr() for y in ys]
        self.ldy = [y.stride(0) for y in ys]
        self.ydt = SVQ_F32 if ys[0].dtype == torch.float32 else SVQ_BF16
        st, need = svq_moe_linear_batched(self.sets, self.count, self.n_exp, None, None, self.x_per_slot,
                                          None, self.m, topk, None, None, self.ydt, None, 0, 0)
        _check(st, "svq_moe_linear_batched (workspace query)")
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xs[0].device)
        self.workspace = workspace
        self.stream = _stream_handle(stream)

    def __call__(self) -> None:
        st, _ = svq_moe_linear_batched(self.sets, self.count, self.n_exp, self.x_ptrs, self.ldx,
                                       self.x_per_slot, self.ids, self.m, self.topk, self.y_ptrs,
                                       self.ldy, self.ydt, self.workspace.data_ptr(),
                                       self.workspace.numel(), self.stream)
        _check(st, "svq_moe_linear_batched")


def moe_linear_batched(pm_sets, xs, expert_ids, topk: int, x_per_slot: bool, outs=None,
                       out_dtype=None, stream=None):
    """Several MoE projections sharing the routing in one call; returns the
    outputs (one [m*topk, n_c] tensor per projection)."""
    import torch
    if outs is None:
        outs = [torch.empty((expert_ids.numel(), p[0].n), dtype=out_dtype or torch.bfloat16,
                            device=x.device) for p, x in zip(pm_sets, xs)]
    MoeBatchedCall(pm_sets, xs, expert_ids, topk, x_per_slot, outs, stream=stream)()
    return outs


def linear_batched(pms: Sequence[PackedMatrix], xs, outs=None, out_dtype=None, stream=None):
    """svq_linear over several matrices sharing m in one call."""
    import torch
    if outs is None:
        outs = [torch.empty((x.shape[0], pm.n), dtype=out_dtype or torch.bfloat16,
                            device=x.device) for pm, x in zip(pms, xs)]
    BatchedCall(pms, xs, outs, stream=stream)()
    return outs


def handle_array(pms: Sequence[PackedMatrix]):
    arr = (Handle * len(pms))()
    for i, pm in enumerate(pms):
        arr[i] = pm.handle
    return arr


def moe_workspace_bytes(handles, num_experts: int, m: int, topk: int, x_per_slot: int) -> int:
    st, nbytes = svq_moe_linear(handles, num_experts, None, handles[0].k, x_per_slot, None, m,
                                topk, None, handles[0].n, SVQ_BF16, None, 0, 0)
    _check(st, "svq_moe_linear (workspace query)")
    return nbytes


def moe_linear(pms: Sequence[PackedMatrix], x, expert_ids, topk: int, x_per_slot: bool,
               out=None, out_dtype=None, workspace=None, handles=None, stream=None):
    """One MoE projection: y[q] = x[row(q)] @ What_{ids[q]}^T for every slot q."""
    import torch
    if handles is None:
        handles = handle_array(pms)
    n_exp = len(handles)
    s_total = expert_ids.numel()
    m = s_total // topk
    n = handles[0].n
    if out is None:
        out = torch.empty((s_total, n), dtype=out_dtype or torch.bfloat16, device=x.device)
    ydt = SVQ_F32 if out.dtype == torch.float32 else SVQ_BF16
    need = moe_workspace_bytes(handles, n_exp, m, topk, int(x_per_slot))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st, _ = svq_moe_linear(handles, n_exp, x.data_ptr(), x.stride(0), int(x_per_slot),
                           expert_ids.data_ptr(), m, topk, out.data_ptr(), out.stride(0), ydt,
                           workspace.data_ptr(), workspace.numel(), _stream_handle(stream))
    _check(st, "svq_moe_linear")
    return out


def esg_perm(x, stream=None):
    """ESG channel energies (device float64 [k]) and permutation (device
    int32 [k]) from device bf16 calibration activations [t, k]."""
    import torch
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bfloat16 tensor with unit column stride")
    t, k = x.shape
    st, need = svq_esg_perm(None, t, x.stride(0), k, None, None, None, 0, 0)
    _check(st, "svq_esg_perm (size query)")
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    energy = torch.empty(k, dtype=torch.float64, device=x.device)
    perm = torch.empty(k, dtype=torch.int32, device=x.device)
    st, _ = svq_esg_perm(x.data_ptr(), t, x.stride(0), k, energy.data_ptr(), perm.data_ptr(),
                         ws.data_ptr(), need, _stream_handle(stream))
    _check(st, "svq_esg_perm")
    return energy, perm


def abs_select(w, perm, h, candidates, stream=None, weighted_fit: bool = False):
    """ABS over ``candidates`` [(bd, codebook bits, radius bits)] for a device
    fp32 weight matrix [n, k] with host permutation ``perm`` and device
    float64 channel weights ``h`` [k]; ``weighted_fit`` codes every candidate
    by activation-weighted fitting with the same h.  Returns (chosen index,
    errors as a host float64 array, the chosen codes as a device uint8
    stream)."""
    import torch
    if w.dtype != torch.float32 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D float32 tensor with unit column stride")
    if h.dtype != torch.float64 or not h.is_contiguous():
        raise ValueError("h must be a contiguous float64 tensor")
    n, k = w.shape
    st, need, _, _ = svq_abs_select(None, w.stride(0), n, k, None, perm, candidates, None, None, 0, 0)
    _check(st, "svq_abs_select (size query)")
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=w.device)
    codes = torch.zeros((n * (k // 8) * 18 + 7) // 8, dtype=torch.uint8, device=w.device)
    st, _, chosen, errs = svq_abs_select(w.data_ptr(), w.stride(0), n, k, h.data_ptr(), perm,
                                         candidates, codes.data_ptr(), ws.data_ptr(), need,
                                         _stream_handle(stream), int(bool(weighted_fit)))
    _check(st, "svq_abs_select")
    return chosen, errs, codes


def encode_weighted(w, perm, h, bd: int, codebook, radius, stream=None):
    """As :func:`encode`, each code chosen by activation-weighted fitting with
    the device float64 channel weights ``h`` [k]."""
    import torch
    if w.dtype != torch.float32 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D float32 tensor with unit column stride")
    if h.dtype != torch.float64 or not h.is_contiguous() or h.numel() != w.shape[1]:
        raise ValueError("h must be a contiguous float64 tensor of k entries")
    n, k = w.shape
    st, need = svq_encode_weighted(None, w.stride(0), n, k, bd, codebook, radius, perm, None, None,
                                   None, 0, 0)
    _check(st, "svq_encode_weighted (size query)")
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=w.device)
    codes = torch.zeros((n * (k // 8) * 18 + 7) // 8, dtype=torch.uint8, device=w.device)
    st, _ = svq_encode_weighted(w.data_ptr(), w.stride(0), n, k, bd, codebook, radius, perm,
                                h.data_ptr(), codes.data_ptr(), ws.data_ptr(), need,
                                _stream_handle(stream))
    _check(st, "svq_encode_weighted")
    return codes


def encode(w, perm, bd: int, codebook, radius, stream=None):
    """Codes of a device fp32 weight matrix [n, k] (rows may be strided) as
    the canonical stream, a device uint8 tensor of ceil(n*k*9/32) bytes."""
    import torch
    if w.dtype != torch.float32 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D float32 tensor with unit column stride")
    n, k = w.shape
    st, need = svq_encode(None, w.stride(0), n, k, bd, codebook, radius, perm, None, None, 0, 0)
    _check(st, "svq_encode (size query)")
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=w.device)
    codes = torch.zeros((n * (k // 8) * 18 + 7) // 8, dtype=torch.uint8, device=w.device)
    st, _ = svq_encode(w.data_ptr(), w.stride(0), n, k, bd, codebook, radius, perm,
                       codes.data_ptr(), ws.data_ptr(), need, _stream_handle(stream))
    _check(st, "svq_encode")
    return codes
